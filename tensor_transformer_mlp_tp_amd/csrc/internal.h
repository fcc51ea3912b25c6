// Internal interface between the C ABI layer (abi.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

constexpr int kMaxPartials = 64;

struct PartialPtrs {
  const float* p[kMaxPartials];
};

// One rank's forward, already validated.  Pointers are device addresses.
struct ShardArgs {
  int M, h, I_s;
  const void* x;            // M x h, bf16 or fp32
  int64_t ldx;
  const void* wg;           // I_s x h
  const void* wu;           // I_s x h
  int64_t ldw_gu;
  const void* wd;           // h x I_s
  int64_t ldw_down;
  const float* sg;          // fp8 only: I_s
  const float* su;          // fp8 only: I_s
  const float* sd;          // fp8 only: h
  float* p;                 // M x h fp32
  int64_t ldp;
  void* a;                  // workspace: M x I_s intermediate
  int64_t lda;
  bool fp8;                 // weights are e4m3fn codes
};

// Largest M served by the weight-streaming (decode) kernels.
constexpr int kDecodeMaxM = 64;

hipError_t launch_partial_reduce(const PartialPtrs& ptrs, int t, float* out, int64_t n,
                                 hipStream_t stream);
hipError_t launch_forward_decode(const ShardArgs& a, hipStream_t stream);
hipError_t launch_forward_prefill(const ShardArgs& a, hipStream_t stream);
hipError_t launch_forward_f32(const ShardArgs& a, hipStream_t stream);

}  // namespace tpmlp
