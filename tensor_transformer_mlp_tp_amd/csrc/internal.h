// Internal interface between the C ABI layer (abi.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

constexpr int kMaxPartials = 64;

struct PartialPtrs {
  const float* p[kMaxPartials];
};

// The activation rows X (M x h): nb row blocks of `rows` rows each, block b
// holding rows b*rows .. b*rows+rows-1 with leading dimension ld (elements).
// A contiguous X is one block of M rows; the sequence-parallel form passes
// the t ranks' row blocks as they are (the gathered X is never built).
struct XRows {
  const void* p[kMaxPartials];
  int nb;
  int rows;
  int64_t ld;
};

// Row `row` of X.  The block is chosen with wave-uniform indices only, so
// the pointer table stays in the kernel-argument segment.
template <typename T>
__device__ __forceinline__ const T* x_row(const XRows& xr, int row) {
  const int b = row / xr.rows;
  const void* base = xr.p[0];
  for (int i = 1; i < xr.nb; ++i)
    if (i == b) base = xr.p[i];
  return reinterpret_cast<const T*>(base) + (int64_t)(row - b * xr.rows) * xr.ld;
}

// One rank's forward, already validated.  Pointers are device addresses.
struct ShardArgs {
  int M, h, I_s;
  XRows x;                  // M x h, bf16 or fp32
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
