// Shared device helpers and the launch wrapper for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "internal.h"

namespace tpmlp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));


// Implemented in abi.cpp: returns the start/stop events to attach to the next
// launch of `kind` when timing is on, or null events.
void profile_events_for_launch(int kind, hipEvent_t* start, hipEvent_t* stop);

// Every kernel of the library is launched through here so that, when timing
// is on, the dispatch itself carries the start and stop timestamps (no extra
// marker packets in the stream).
template <typename... Params, typename... Args>
inline hipError_t launch(int kind, void (*kernel)(Params...), dim3 grid, dim3 block,
                         uint32_t lds_bytes, hipStream_t stream, Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  profile_events_for_launch(kind, &e0, &e1);
  hipExtLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, e0, e1, 0,
                        static_cast<Params>(args)...);
  return hipGetLastError();
}

// Workgroup barrier ordering LDS accesses only.  __syncthreads() would also
// wait for every outstanding global load (vmcnt(0)), which would drain a
// direct-load ring at each step; the ring's completion is tracked with
// explicit vmcnt waits instead.
// Before it, this wave's LDS reads are complete (lgkmcnt(0)); the acquire
// fence after it keeps later LDS reads below the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((15 << 0) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------- numerics

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// SiLU(z) = z / (1 + e^-z).  For z below about -88 the exponential is +inf and
// the quotient is -0, the limit of the function.
__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Eight OCP e4m3fn codes (two dwords) -> eight bf16 (exact: every e4m3 value
// is a bf16 value).  Hardware conversion, unit scale.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Eight int8 codes (two dwords) -> eight bf16, exact: an int8 value has at
// most 8 significant bits.  Each byte is biased to unsigned (xor 0x80),
// converted to fp32 (exact), unbiased by an exact fp32 subtraction, and the
// bf16 is the upper half of the fp32 word (exact, the low half is zero).
__device__ __forceinline__ uint32_t i8pair_to_bf16x2(uint32_t u, int sh) {
  const float f0 = (float)((u >> sh) & 0xffu) - 128.0f;
  const float f1 = (float)((u >> (sh + 8)) & 0xffu) - 128.0f;
  return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
}

__device__ __forceinline__ bf16x8 i8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  const uint32_t a = lo ^ 0x80808080u, b = hi ^ 0x80808080u;
  const u32x4 r = {i8pair_to_bf16x2(a, 0), i8pair_to_bf16x2(a, 16), i8pair_to_bf16x2(b, 0),
                   i8pair_to_bf16x2(b, 16)};
  return as_bf16x8(r);
}

// Eight one-byte weight codes of format WB (kWeightE4M3 or kWeightI8) -> bf16.
template <int WB>
__device__ __forceinline__ bf16x8 byte8_to_bf16x8(uint32_t lo, uint32_t hi) {
  if constexpr (WB == kWeightI8)
    return i8x8_to_bf16x8(lo, hi);
  else
    return fp8x8_to_bf16x8(lo, hi);
}

// Four consecutive outputs at element index idx of `out`: fp32, or bf16
// rounded to nearest even (OBF).
template <bool OBF>
__device__ __forceinline__ void store_out4(void* out, int64_t idx, f32x4 v) {
  if constexpr (OBF) {
    const u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + idx) = pk;
  } else {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + idx) = v;
  }
}

// 16x16x32 bf16 MFMA: D(16x16) += A(16x32) * B(32x16).  Lane l supplies row
// (l % 16) of A and column (l % 16) of B, each with the eight k values of
// group (l / 16); it receives D rows 4*(l/16) .. 4*(l/16)+3 of column l % 16.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace tpmlp
