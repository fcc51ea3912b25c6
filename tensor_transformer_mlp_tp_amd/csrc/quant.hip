// Per-row dynamic quantisation of bf16 activations to OCP e4m3fn codes, for
// the fp8 x fp8 (W8A8) forward.  The pages name fp8 only as a one-byte
// storage mode for weights ("Build a model sharding system for serving 70B+
// parameter models", scalablesystem.dev, the shard planner's bytes per
// parameter); quantising the activations as well lets both GEMM operands use
// gfx950's fp8 matrix instructions, at twice the bf16 rate, with changed
// numerics.
//
// Row m (a token): s_m = amax_m / 448 in fp32 (1 for an all-zero row) and
// q = e4m3fn(x / s_m), the fp32 quotient rounded to the nearest code, ties to
// even (the quotients stay below 448 (1 + 2^-23), so 448 is the largest
// code).  Both roundings are exactly those of the definition, so the codes
// are a function of the input bits alone (rows must be finite):
//  - the quotient: fp32(x * r) computed in fp64, with r = 1 / s_m rounded
//    to fp64 once per row, is the correctly rounded fp32 x / s_m.  The fp64
//    product is within 2^-52 (relative) of x / s_m, while x / s_m, for x a
//    bf16 value (at most 8 significant bits) and s_m an fp32 value, is never
//    an fp32 rounding midpoint and is at least 2^-50 (relative) away from
//    every midpoint m near it: m is an odd multiple of half an ulp (25
//    significant bits), so the odd part of s_m m has at least 25 bits and
//    that of x at most 8, and x - s_m m is a nonzero multiple of a power of
//    two that is at least min(x 2^-8, s_m m 2^-49).  Both values thus round
//    to the same fp32 number.  (Quotients below 2^-126, where the fp32
//    spacing is absolute, give the zero code either way.)
//  - the code is the fp32 -> e4m3fn conversion instruction
//    (v_cvt_pk_fp8_f32, round to nearest even), which was compared with the
//    definition's rounding on every fp32 input of magnitude up to 464
//    without a difference.
// Per element that is three fp64 instructions and half a conversion, against
// about thirty for an IEEE fp32 division plus the rounding in integer
// arithmetic, which made the kernel ALU-bound.
//
// One workgroup per row.  Each thread loads all of its 16-byte chunks of
// the row at once (KC per thread, so the whole row is in flight), takes the
// amax (wave max, then across the four waves through LDS), and writes eight
// codes per chunk from the same registers: the row is read once.  Rows
// longer than 256 * 8 * kQuantMaxKC elements take a two-pass loop instead.
#include "common.h"
#include "internal.h"

namespace tpmlp {

namespace {

constexpr int kQuantThreads = 256;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float amax8(float amax, u32x4 v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[i])), fabsf(bf16_hi(v[i]))));
  return amax;
}

// Codes of the eight bf16 values in v (little-endian byte order); rd: the
// row's 1 / s in fp64 (see the header).
__device__ __forceinline__ u32x2 codes8(u32x4 v, double rd) {
  float q[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    q[2 * i] = (float)((double)bf16_lo(v[i]) * rd);
    q[2 * i + 1] = (float)((double)bf16_hi(v[i]) * rd);
  }
  uint32_t w[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    w[j] = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * j], q[4 * j + 1], 0, false);
    w[j] = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * j + 2], q[4 * j + 3], w[j], true);
  }
  return u32x2{w[0], w[1]};
}


// The row's amax across the workgroup, and its scale (1 for an all-zero row).
__device__ __forceinline__ float row_scale(float amax, float* part, int tid) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((tid & 63) == 0) part[tid >> 6] = amax;
  __syncthreads();
  amax = part[0];
#pragma unroll
  for (int w = 1; w < kQuantThreads / 64; ++w) amax = fmaxf(amax, part[w]);
  return amax == 0.f ? 1.f : amax / 448.0f;
}

// KC > 0: chunks c = tid + i * kQuantThreads (i < KC) held in registers; KC
// == 0: any row length, two passes.
template <int KC>
__global__ __launch_bounds__(kQuantThreads) void quant_rows_kernel(int K, const uint16_t* __restrict__ x,
                                                                    int64_t ldx, uint8_t* __restrict__ q,
                                                                    int64_t ldq, float* __restrict__ scales) {
  __shared__ float part[kQuantThreads / 64];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + (int64_t)row * ldx);
  u32x2* dst = reinterpret_cast<u32x2*>(q + (int64_t)row * ldq);
  const int nchunk = K / 8;
  float amax = 0.f;
  if constexpr (KC > 0) {
    u32x4 v[KC];
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int c = tid + i * kQuantThreads;
      v[i] = c < nchunk ? __builtin_nontemporal_load(src + c) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < KC; ++i) amax = amax8(amax, v[i]);
    const float s = row_scale(amax, part, tid);
    if (tid == 0) scales[row] = s;
    const double rd = 1.0 / (double)s;
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int c = tid + i * kQuantThreads;
      if (c < nchunk) dst[c] = codes8(v[i], rd);
    }
  } else {
    for (int c = tid; c < nchunk; c += kQuantThreads) amax = amax8(amax, src[c]);
    const float s = row_scale(amax, part, tid);
    if (tid == 0) scales[row] = s;
    const double rd = 1.0 / (double)s;
    for (int c = tid; c < nchunk; c += kQuantThreads) dst[c] = codes8(src[c], rd);
  }
}

constexpr int kQuantMaxKC = 8;

}  // namespace

hipError_t launch_quant_rows(int M, int K, const void* x, int64_t ldx, void* q, int64_t ldq, float* scales,
                             hipStream_t stream) {
  const int per_thread = (K / 8 + kQuantThreads - 1) / kQuantThreads;
  auto go = [&](auto kern) {
    return launch(K_QUANT_ROWS, kern, dim3((unsigned)M), dim3(kQuantThreads), 0, stream, K, (const uint16_t*)x, ldx,
                  (uint8_t*)q, ldq, scales);
  };
  if (per_thread <= 1) return go(quant_rows_kernel<1>);
  if (per_thread <= 2) return go(quant_rows_kernel<2>);
  if (per_thread <= 4) return go(quant_rows_kernel<4>);
  if (per_thread <= kQuantMaxKC) return go(quant_rows_kernel<kQuantMaxKC>);
  return go(quant_rows_kernel<0>);
}

}  // namespace tpmlp
