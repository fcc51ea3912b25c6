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
// even, magnitudes of 448 and above saturating to 448.  The quotient and its
// rounding are computed exactly as defined (IEEE fp32 division; the
// conversion below is integer arithmetic on the fp32 bits), so the codes are
// a function of the input bits alone.
//
// One workgroup per row: a pass for the amax (wave max, then across the four
// waves through LDS), then a pass writing eight codes per thread step.
#include "common.h"
#include "internal.h"

namespace tpmlp {

namespace {

constexpr int kQuantThreads = 256;

// fp32 -> e4m3fn code, round to nearest even, saturating (|v| >= 448 -> 448).
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x43E00000u) {                 // |v| >= 448
    code = 0x7Eu;
  } else if (a >= 0x3C800000u) {          // |v| >= 2^-6: normal codes, 3 mantissa bits
    const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;   // ties to even; a carry bumps the exponent
    code = r - (120u << 3);                                        // exponent bias 127 -> 7
  } else {                                // subnormal codes: multiples of 2^-9 (8 steps = 2^-6)
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  }
  return sign | code;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__global__ __launch_bounds__(kQuantThreads) void quant_rows_kernel(int K, const uint16_t* __restrict__ x,
                                                                    int64_t ldx, uint8_t* __restrict__ q,
                                                                    int64_t ldq, float* __restrict__ scales) {
  __shared__ float part[kQuantThreads / 64];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + (int64_t)row * ldx);
  const int nchunk = K / 8;
  float amax = 0.f;
  for (int c = tid; c < nchunk; c += kQuantThreads) {
    const u32x4 v = src[c];
#pragma unroll
    for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[i])), fabsf(bf16_hi(v[i]))));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((tid & 63) == 0) part[tid >> 6] = amax;
  __syncthreads();
  amax = part[0];
#pragma unroll
  for (int w = 1; w < kQuantThreads / 64; ++w) amax = fmaxf(amax, part[w]);
  const float s = amax == 0.f ? 1.f : amax / 448.0f;
  if (tid == 0) scales[row] = s;
  u32x2* dst = reinterpret_cast<u32x2*>(q + (int64_t)row * ldq);
  for (int c = tid; c < nchunk; c += kQuantThreads) {
    const u32x4 v = src[c];
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      b[2 * i] = e4m3_rne(bf16_lo(v[i]) / s);
      b[2 * i + 1] = e4m3_rne(bf16_hi(v[i]) / s);
    }
    dst[c] = u32x2{b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24), b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24)};
  }
}

}  // namespace

hipError_t launch_quant_rows(int M, int K, const void* x, int64_t ldx, void* q, int64_t ldq, float* scales,
                             hipStream_t stream) {
  return launch(K_QUANT_ROWS, quant_rows_kernel, dim3((unsigned)M), dim3(kQuantThreads), 0, stream, K,
                (const uint16_t*)x, ldx, (uint8_t*)q, ldq, scales);
}

}  // namespace tpmlp
