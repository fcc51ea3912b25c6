// Row-streaming kernel for narrow projections at one or two tokens, bf16
// weights: a rank's QKV projection (1280 rows of W over h = 8192 at 70B,
// TP = 8).
//
// The matrix-core streams (decode.hip) read 16 rows of W side by side and,
// with so few row blocks for the chip, split K over extra workgroups whose
// sums meet in memory.  At M <= 2 a row is 2*M FLOP per weight, so the dot
// products fit on the VALU (v_dot2_f32_bf16: two bf16 products and their sum
// into fp32 per instruction) and each wave can stream whole rows of W one
// after the other, one kilobyte per load instruction (lane l holds eight
// consecutive k of a 512-k chunk): with 1280 rows that is enough waves for
// the chip without a split.  Measured at M = 1 on the 70B QKV shard: 7.0 us
// against 7.3 us + 4.2 us (split + a separate finishing kernel, the split's
// form when this kernel was written).  Eight tokens measured slower than the
// split streams (16.3 against about 10 us at 70B TP = 8): one wave per row
// (1280 waves), eight times the VALU and LDS work per weight byte, and 128
// KB of activations in LDS leave too little in flight.  (For wide outputs
// and for the MLP the matrix-core streams are as fast or faster; they stay
// there.)
//
// The activations of the M tokens (M x K bf16) are copied into LDS once per
// workgroup; per chunk each lane reads its 16 bytes of every token from
// there.  A row's sum is finished with a butterfly over the wave's 64 lanes
// (every lane ends with the same bits, the order fixed: the result is
// deterministic) and written by the lanes of the tokens.
#include "common.h"
#include "internal.h"

namespace tpmlp {

namespace {

constexpr int kGWaves = 8;      // waves per workgroup (they share the activations in LDS)
constexpr int kGChunk = 512;    // k per load instruction of a wave (1 KB of bf16)
constexpr int kGUnroll = 8;     // load instructions in flight per wave

// Largest K held in LDS (static: 32 KB per token).
constexpr int kGKmax = 16384;

__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// acc + the dot product of eight bf16 pairs, in pair order.  (The pairs are
// taken by name: a loop over the vector's elements compiled to four uses of
// element 0.)
__device__ __forceinline__ float dot8(u32x4 w, u32x4 x, float acc) {
  const uint32_t w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;
  const uint32_t x0 = x.x, x1 = x.y, x2 = x.z, x3 = x.w;
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), __builtin_bit_cast(bf16x2, x0), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), __builtin_bit_cast(bf16x2, x1), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w2), __builtin_bit_cast(bf16x2, x2), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w3), __builtin_bit_cast(bf16x2, x3), acc, false);
  return acc;
}

// Sum over the 64 lanes; every lane returns the same value.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// RPW consecutive rows of w per wave (nrows of them); out = w * act^T,
// fp32 or (OBF) bf16, M x nrows with leading dimension ldo.
template <int MT, int RPW, bool OBF>
__global__ __launch_bounds__(kGWaves * 64) void gemv_kernel(int M, int K, int nrows, const XRows xr,
                                                          const uint16_t* __restrict__ w, int64_t ldw,
                                                          void* __restrict__ out, int64_t ldo) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[MT * kGKmax];   // MT x K, row length K
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // activations into LDS, token rows past M as zeros
  {
    const int per_row = K / 8;
    for (int i = tid; i < MT * per_row; i += kGWaves * 64) {
      const int m = i / per_row, c = i - m * per_row;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (m < M) v = *reinterpret_cast<const u32x4*>(x_row<uint16_t>(xr, m) + (int64_t)c * 8);
      *reinterpret_cast<u32x4*>(xs + (int64_t)m * K + (int64_t)c * 8) = v;
    }
  }
  __syncthreads();

  const int row0 = (blockIdx.x * kGWaves + wave) * RPW;   // first row of this wave
  if (row0 >= nrows) return;                                // (no barrier follows)
  // row r (0 .. RPW-1) of this wave; rows past nrows re-read the last one
  auto row_ptr = [&](int r) -> const uint16_t* { return w + (int64_t)min(row0 + r, nrows - 1) * ldw; };
  const int KC = K / kGChunk;
  const int T = RPW * KC;                                  // chunks this wave streams
  const int NG = (T + kGUnroll - 1) / kGUnroll;

  // Next chunk to load (row, chunk).  Loads are issued unconditionally (past
  // the end they repeat the last chunk, just read: a cache hit), so the
  // compiler can count them and wait only for the group it consumes; loads
  // behind a branch make it wait for all of them.
  int lr = 0, lc = 0;
  auto load_group = [&](u32x4 (&dst)[kGUnroll]) {
#pragma unroll
    for (int u = 0; u < kGUnroll; ++u) {
      const bool live = lr < RPW;
      dst[u] = ld16_nt(row_ptr(live ? lr : RPW - 1) + (int64_t)(live ? lc : KC - 1) * kGChunk + lane * 8);
      if (live && ++lc == KC) {
        lc = 0;
        ++lr;
      }
    }
  };

  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.f;
  auto finish_row = [&](int r) {
    const int row = row0 + r;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float tot = wave_sum(acc[m]);
      acc[m] = 0.f;
      if (lane == m && m < M && row < nrows) {
        if constexpr (OBF)
          reinterpret_cast<uint16_t*>(out)[(int64_t)m * ldo + row] = (uint16_t)f32_to_bf16_bits(tot);
        else
          reinterpret_cast<float*>(out)[(int64_t)m * ldo + row] = tot;
      }
    }
  };

  int pr = 0, pc = 0;   // next chunk to accumulate
  auto proc_group = [&](const u32x4 (&src)[kGUnroll]) {
#pragma unroll
    for (int u = 0; u < kGUnroll; ++u) {
      if (pr < RPW) {   // wave-uniform
        const uint16_t* xk = xs + (int64_t)pc * kGChunk + lane * 8;
#pragma unroll
        for (int m = 0; m < MT; ++m)
          acc[m] = dot8(src[u], *reinterpret_cast<const u32x4*>(xk + (int64_t)m * K), acc[m]);
        if (++pc == KC) {
          finish_row(pr);
          pc = 0;
          ++pr;
        }
      }
    }
  };

  u32x4 wa[kGUnroll], wb[kGUnroll];
  load_group(wa);
  for (int g = 0; g < NG; g += 2) {
    load_group(wb);
    proc_group(wa);
    load_group(wa);
    proc_group(wb);
  }
}

template <int MT, bool OBF>
hipError_t run_gemv(const RowGemm& g, const XRows& xr, hipStream_t stream) {
  // rows per wave: about 2048 waves for the chip (8 per CU), at most 4 rows
  auto go = [&](auto kernel, int rpw) {
    const int waves = (g.N + rpw - 1) / rpw;
    return launch(g.kind_decode, kernel, dim3((unsigned)((waves + kGWaves - 1) / kGWaves)), dim3(kGWaves * 64), 0,
                  stream, g.M, g.K, g.N, xr, (const uint16_t*)g.w, g.ldw, g.out, g.ldo);
  };
  if (g.N >= 8192) return go(gemv_kernel<MT, 4, OBF>, 4);
  if (g.N >= 4096) return go(gemv_kernel<MT, 2, OBF>, 2);
  return go(gemv_kernel<MT, 1, OBF>, 1);
}

}  // namespace

bool gemv_supported(int M, int K, int wb) {
  return wb == kWeightWide && M >= 1 && M <= kGemvMaxM && K % kGChunk == 0 && K <= kGKmax;
}

hipError_t launch_rowgemm_gemv(const RowGemm& g, hipStream_t stream) {
  XRows ar{};
  ar.p[0] = g.a;
  ar.nb = 1;
  ar.rows = g.M;
  ar.ld = g.lda;
  if (g.M <= 1) return g.out_bf16 ? run_gemv<1, true>(g, ar, stream) : run_gemv<1, false>(g, ar, stream);
  return g.out_bf16 ? run_gemv<2, true>(g, ar, stream) : run_gemv<2, false>(g, ar, stream);
}

}  // namespace tpmlp
