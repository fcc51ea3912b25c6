// Weight-streaming kernels for small token counts (decode, M <= 64).
//
// At decode the time of a rank's MLP is the time to read its weight shards
// ("decode is limited by how fast a GPU reads its weights": vidyal.ai page,
// "Why it matters"), so both kernels are built around one thing: every byte
// of W_gate_k / W_up_k / W_down_k is read from HBM exactly once, with 16-byte
// loads per lane, many in flight per wave, and the dot products done on the
// matrix cores (fp32 VALU cannot keep up at M = 64: 11 GFLOP per rank).
//
// MFMA orientation: the weight rows are the MFMA "A" rows (16 per block) and
// the tokens its "B" columns (16 per block, zero-padded past M), so
// D[row][token] leaves each lane with four consecutive rows of one token.
//
// Gate/up kernel: one workgroup owns 8*RB intermediate channels.  Each 16-row
// MFMA block holds 8 gate rows (rows 0-7) and the same 8 channels' up rows
// (rows 8-15), so after the MMA lane l (< 32) and lane l + 32 hold gate and up
// of the same four channels and token: one cross-half swap pairs them and
// SiLU(gate) * up is applied in registers (SwiGLU fused into the epilogue;
// activation applied locally after the column split: vidyal.ai, "Step 1").
// The WAVES waves of a workgroup split the hidden (K) dimension into
// contiguous ranges and their fp32 partial sums are added through LDS in wave
// order, so results are deterministic.
//
// Down kernel: one workgroup owns 16*RB output features (rows of W_down_k),
// waves split I_s, same fixed-order LDS reduction, fp32 partial written once
// (the row-parallel partial of "The Tensor-Parallel Shard Group").
//
// fp8 weights (OCP e4m3fn): each lane's 16-byte load carries 16 codes of one
// row = two MFMA k-groups; they are widened to bf16 in registers (exact) and
// the per-output-channel fp32 scale is applied to the fp32 sums.  The
// activations are read with the same k order, so the dot products are exact
// reorderings of the definition.
#include "common.h"
#include "internal.h"

namespace tpmlp {

namespace {

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Weights are read exactly once per call: non-temporal loads keep them from
// displacing the activations, which every workgroup re-reads from L2.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// A batch of U consecutive k-steps held in registers.  A step is 32 k (bf16
// weights) or 64 k (fp8 weights): one 16-byte weight load per lane per row
// block, plus the matching activation fragments.
template <int NT, int RB, int U, bool FP8>
struct Batch {
  static constexpr int XJ = FP8 ? 2 : 1;
  u32x4 wf[U][RB];
  u32x4 xf[U][NT][XJ];
};

// Issue the loads of the batch starting at step s.  Steps at or past s_end
// (only in the last, partial batch) re-read step s_end - 1, which is valid
// memory; their products are skipped in mac_batch.
template <int NT, int RB, int U, bool FP8>
__device__ __forceinline__ void load_batch(Batch<NT, RB, U, FP8>& bt, const uint8_t* const (&wrow)[RB],
                                           const uint16_t* const (&xrow)[NT], int s, int s_end, int grp) {
  constexpr int KSTEP = FP8 ? 64 : 32;
  constexpr int EB = FP8 ? 1 : 2;
  constexpr int XJ = FP8 ? 2 : 1;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t st = min(s + u, s_end - 1);
#pragma unroll
    for (int r = 0; r < RB; ++r) bt.wf[u][r] = ld16_stream(wrow[r] + st * KSTEP * EB + grp * 16);
#pragma unroll
    for (int b = 0; b < NT; ++b)
#pragma unroll
      for (int j = 0; j < XJ; ++j) bt.xf[u][b][j] = ld16(xrow[b] + st * KSTEP + grp * (8 * XJ) + j * 8);
  }
}

// MFMAs of the first n (<= U) steps of a loaded batch.  Token rows past M
// were loaded from a clamped row and are zeroed here.
template <int NT, int RB, int U, bool FP8>
__device__ __forceinline__ void mac_batch(f32x4 (&acc)[RB][NT], const Batch<NT, RB, U, FP8>& bt,
                                          const bool (&xok)[NT], int n) {
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u >= n) break;  // wave-uniform
    bf16x8 xv[NT][FP8 ? 2 : 1];
#pragma unroll
    for (int b = 0; b < NT; ++b)
#pragma unroll
      for (int j = 0; j < (FP8 ? 2 : 1); ++j) xv[b][j] = as_bf16x8(xok[b] ? bt.xf[u][b][j] : zero);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      if constexpr (FP8) {
        const bf16x8 lo = fp8x8_to_bf16x8(bt.wf[u][r][0], bt.wf[u][r][1]);
        const bf16x8 hi = fp8x8_to_bf16x8(bt.wf[u][r][2], bt.wf[u][r][3]);
#pragma unroll
        for (int b = 0; b < NT; ++b) {
          acc[r][b] = mfma16(lo, xv[b][0], acc[r][b]);
          acc[r][b] = mfma16(hi, xv[b][1], acc[r][b]);
        }
      } else {
        const bf16x8 w = as_bf16x8(bt.wf[u][r]);
#pragma unroll
        for (int b = 0; b < NT; ++b) acc[r][b] = mfma16(w, xv[b][0], acc[r][b]);
      }
    }
  }
}

// Steps [s_beg, s_end) with two register batches in flight: the loads of
// batch i+1 are issued before the MFMAs of batch i.
template <int NT, int RB, int U, bool FP8>
__device__ __forceinline__ void mac_range(f32x4 (&acc)[RB][NT], const uint8_t* const (&wrow)[RB],
                                          const uint16_t* const (&xrow)[NT], const bool (&xok)[NT],
                                          int s_beg, int s_end, int grp) {
  if (s_beg >= s_end) return;
  Batch<NT, RB, U, FP8> b0, b1;
  int s = s_beg;
  load_batch(b0, wrow, xrow, s, s_end, grp);
  while (true) {
    int nxt = s + U;
    if (nxt < s_end) load_batch(b1, wrow, xrow, nxt, s_end, grp);
    mac_batch(acc, b0, xok, s_end - s);
    if (nxt >= s_end) break;
    s = nxt;
    nxt = s + U;
    if (nxt < s_end) load_batch(b0, wrow, xrow, nxt, s_end, grp);
    mac_batch(acc, b1, xok, s_end - s);
    if (nxt >= s_end) break;
    s = nxt;
  }
}

// Sum the WAVES partial accumulators of (row block r, token block b) pairs in
// wave order and hand each finished pair to `epi`.  Pairs are spread over the
// waves.
template <int NT, int RB, int WAVES, typename Epi>
__device__ __forceinline__ void reduce_waves(f32x4 (&acc)[RB][NT], int wave, int lane, Epi epi) {
  if constexpr (WAVES == 1) {
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int b = 0; b < NT; ++b) epi(r, b, acc[r][b]);
  } else {
    __shared__ f32x4 red[WAVES][RB * NT][64];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int b = 0; b < NT; ++b) red[wave][r * NT + b][lane] = acc[r][b];
    __syncthreads();
    for (int q = wave; q < RB * NT; q += WAVES) {
      f32x4 s = red[0][q][lane];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) s = s + red[w][q][lane];
      epi(q / NT, q % NT, s);
    }
  }
}

template <int NT, int RB, int WAVES, int UNROLL, bool FP8>
__global__ __launch_bounds__(WAVES * 64) void gateup_decode_kernel(
    int M, int h, int I_s, const uint16_t* __restrict__ x, int64_t ldx,
    const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu, int64_t ldw,
    const float* __restrict__ sg, const float* __restrict__ su,
    uint16_t* __restrict__ a_out, int64_t lda) {
  constexpr int EB = FP8 ? 1 : 2;
  constexpr int KSTEP = FP8 ? 64 : 32;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int row16 = lane & 15;
  const int grp = lane >> 4;
  const int c0 = blockIdx.x * (8 * RB);

  const uint8_t* wrow[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int ch = min(c0 + 8 * r + (row16 & 7), I_s - 1);
    wrow[r] = (row16 < 8 ? wg : wu) + (int64_t)ch * ldw * EB;
  }
  const uint16_t* xrow[NT];
  bool xok[NT];
#pragma unroll
  for (int b = 0; b < NT; ++b) {
    const int tok = b * 16 + row16;
    xok[b] = tok < M;
    xrow[b] = x + (int64_t)min(tok, M - 1) * ldx;
  }

  const int nsteps = h / KSTEP;
  const int s_beg = (wave * nsteps) / WAVES;
  const int s_end = ((wave + 1) * nsteps) / WAVES;
  f32x4 acc[RB][NT];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[r][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  mac_range<NT, RB, UNROLL, FP8>(acc, wrow, xrow, xok, s_beg, s_end, grp);

  reduce_waves<NT, RB, WAVES>(acc, wave, lane, [&](int r, int b, f32x4 v) {
    f32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __shfl_xor(v[i], 32);
    if (grp < 2) {
      const int ch = c0 + 8 * r + 4 * grp;  // four channels ch .. ch+3
      const int tok = b * 16 + row16;
      if (tok < M && ch < I_s) {
        float a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float g = v[i], u = o[i];
          if constexpr (FP8) {
            g *= sg[ch + i];
            u *= su[ch + i];
          }
          a[i] = silu(g) * u;
        }
        u32x2 packed = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
        *reinterpret_cast<u32x2*>(a_out + (int64_t)tok * lda + ch) = packed;
      }
    }
  });
}

template <int NT, int RB, int WAVES, int UNROLL, bool FP8>
__global__ __launch_bounds__(WAVES * 64) void down_decode_kernel(
    int M, int h, int I_s, const uint16_t* __restrict__ a_in, int64_t lda,
    const uint8_t* __restrict__ wd, int64_t ldw, const float* __restrict__ sd,
    float* __restrict__ p, int64_t ldp) {
  constexpr int EB = FP8 ? 1 : 2;
  constexpr int KSTEP = FP8 ? 64 : 32;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int row16 = lane & 15;
  const int grp = lane >> 4;
  const int n0 = blockIdx.x * (16 * RB);

  const uint8_t* wrow[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int f = min(n0 + 16 * r + row16, h - 1);
    wrow[r] = wd + (int64_t)f * ldw * EB;
  }
  const uint16_t* xrow[NT];
  bool xok[NT];
#pragma unroll
  for (int b = 0; b < NT; ++b) {
    const int tok = b * 16 + row16;
    xok[b] = tok < M;
    xrow[b] = a_in + (int64_t)min(tok, M - 1) * lda;
  }

  const int nsteps = I_s / KSTEP;
  const int s_beg = (wave * nsteps) / WAVES;
  const int s_end = ((wave + 1) * nsteps) / WAVES;
  f32x4 acc[RB][NT];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[r][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  mac_range<NT, RB, UNROLL, FP8>(acc, wrow, xrow, xok, s_beg, s_end, grp);

  reduce_waves<NT, RB, WAVES>(acc, wave, lane, [&](int r, int b, f32x4 v) {
    const int f = n0 + 16 * r + 4 * grp;  // features f .. f+3
    const int tok = b * 16 + row16;
    if (tok < M && f < h) {
      if constexpr (FP8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] *= sd[f + i];
      }
      *reinterpret_cast<f32x4*>(p + (int64_t)tok * ldp + f) = v;
    }
  });
}

// Launch shape (waves per workgroup splitting K; steps per register batch).
#ifndef TPMLP_DECODE_WAVES
#define TPMLP_DECODE_WAVES 4
#endif
#ifndef TPMLP_DECODE_UNROLL
#define TPMLP_DECODE_UNROLL 8
#endif
constexpr int kWaves = TPMLP_DECODE_WAVES;
constexpr int kUnroll = TPMLP_DECODE_UNROLL;

template <int NT, bool FP8>
hipError_t run_decode(const ShardArgs& a, hipStream_t stream) {
  // Row blocks per workgroup: with more token blocks, two weight blocks share
  // each activation fragment load.  Batches shrink as fragments per step grow.
  constexpr int RB_GU = NT >= 3 ? 2 : 1;
  constexpr int UN_GU = FP8 ? (NT >= 3 ? kUnroll / 4 : kUnroll / 2) : (NT >= 3 ? kUnroll / 2 : kUnroll);
  constexpr int RB_DN = 1;
  constexpr int UN_DN = FP8 ? (NT >= 3 ? kUnroll / 4 : kUnroll / 2) : (NT >= 3 ? kUnroll / 2 : kUnroll);
  const dim3 block(kWaves * 64);
  const dim3 grid_gu((a.I_s + 8 * RB_GU - 1) / (8 * RB_GU));
  hipError_t e = launch(K_GATEUP_DECODE, gateup_decode_kernel<NT, RB_GU, kWaves, UN_GU, FP8>, grid_gu,
                        block, 0, stream, a.M, a.h, a.I_s, (const uint16_t*)a.x, a.ldx,
                        (const uint8_t*)a.wg, (const uint8_t*)a.wu, a.ldw_gu, a.sg, a.su,
                        (uint16_t*)a.a, a.lda);
  if (e != hipSuccess) return e;
  const dim3 grid_dn((a.h + 16 * RB_DN - 1) / (16 * RB_DN));
  return launch(K_DOWN_DECODE, down_decode_kernel<NT, RB_DN, kWaves, UN_DN, FP8>, grid_dn, block, 0,
                stream, a.M, a.h, a.I_s, (const uint16_t*)a.a, a.lda, (const uint8_t*)a.wd,
                a.ldw_down, a.sd, a.p, a.ldp);
}

template <bool FP8>
hipError_t run_decode_nt(const ShardArgs& a, hipStream_t stream) {
  switch ((a.M + 15) / 16) {
    case 1: return run_decode<1, FP8>(a, stream);
    case 2: return run_decode<2, FP8>(a, stream);
    case 3: return run_decode<3, FP8>(a, stream);
    case 4: return run_decode<4, FP8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_forward_decode(const ShardArgs& a, hipStream_t stream) {
  return a.fp8 ? run_decode_nt<true>(a, stream) : run_decode_nt<false>(a, stream);
}

}  // namespace tpmlp
