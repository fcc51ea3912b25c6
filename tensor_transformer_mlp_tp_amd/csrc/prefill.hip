// MFMA GEMM kernels for many tokens (prefill).
//
// At prefill the rank's MLP is a dense contraction (6*M*h*I_s FLOP against
// 3*h*I_s weights: ~1650 FLOP/byte at 4096 tokens), so it runs on the bf16
// matrix cores.  Two kernels:
//
//   gate/up:  G|U = X * [W_gate_k; W_up_k]^T with SiLU(G) * U in the epilogue,
//             A written once in bf16 (column-parallel projections with the
//             activation applied locally: "The Tensor-Parallel Shard Group",
//             scalablesystem.dev; vidyal.ai "Step 1").
//   down:     P_k = A * W_down_k^T written once in fp32 (the row-parallel
//             partial).
//
// Both are C^T = W * act^T with K-contiguous operands (the (out, in) weight
// layout and row-major activations), 256 x 256 output tiles, BK = 64, four
// waves in a 2 x 2 grid with a 128 x 128 sub-tile each (8 x 8 MFMA 16x16x32
// blocks: 256 fp32 accumulators per lane), and a two-stage LDS ring filled
// with 16-byte global loads staged through registers: the loads for k-tile
// kt+1 are in flight while the MFMAs of kt run, with one barrier per k-tile.
//
// LDS rows are BK elements (128 B bf16, 64 B fp8) split in 16-byte chunks
// stored XOR-swizzled by row, so the eight lanes that share an LDS cycle in a
// 16-byte fragment read hit eight different bank groups.
//
// A gate/up tile holds 128 channels: LDS weight rows 0-127 are their gate
// rows and 128-255 their up rows, and a wave's 8 row blocks are 4 gate + the
// matching 4 up blocks, so SiLU(G) * U is formed in registers.
//
// fp8 (e4m3fn) weights are staged in LDS as bytes (half the traffic) and
// widened to bf16 when the fragments are read; one 16-byte LDS read gives a
// lane 16 codes = the k values of two MFMA steps, and the activation
// fragments are read in the same k order.  Per-channel scales multiply the
// fp32 accumulators in the epilogue.
//
// Workgroup-to-tile mapping: consecutive workgroup ids are dispatched
// round-robin to the eight XCDs, each with its own L2, so the id is first
// folded so that every XCD receives a contiguous run of tiles, and the run is
// walked in groups of four M-tiles, which keeps the activation and weight
// panels a set of concurrently running workgroups needs inside one L2.
#include "common.h"
#include "internal.h"

namespace tpmlp {

namespace {

constexpr int BM = 256;      // tokens per tile
constexpr int BN = 256;      // weight rows per tile
constexpr int BK = 64;       // k per stage
constexpr int THREADS = 256; // 4 waves
constexpr int GROUP_M = 4;

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

struct TileCoord {
  int tm, tn;
};

__device__ __forceinline__ TileCoord tile_of_block(int b, int tiles_m, int tiles_n) {
  const int nb = tiles_m * tiles_n;
  const int xcd = b & 7, local = b >> 3;
  const int q = nb >> 3, r = nb & 7;
  const int L = xcd * q + min(xcd, r) + local;
  const int per_group = GROUP_M * tiles_n;
  const int group = L / per_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int i = L - group * per_group;
  return TileCoord{first_m + i % gsize, i / gsize};
}

template <bool SWIGLU, bool FP8>
__global__ __launch_bounds__(THREADS, 1) void gemm_kernel(
    int M, int N, int K, const uint16_t* __restrict__ act, int64_t ld_act,
    const uint8_t* __restrict__ w0, const uint8_t* __restrict__ w1, int64_t ldw,
    const float* __restrict__ s0, const float* __restrict__ s1, void* __restrict__ out,
    int64_t ld_out, int tiles_m, int tiles_n) {
  constexpr int EB = FP8 ? 1 : 2;              // weight bytes per element
  constexpr int WCH = BK * EB / 16;            // 16-byte chunks per LDS weight row
  constexpr int XLOADS = BM * 8 / THREADS;     // activation chunks per thread per stage (8)
  constexpr int WLOADS = BN * WCH / THREADS;   // weight chunks per thread per stage (8 or 4)
  constexpr int TILE_N = SWIGLU ? BN / 2 : BN; // output columns per tile

  __shared__ u32x4 lds_x[2][BM * 8];
  __shared__ u32x4 lds_w[2][BN * WCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int row16 = lane & 15, grp = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;

  const TileCoord tc = tile_of_block(blockIdx.x, tiles_m, tiles_n);
  const int m0 = tc.tm * BM;
  const int n0 = tc.tn * TILE_N;

  // ---- global load addressing (fixed per thread, advanced by BK per stage)
  const uint16_t* xsrc[XLOADS];
  bool xok[XLOADS];
  int xdst[XLOADS];
#pragma unroll
  for (int i = 0; i < XLOADS; ++i) {
    const int q = tid + THREADS * i;
    const int row = q >> 3, c = q & 7;
    const int tok = m0 + row;
    xok[i] = tok < M;
    xsrc[i] = act + (int64_t)min(tok, M - 1) * ld_act + c * 8;
    xdst[i] = row * 8 + (c ^ (row & 7));
  }
  const uint8_t* wsrc[WLOADS];
  bool wok[WLOADS];
  int wdst[WLOADS];
#pragma unroll
  for (int i = 0; i < WLOADS; ++i) {
    const int q = tid + THREADS * i;
    int row, c, sw;
    if constexpr (FP8) {
      row = q >> 2; c = q & 3; sw = c ^ ((row >> 1) & 3);
    } else {
      row = q >> 3; c = q & 7; sw = c ^ (row & 7);
    }
    int ch;
    const uint8_t* base;
    if constexpr (SWIGLU) {
      ch = n0 + (row & (BN / 2 - 1));
      base = row < BN / 2 ? w0 : w1;
    } else {
      ch = n0 + row;
      base = w0;
    }
    wok[i] = ch < N;
    wsrc[i] = base + ((int64_t)min(ch, N - 1) * ldw) * EB + c * 16;
    wdst[i] = row * WCH + sw;
  }

  u32x4 xs[XLOADS], ws[WLOADS];
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto load_stage = [&](int kt) {
#pragma unroll
    for (int i = 0; i < XLOADS; ++i) {
      const u32x4 v = ld16(xsrc[i] + (int64_t)kt * BK);
      xs[i] = xok[i] ? v : zero;
    }
#pragma unroll
    for (int i = 0; i < WLOADS; ++i) {
      const u32x4 v = ld16(wsrc[i] + (int64_t)kt * BK * EB);
      ws[i] = wok[i] ? v : zero;
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XLOADS; ++i) lds_x[buf][xdst[i]] = xs[i];
#pragma unroll
    for (int i = 0; i < WLOADS; ++i) lds_w[buf][wdst[i]] = ws[i];
  };

  // ---- LDS fragment rows of this lane
  int wrow[8], xrow[8];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    if constexpr (SWIGLU)
      wrow[cb] = (cb < 4 ? 0 : BN / 2) + wn * 64 + (cb & 3) * 16 + row16;
    else
      wrow[cb] = wn * 128 + cb * 16 + row16;
  }
#pragma unroll
  for (int tb = 0; tb < 8; ++tb) xrow[tb] = wm * 128 + tb * 16 + row16;

  f32x4 acc[8][8];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb)
#pragma unroll
    for (int tb = 0; tb < 8; ++tb) acc[cb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute_stage = [&](int buf) {
    u32x4 wq[8];
    if constexpr (FP8) {
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) wq[cb] = lds_w[buf][wrow[cb] * WCH + (grp ^ ((wrow[cb] >> 1) & 3))];
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 wf[8], xf[8];
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        if constexpr (FP8) {
          wf[cb] = kk == 0 ? fp8x8_to_bf16x8(wq[cb][0], wq[cb][1]) : fp8x8_to_bf16x8(wq[cb][2], wq[cb][3]);
        } else {
          const int ch = kk * 4 + grp;
          wf[cb] = as_bf16x8(lds_w[buf][wrow[cb] * 8 + (ch ^ (wrow[cb] & 7))]);
        }
      }
#pragma unroll
      for (int tb = 0; tb < 8; ++tb) {
        const int ch = FP8 ? (2 * grp + kk) : (kk * 4 + grp);
        xf[tb] = as_bf16x8(lds_x[buf][xrow[tb] * 8 + (ch ^ (xrow[tb] & 7))]);
      }
#pragma unroll
      for (int cb = 0; cb < 8; ++cb)
#pragma unroll
        for (int tb = 0; tb < 8; ++tb) acc[cb][tb] = mfma16(wf[cb], xf[tb], acc[cb][tb]);
    }
  };

  // ---- main loop: two-stage ring, one barrier per k-tile
  const int KT = K / BK;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_stage(kt + 1);
    compute_stage(cur);
    if (kt + 1 < KT) store_stage(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  Lane holds D[4*grp + i][row16] of each block: four
  // consecutive weight rows (channels / features) of one token.
  if constexpr (SWIGLU) {
    uint16_t* a_out = reinterpret_cast<uint16_t*>(out);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int ch = n0 + wn * 64 + cb * 16 + 4 * grp;
      if (ch >= N) continue;
      float sgv[4] = {1.f, 1.f, 1.f, 1.f}, suv[4] = {1.f, 1.f, 1.f, 1.f};
      if constexpr (FP8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sgv[i] = s0[ch + i];
          suv[i] = s1[ch + i];
        }
      }
#pragma unroll
      for (int tb = 0; tb < 8; ++tb) {
        const int tok = m0 + wm * 128 + tb * 16 + row16;
        if (tok >= M) continue;
        float a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float g = acc[cb][tb][i], u = acc[cb + 4][tb][i];
          if constexpr (FP8) {
            g *= sgv[i];
            u *= suv[i];
          }
          a[i] = silu(g) * u;
        }
        u32x2 packed = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
        *reinterpret_cast<u32x2*>(a_out + (int64_t)tok * ld_out + ch) = packed;
      }
    }
  } else {
    float* p = reinterpret_cast<float*>(out);
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const int f = n0 + wn * 128 + cb * 16 + 4 * grp;
      if (f >= N) continue;
      float sv[4] = {1.f, 1.f, 1.f, 1.f};
      if constexpr (FP8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[i] = s0[f + i];
      }
#pragma unroll
      for (int tb = 0; tb < 8; ++tb) {
        const int tok = m0 + wm * 128 + tb * 16 + row16;
        if (tok >= M) continue;
        f32x4 v = acc[cb][tb];
        if constexpr (FP8) {
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] *= sv[i];
        }
        *reinterpret_cast<f32x4*>(p + (int64_t)tok * ld_out + f) = v;
      }
    }
  }
}

template <bool FP8>
hipError_t run_prefill(const ShardArgs& a, hipStream_t stream) {
  const int tiles_m = (a.M + BM - 1) / BM;
  const dim3 block(THREADS);
  {
    const int tiles_n = (a.I_s + BN / 2 - 1) / (BN / 2);
    const dim3 grid((unsigned)(tiles_m * tiles_n));
    hipError_t e = launch(K_GATEUP_PREFILL, gemm_kernel<true, FP8>, grid, block, 0, stream, a.M, a.I_s,
                          a.h, (const uint16_t*)a.x, a.ldx, (const uint8_t*)a.wg,
                          (const uint8_t*)a.wu, a.ldw_gu, a.sg, a.su, a.a, a.lda, tiles_m, tiles_n);
    if (e != hipSuccess) return e;
  }
  const int tiles_n = (a.h + BN - 1) / BN;
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  return launch(K_DOWN_PREFILL, gemm_kernel<false, FP8>, grid, block, 0, stream, a.M, a.h, a.I_s,
                (const uint16_t*)a.a, a.lda, (const uint8_t*)a.wd, (const uint8_t*)nullptr,
                a.ldw_down, a.sd, (const float*)nullptr, (void*)a.p, a.ldp, tiles_m, tiles_n);
}

}  // namespace

hipError_t launch_forward_prefill(const ShardArgs& a, hipStream_t stream) {
  return a.fp8 ? run_prefill<true>(a, stream) : run_prefill<false>(a, stream);
}

}  // namespace tpmlp
