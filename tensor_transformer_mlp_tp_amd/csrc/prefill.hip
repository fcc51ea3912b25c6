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
// Both compute C^T = W * act^T with K-contiguous operands (the (out, in)
// weight layout and row-major activations): 256 x 256 output tiles, BK = 64,
// four waves in a 2 x 2 grid with a 128 x 128 sub-tile each, built from
// 32x32x16 bf16 MFMAs (the full-rate bf16 matrix instruction on gfx950;
// 4 x 4 blocks = 256 fp32 accumulators per lane, held in AGPRs).
//
// Global -> LDS: direct-to-LDS 16-byte loads (global_load_lds_dwordx4), two
// stages.  The loads of k-tile kt+1 are issued right after the barrier that
// opens k-tile kt and land while its MFMAs run; nothing is staged in VGPRs.
// Rows past M (tokens) or N (channels) are loaded from the last valid row: a
// row of the output depends only on its own activation row and its own weight
// row, so those rows only feed outputs that are never stored.
//
// LDS rows are BK elements (128 B bf16, 64 B fp8) split in 16-byte chunks
// stored XOR-swizzled by row.  gfx950's LDS has 64 four-byte banks and serves
// a 16-byte-per-lane read 16 lanes per cycle, so the 16 rows those lanes read
// (same logical chunk) must land in 16 different 16-byte bank slots: physical
// chunk = logical ^ ((row >> 1) & 7) for 128-byte rows (rows of equal parity
// then differ in chunk) and logical ^ ((row >> 2) & 3) for 64-byte rows.  A
// direct-to-LDS load writes 64 consecutive 16-byte slots, so the swizzle is
// applied by choosing which global chunk each lane fetches.
//
// A gate/up tile holds 128 channels: LDS weight rows 0-127 are their gate
// rows and 128-255 their up rows; a wave's four 32-row blocks are two gate
// blocks and the matching two up blocks, so SiLU(G) * U is formed in
// registers.
//
// fp8 (e4m3fn) weights are staged in LDS as bytes (half the traffic) and
// widened to bf16 (exact) when the fragments are read; one 16-byte LDS read
// gives a lane the k values of two MFMA steps, and the activation fragments
// are read in the same k order.  Per-channel scales multiply the fp32
// accumulators in the epilogue.
//
// Workgroup-to-tile mapping: consecutive workgroup ids are dispatched
// round-robin to the eight XCDs, each with its own L2, so the id is first
// folded so that every XCD receives a contiguous run of tiles, and the run is
// walked in groups of four M-tiles, which keeps the activation and weight
// panels of concurrently running workgroups inside one L2.
#include "common.h"
#include "internal.h"

namespace tpmlp {

namespace {

constexpr int BM = 256;      // tokens per tile
constexpr int BN = 256;      // weight rows per tile
constexpr int BK = 64;       // k per stage
constexpr int THREADS = 256; // 4 waves
constexpr int GROUP_M = 4;

typedef float f32x16 __attribute__((ext_vector_type(16)));

// 32x32x16 bf16 MFMA: D(32x32) += A(32x16) * B(16x32).  Lane l supplies row
// (l % 32) of A and column (l % 32) of B with the eight k values of group
// (l / 32); it receives D[8*(i/4) + 4*(l/32) + i%4][l % 32], i = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void load_lds16(const void* gsrc, void* lds_dst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gsrc,
                                   (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}

__device__ __forceinline__ u32x4 lds_read16(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// Physical 16-byte chunk of a logical chunk: 128-byte and 64-byte LDS rows.
__device__ __forceinline__ int swz128(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz64(int row) { return (row >> 2) & 3; }

// Scheduling groups for one sub-step: its 16 MFMAs with NDS fragment reads
// of the next sub-step threaded one after each of the first NDS MFMAs.
template <int NDS>
__device__ __forceinline__ void sched_substep() {
#pragma unroll
  for (int i = 0; i < NDS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 16 - NDS, 0);
}

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
  constexpr int WROWB = BK * EB;               // bytes per LDS weight row
  constexpr int XBYTES = BM * BK * 2;          // activation stage (32 KB)
  constexpr int WBYTES = BN * WROWB;           // weight stage (32 KB / 16 KB)
  constexpr int SBYTES = XBYTES + WBYTES;
  constexpr int XINST = XBYTES / 1024 / 4;     // 1 KB direct loads per wave per stage
  constexpr int WINST = WBYTES / 1024 / 4;
  constexpr int TILE_N = SWIGLU ? BN / 2 : BN; // output columns per tile

  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * SBYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int r32 = lane & 31, g = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;

  const TileCoord tc = tile_of_block(blockIdx.x, tiles_m, tiles_n);
  const int m0 = tc.tm * BM;
  const int n0 = tc.tn * TILE_N;

  // ---- direct-to-LDS sources: instruction i of this wave fills LDS bytes
  // [(wave*INST + i) KB, +1 KB) of the stage; lane l fills 16 bytes of it.
  const uint8_t* xsrc[XINST];
#pragma unroll
  for (int i = 0; i < XINST; ++i) {
    const int row = (wave * XINST + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz128(row);
    const int tok = min(m0 + row, M - 1);
    xsrc[i] = reinterpret_cast<const uint8_t*>(act + (int64_t)tok * ld_act) + c * 16;
  }
  const uint8_t* wsrc[WINST];
#pragma unroll
  for (int i = 0; i < WINST; ++i) {
    int row, c;
    if constexpr (FP8) {
      row = (wave * WINST + i) * 16 + (lane >> 2);
      c = (lane & 3) ^ swz64(row);
    } else {
      row = (wave * WINST + i) * 8 + (lane >> 3);
      c = (lane & 7) ^ swz128(row);
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
    wsrc[i] = base + (int64_t)min(ch, N - 1) * ldw * EB + c * 16;
  }
  auto issue_stage = [&](int kt, int buf) {
    uint8_t* xdst = lds + buf * SBYTES + wave * XINST * 1024;
    uint8_t* wdst = lds + buf * SBYTES + XBYTES + wave * WINST * 1024;
#pragma unroll
    for (int i = 0; i < XINST; ++i) load_lds16(xsrc[i] + (int64_t)kt * BK * 2, xdst + i * 1024);
#pragma unroll
    for (int i = 0; i < WINST; ++i) load_lds16(wsrc[i] + (int64_t)kt * BK * EB, wdst + i * 1024);
  };

  // ---- fragment rows of this lane inside a stage
  int wrow[4], xrow[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    if constexpr (SWIGLU)
      wrow[cb] = (cb < 2 ? 0 : BN / 2) + wn * 64 + (cb & 1) * 32 + r32;
    else
      wrow[cb] = wn * 128 + cb * 32 + r32;
  }
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) xrow[tb] = wm * 128 + tb * 32 + r32;

  f32x16 acc[4][4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[cb][tb][i] = 0.f;

  // Fragments of sub-step kk (16 k).  bf16: lane group g holds chunk 2kk+g of
  // both operands.  fp8: at even kk the weight lane reads 16-byte chunk kk+g
  // (16 codes) once; its low 8 codes serve sub-step kk and its high 8 codes
  // sub-step kk+1, so the activation chunk of 8 elements is 4*(kk/2) + 2g +
  // kk%2.
  u32x4 wq[4];
  auto read_frags = [&](const uint8_t* sx, const uint8_t* sw, int kk, bf16x8 (&wf)[4], bf16x8 (&xf)[4]) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int r = wrow[cb];
      if constexpr (FP8) {
        if ((kk & 1) == 0) {
          const int q = kk + g;
          wq[cb] = lds_read16(sw + r * WROWB + ((q ^ swz64(r)) * 16));
          wf[cb] = fp8x8_to_bf16x8(wq[cb][0], wq[cb][1]);
        } else {
          wf[cb] = fp8x8_to_bf16x8(wq[cb][2], wq[cb][3]);
        }
      } else {
        const int ch = 2 * kk + g;
        wf[cb] = as_bf16x8(lds_read16(sw + r * WROWB + ((ch ^ swz128(r)) * 16)));
      }
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int r = xrow[tb];
      const int ch = FP8 ? (4 * (kk >> 1) + 2 * g + (kk & 1)) : (2 * kk + g);
      xf[tb] = as_bf16x8(lds_read16(sx + r * 128 + ((ch ^ swz128(r)) * 16)));
    }
  };

  // Main loop, one barrier per k-tile.  The body is a single basic block (the
  // last iteration re-loads its own k-tile into the idle buffer rather than
  // branching), so the scheduling groups below order the whole of it: the
  // direct loads of the next k-tile first, then the fragments of sub-step 0,
  // then each sub-step's 16 MFMAs with the 8 fragment reads of the following
  // sub-step threaded between them, so the matrix core never waits on LDS
  // inside a k-tile.
  const int KT = K / BK;
  issue_stage(0, 0);
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads of stage kt have landed
    __syncthreads();                // ... and every wave's; stage kt-1 is no longer read
    issue_stage(min(kt + 1, KT - 1), cur ^ 1);
    const uint8_t* sx = lds + cur * SBYTES;
    const uint8_t* sw = sx + XBYTES;
    bf16x8 wf[2][4], xf[2][4];
    read_frags(sx, sw, 0, wf[0], xf[0]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk + 1 < 4) read_frags(sx, sw, kk + 1, wf[(kk + 1) & 1], xf[(kk + 1) & 1]);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) acc[cb][tb] = mfma32(wf[kk & 1][cb], xf[kk & 1][tb], acc[cb][tb]);
    }
    // fragment reads per sub-step: 8 (bf16); fp8: 8 at even sub-steps
    // (4 weight + 4 activation), 4 at odd ones (activations only)
    __builtin_amdgcn_sched_group_barrier(0x020, XINST + WINST, 0);  // direct loads
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);              // fragments of sub-step 0
    sched_substep<FP8 ? 4 : 8>();
    sched_substep<8>();
    sched_substep<FP8 ? 4 : 8>();
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);  // no direct load is left in flight at exit

  // ---- epilogue.  Lane holds, per block, rows 8j + 4g + (0..3) (j = 0..3)
  // of weight-row block cb for token column r32 of block tb.
  if constexpr (SWIGLU) {
    uint16_t* a_out = reinterpret_cast<uint16_t*>(out);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ch = n0 + wn * 64 + cb * 32 + 8 * j + 4 * g;  // channels ch .. ch+3
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
        for (int tb = 0; tb < 4; ++tb) {
          const int tok = m0 + wm * 128 + tb * 32 + r32;
          if (tok >= M) continue;
          float a[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float gv = acc[cb][tb][4 * j + i], uv = acc[cb + 2][tb][4 * j + i];
            if constexpr (FP8) {
              gv *= sgv[i];
              uv *= suv[i];
            }
            a[i] = silu(gv) * uv;
          }
          u32x2 packed = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
          *reinterpret_cast<u32x2*>(a_out + (int64_t)tok * ld_out + ch) = packed;
        }
      }
    }
  } else {
    float* p = reinterpret_cast<float*>(out);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int f = n0 + wn * 128 + cb * 32 + 8 * j + 4 * g;  // features f .. f+3
        if (f >= N) continue;
        float sv[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (FP8) {
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[i] = s0[f + i];
        }
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          const int tok = m0 + wm * 128 + tb * 32 + r32;
          if (tok >= M) continue;
          f32x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = acc[cb][tb][4 * j + i] * sv[i];
          *reinterpret_cast<f32x4*>(p + (int64_t)tok * ld_out + f) = v;
        }
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
