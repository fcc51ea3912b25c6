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
// weight layout and row-major activations): output tiles of 256 weight rows
// by 256 tokens, four waves in a 2 x 2 grid with a 128 x 128 sub-tile each,
// built from 32x32x16 bf16 MFMAs (the full-rate bf16 matrix instruction on
// gfx950; 4 x 4 blocks = 256 fp32 accumulators per lane, held in AGPRs).
// With a few hundred tokens the tiles are 128 or 64 tokens high, the four
// waves side by side across the weight rows (tile_bm).
//
// Global -> LDS: direct-to-LDS 16-byte loads (global_load_lds_dwordx4) into a
// ring of NS stages of BK k-values; a stage's loads are issued NS-1 k-tiles
// before it is used and nothing is staged in VGPRs.  bf16 weights run two
// stages of 64 (128 KB); fp8 weights, with smaller stages, three.  Rows past M
// (tokens) or N (channels) are loaded from the last valid row: a row of the
// output depends only on its own activation row and its own weight row, so
// those rows only feed outputs that are never stored.
//
// LDS rows are BK elements split in 16-byte chunks stored XOR-swizzled by
// row.  gfx950's LDS has 64 four-byte banks and serves a 16-byte-per-lane
// read 16 lanes per cycle, so the 16 rows those lanes read (same logical
// chunk) must land in 16 different 16-byte bank slots (swz below; measured
// SQ_LDS_BANK_CONFLICT = 0).  A direct-to-LDS load writes 64 consecutive
// 16-byte slots, so the swizzle is applied by choosing which global chunk each
// lane fetches.
//
// A gate/up tile holds 128 channels: LDS weight rows 0-127 are their gate
// rows and 128-255 their up rows; a wave's four 32-row blocks are two gate
// blocks and the matching two up blocks, so SiLU(G) * U is formed in
// registers.
//
// fp8 (e4m3fn) weights are staged in LDS as bytes (half the traffic) and
// widened to bf16 (exact) when the fragments are read; one 16-byte LDS read
// gives a lane the k values of both MFMA steps of a stage, and the activation
// fragments are read in the same k order.  Per-channel scales multiply the
// fp32 accumulators in the epilogue.
//
// Workgroup-to-tile mapping: consecutive workgroup ids are dispatched
// round-robin to the eight XCDs, each with its own L2, so the id is first
// folded so that every XCD receives a contiguous run of tiles, and the run is
// walked in groups of four M-tiles, which keeps the activation and weight
// panels of concurrently running workgroups inside one L2.
//
// When the tiles do not fill whole rounds of the 256 CUs, the tiles of the
// last round are cut along K into pieces that together fill one round
// (stream-K; SkTail below), their fp32 sums added in a fixed order.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace tpmlp {

namespace {

constexpr int BN = 256;      // weight rows per tile
constexpr int GROUP_M = 4;

typedef float f32x16 __attribute__((ext_vector_type(16)));

// 32x32x16 bf16 MFMA: D(32x32) += A(32x16) * B(16x32).  Lane l supplies row
// (l % 32) of A and column (l % 32) of B with the eight k values of group
// (l / 32); it receives D[8*(i/4) + 4*(l/32) + i%4][l % 32], i = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef int v8i __attribute__((ext_vector_type(8)));

// 32x32x64 e4m3 x e4m3 MFMA (unit block scales): D(32x32) += A(32x64) *
// B(64x32).  Lane l supplies 32 k values of row (l % 32) of A and of column
// (l % 32) of B; A and B must use the same lane/byte -> k assignment (any
// assignment gives the same sums).  D's layout is that of mfma32.  The
// hardware's sums are not exact fp32 (a probe with random codes agreed with
// the fp64 dot products to about 2^-13 of the sum of the magnitudes).
__device__ __forceinline__ f32x16 mfma32x64_f8(v8i a, v8i b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ void load_lds16(const void* gsrc, void* lds_dst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gsrc,
                                   (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}

__device__ __forceinline__ u32x4 lds_read16(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// Physical 16-byte chunk of a logical chunk in an LDS row of ROWB bytes:
// the 16 rows read by one 16-lane LDS cycle land in 16 different 16-byte
// bank slots (64 banks x 4 bytes).
template <int ROWB>
__device__ __forceinline__ int swz(int row) {
  if constexpr (ROWB == 128) return (row >> 1) & 7;
  else if constexpr (ROWB == 64) return (row >> 2) & 3;
  else return (row >> 3) & 1;  // 32-byte rows
}

// s_waitcnt that waits until at most n vector-memory loads of this wave are
// outstanding (expcnt and lgkmcnt not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Scheduling groups for one sub-step: its NMF MFMAs with NDS fragment reads
// of the next sub-step threaded one after each of the first NDS MFMAs.
// (More reads than MFMAs: the rest follow the last MFMA.)
template <int NDS, int NMF>
__device__ __forceinline__ void sched_substep() {
  constexpr int P = NDS < NMF ? NDS : NMF;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  if constexpr (NMF > P) __builtin_amdgcn_sched_group_barrier(0x008, NMF - P, 0);
  if constexpr (NDS > P) __builtin_amdgcn_sched_group_barrier(0x100, NDS - P, 0);
}

struct TileCoord {
  int tm, tn;
};

// Permutation of [0, n) for workgroup ids: id j runs on XCD j % 8, and the
// ids of one XCD receive a contiguous run of indices.
__device__ __forceinline__ int xcd_fold(int j, int n) {
  const int xcd = j & 7, local = j >> 3;
  const int q = n >> 3, r = n & 7;
  return xcd * q + min(xcd, r) + local;
}

// Tile of linear index L, walked in groups of GROUP_M M-tiles.
__device__ __forceinline__ TileCoord tile_coord(int L, int tiles_m, int tiles_n) {
  const int per_group = GROUP_M * tiles_n;
  const int group = L / per_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int i = L - group * per_group;
  return TileCoord{first_m + i % gsize, i / gsize};
}

// Stream-K tail.  One workgroup fills a CU (LDS), so the tiles run in rounds
// of one per CU, and a last round of rem tiles costs as much as a full one
// while the other CUs idle.  Instead, the first nfull = tiles - rem tiles are
// computed whole (workgroups 0 .. nfull-1) and each of the rem tail tiles is
// cut along K into d pieces of KT / d k-tiles, one workgroup each.  A piece
// stores its raw fp32 sums in its slot of `part`, then counts itself in its
// tile's arrival counter; the piece that arrives last adds the tile's d
// slots in k order (the same sum whichever piece arrives last) and writes the
// tile through the ordinary epilogue.  No workgroup waits for another.
struct SkTail {
  float* part;   // rem * d slots of BM * BN floats, slot = tail tile * d + piece
  int* cnt;      // one arrival counter per tail tile, zero at launch
  int nfull;     // tiles computed whole
  int d;         // pieces per tail tile; 0: no tail split
};

// A tail tile's piece (see SkTail): store this workgroup's raw fp32 sums in
// its slot and count the arrival; the piece that arrives last adds the tile's
// d slots in k order into acc and returns true (it writes the tile), every
// other piece returns false.  NT threads, each holding CB x TB 32x32 blocks;
// `flag` is an int in LDS.
template <int CB, int TB, int NT, int BM, int TBC = TB>
__device__ __forceinline__ bool sk_handoff(f32x16 (&acc)[CB][TB], const SkTail sk, int tail, int piece, int tid,
                                           int* flag) {
  static_assert(TB % TBC == 0, "token blocks per round trip");
  constexpr int SLOT = BM * BN * 4;     // bytes per slot
  static_assert(CB * TB * 16 * NT * 4 == SLOT, "a slot holds the tile");
  constexpr int kDeviceScope = 16;      // buffer cache policy: sc1
  // raw buffer over this tile's d slots (word 3 of a gfx9 buffer descriptor:
  // 32-bit data format, no swizzle); offsets past d * SLOT read zero
  const __amdgpu_buffer_rsrc_t slots = __builtin_amdgcn_make_buffer_rsrc(
      sk.part + (int64_t)tail * sk.d * (BM * BN), 0, sk.d * SLOT, 0x00020000);
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = acc[cb][tb][4 * qd + i];
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), slots,
                                               piece * SLOT + (((cb * TB + tb) * 4 + qd) * NT + tid) * 16, 0,
                                               kDeviceScope);
      }
  // Ordering.  The LLVM AMDGPU memory model's agent-scope release on
  // gfx942/gfx950 is "buffer_wbl2 sc1; s_waitcnt vmcnt(0)" before the
  // atomic, and its acquire "buffer_inv sc1" after it: the write-back pushes
  // out L2 lines that were written without the agent-scope (sc1) policy and
  // the invalidate drops lines that later non-sc1 loads could hit.  Every
  // store and load of the slots here carries sc1 (they go through to the
  // point of coherence shared by the XCDs), so only the s_waitcnt part of the
  // release is needed: vmcnt(0) makes each lane's slot stores complete at
  // agent scope, the workgroup barrier orders all lanes before lane 0's
  // counter increment, and the last piece's slot loads are issued only after
  // the increment's returned value is known (a control dependence through the
  // barrier below).  Dropping the write-back and invalidate keeps the GEMM's
  // L2 panels: a full fence here measured the tail at half speed.
  __builtin_amdgcn_s_waitcnt(0);        // this piece's slot stores are complete
  __syncthreads();
  if (tid == 0) *flag = __hip_atomic_fetch_add(sk.cnt + tail, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (*flag != sk.d - 1) return false;  // another piece writes the tile
  // k-order sum, TBC token blocks of one weight-row block at a time: their
  // 4 TBC f32x4 of a slot are loaded together (one memory round trip per
  // slot and chunk; a smaller TBC needs fewer registers)
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int t0 = 0; t0 < TB; t0 += TBC) {
      f32x4 sum[TBC * 4], v[TBC * 4];
      auto own = [&](f32x4 (&dst)[TBC * 4]) {
#pragma unroll
        for (int tb = 0; tb < TBC; ++tb)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[tb * 4 + qd][i] = acc[cb][t0 + tb][4 * qd + i];
      };
      auto load = [&](int p, f32x4 (&dst)[TBC * 4]) {
#pragma unroll
        for (int tb = 0; tb < TBC; ++tb)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd)
            dst[tb * 4 + qd] = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                           slots, p * SLOT + (((cb * TB + t0 + tb) * 4 + qd) * NT + tid) * 16, 0, kDeviceScope));
      };
      if (piece == 0) own(sum);
      else load(0, sum);
      for (int p = 1; p < sk.d; ++p) {
        if (p == piece) own(v);
        else load(p, v);
#pragma unroll
        for (int e = 0; e < TBC * 4; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i) sum[e][i] += v[e][i];
      }
#pragma unroll
      for (int tb = 0; tb < TBC; ++tb)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[cb][t0 + tb][4 * qd + i] = sum[tb * 4 + qd][i];
    }
  return true;
}

// Epilogue of a wave's CB x TB blocks.  The lane holds, per block, weight
// rows 8j + 4g + (0..3) (j = 0..3) of block cb for token r32 of block tb.
// Gate/up (SWIGLU): blocks 0 .. CB/2-1 are gate rows of channels ch0 +
// 32 cb + ..., blocks CB/2 .. CB-1 the same channels' up rows; A =
// SiLU(G) * U is written in bf16.  Otherwise rows are output features f0 +
// 32 cb + ... (fp32, or bf16 with OBF).  Tokens: tok0 + 32 tb + r32.  One-byte
// weights scale by the row scales s0 (s1: up), fp8 activations by sx.
template <bool SWIGLU, int WB, bool A8, bool OBF, int CB, int TB>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[CB][TB], int M, int N, int ch0, int tok0, int r32, int g,
                                           const float* __restrict__ s0, const float* __restrict__ s1,
                                           const float* __restrict__ sx, void* __restrict__ out, int64_t ld_out) {
  if constexpr (SWIGLU) {
    uint16_t* a_out = reinterpret_cast<uint16_t*>(out);
#pragma unroll
    for (int cb = 0; cb < CB / 2; ++cb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ch = ch0 + cb * 32 + 8 * j + 4 * g;  // channels ch .. ch+3
        if (ch >= N) continue;
        float sgv[4] = {1.f, 1.f, 1.f, 1.f}, suv[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (WB) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sgv[i] = s0[ch + i];
            suv[i] = s1[ch + i];
          }
        }
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          const int tok = tok0 + tb * 32 + r32;
          if (tok >= M) continue;
          const float st = A8 ? sx[tok] : 1.f;
          float a[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float gv = acc[cb][tb][4 * j + i], uv = acc[cb + CB / 2][tb][4 * j + i];
            if constexpr (WB) {
              gv *= sgv[i];
              uv *= suv[i];
            }
            if constexpr (A8) {
              gv *= st;
              uv *= st;
            }
            a[i] = silu(gv) * uv;
          }
          u32x2 packed = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
          *reinterpret_cast<u32x2*>(a_out + (int64_t)tok * ld_out + ch) = packed;
        }
      }
    }
  } else {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int f = ch0 + cb * 32 + 8 * j + 4 * g;  // features f .. f+3
        if (f >= N) continue;
        float sv[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (WB) {
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[i] = s0[f + i];
        }
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          const int tok = tok0 + tb * 32 + r32;
          if (tok >= M) continue;
          f32x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = acc[cb][tb][4 * j + i] * sv[i];
          if constexpr (A8) {
            const float st = sx[tok];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] *= st;
          }
          store_out4<OBF>(out, (int64_t)tok * ld_out + f, v);
        }
      }
    }
  }
}

// Epilogue of the down projection (fp32 or bf16 rows of out) through LDS, for
// waves of 32 CB consecutive features and TB 32-token blocks.  In the MFMA
// layout a lane holds four consecutive features of one token, so a direct
// store instruction writes 32-byte pieces of 32 rows; here each wave writes
// its 32-token x 32 CB-feature block of one token block to LDS, reads it
// back row-wise and stores whole 32 CB-feature row pieces (64 / 2 CB rows
// per instruction, 128 CB bytes each in fp32).  LDS: 32 x (32 CB + 4)
// floats per wave; every wave of the workgroup calls it (block barriers).
// One-byte weights scale by the row scales s0, fp8 activations by sx.
template <int CB>
constexpr int rows_epilogue_lds(int waves) { return waves * 32 * (32 * CB + 4) * 4; }

template <int WB, bool A8, bool OBF, int CB, int TB>
__device__ __forceinline__ void store_tile_rows(const f32x16 (&acc)[CB][TB], int M, int N, int ch0, int tok0,
                                                int lane, int wave, const float* __restrict__ s0,
                                                const float* __restrict__ sx, void* __restrict__ out,
                                                int64_t ld_out, uint8_t* lds) {
  static_assert(CB == 2 || CB == 4, "64 or 128 features per wave");
  constexpr int RP = 32 * CB + 4;             // LDS row pitch in floats
  constexpr int LPR = 8 * CB;                 // lanes per row on the read side
  constexpr int RPI = 64 / LPR;               // rows per store instruction
  float* buf = reinterpret_cast<float*>(lds) + wave * 32 * RP;
  const int r32 = lane & 31, g = lane >> 5;
  const int c = lane % LPR, tr = lane / LPR;  // read side: features 4c .. 4c+3 of token tr + RPI it
  const int f = ch0 + 4 * c;
  float sv[4] = {1.f, 1.f, 1.f, 1.f};
  if constexpr (WB != 0) {
    if (f < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[i] = s0[f + i];
    }
  }
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    asm volatile("" ::: "memory");
    lds_barrier();                            // every wave is done with the buffer (k-loop stages, block tb-1)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 v = {acc[cb][tb][4 * j], acc[cb][tb][4 * j + 1], acc[cb][tb][4 * j + 2], acc[cb][tb][4 * j + 3]};
        *reinterpret_cast<f32x4*>(buf + r32 * RP + cb * 32 + 8 * j + 4 * g) = v;
      }
    asm volatile("" ::: "memory");
    lds_barrier();
#pragma unroll
    for (int it = 0; it < 32 / RPI; ++it) {
      const int t = RPI * it + tr;
      const int tok = tok0 + tb * 32 + t;
      f32x4 v = *reinterpret_cast<const f32x4*>(buf + t * RP + 4 * c);
      if (tok < M && f < N) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] *= sv[i];
        if constexpr (A8) {
          const float st = sx[tok];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] *= st;
        }
        store_out4<OBF>(out, (int64_t)tok * ld_out + f, v);
      }
    }
  }
}

// A8: the activations are e4m3fn codes too (W8A8): one byte per element in
// LDS, 32x32x64 fp8 MFMAs (twice the bf16 rate), and the per-token scales sx
// applied in the epilogue with the weight row scales.
// SK: the launch has a stream-K tail (sk.d > 0).  Launches without one use
// the SK = false instance, which has no tail code: with it, the compiler
// moves all accumulators out of AGPRs ahead of the tail branch and spills,
// which slows every tile's epilogue.
template <bool SWIGLU, int WB, int BK, int NS, int WV, int BM, bool OBF, bool A8, bool SK>
__global__ __launch_bounds__(WV * 64, 1) void gemm_kernel(
    int M, int N, int K, const XRows xr,
    const uint8_t* __restrict__ w0, const uint8_t* __restrict__ w1, int64_t ldw,
    const float* __restrict__ s0, const float* __restrict__ s1, const float* __restrict__ sx,
    void* __restrict__ out, int64_t ld_out, int tiles_m, int tiles_n, const SkTail sk) {
  static_assert(A8 ? (BK == 128 && WB == kWeightE4M3) : (BK == 32 || BK == 64), "stage depth");
  static_assert(WV == 4 || WV == 8, "waves per workgroup");
  using XT = typename std::conditional<A8, uint8_t, uint16_t>::type;
  static_assert(BM == 64 || BM == 128 || BM == 256, "tokens per tile");
  constexpr int WM = BM == 256 ? 2 : 1;        // waves across the tokens
  constexpr int WN = WV / WM;                  // waves across the weight rows
  constexpr int CB = BN / WN / 32;             // 32-row weight blocks per wave
  constexpr int TB = BM / WM / 32;             // 32-token blocks per wave
  static_assert(CB >= 1 && (!SWIGLU || CB % 2 == 0), "weight blocks per wave");
  constexpr int EB = WB ? 1 : 2;              // weight bytes per element
  constexpr int XE = A8 ? 1 : 2;               // activation bytes per element
  constexpr int KSUB = BK / (A8 ? 64 : 16);    // MFMA sub-steps per stage
  constexpr int XROWB = BK * XE;               // bytes per LDS activation row
  constexpr int WROWB = BK * EB;               // bytes per LDS weight row
  constexpr int XBYTES = BM * XROWB;
  constexpr int WBYTES = BN * WROWB;
  constexpr int SBYTES = XBYTES + WBYTES;
  constexpr int XINST = XBYTES / 1024 / WV;    // 1 KB direct loads per wave per stage
  constexpr int WINST = WBYTES / 1024 / WV;
  constexpr int LPS = XINST + WINST;           // loads per wave per stage
  constexpr int TILE_N = SWIGLU ? BN / 2 : BN; // output columns per tile
  constexpr int XRPI = 1024 / XROWB;           // rows per 1 KB load
  constexpr int WRPI = 1024 / WROWB;
  constexpr int XCH = XROWB / 16;              // 16-byte chunks per row
  constexpr int WCH = WROWB / 16;

  // Stages, the L2 touch scratch and the stream-K arrival flag in one LDS
  // object: with a second __shared__ object the compiler no longer tells the
  // direct-to-LDS destinations from the fragment reads and drains the load
  // ring (vmcnt(0)) before every k-tile's reads.
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * SBYTES + WV * 512 + (SK ? 16 : 0)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int r32 = lane & 31, g = lane >> 5;
  const int wm = wave / WN, wn = wave % WN;

  // ---- this workgroup's tile and k-tiles kt0 .. kt1-1: a whole tile, or one
  // piece of a tail tile (tail >= 0; see SkTail)
  const int KT = K / BK;
  const int blk = blockIdx.x;
  int L, kt0 = 0, kt1 = KT, tail = -1, piece = 0;
  if (SK && blk >= sk.nfull) {
    // piece-major: the workgroups running together on an XCD hold the same
    // k-range of neighbouring tiles, which share panels in its L2 as whole
    // tiles do
    const int rem = tiles_m * tiles_n - sk.nfull;
    const int j = xcd_fold(blk - sk.nfull, rem * sk.d);
    piece = j / rem;
    tail = j - piece * rem;
    kt0 = (int)((int64_t)piece * KT / sk.d);
    kt1 = (int)((int64_t)(piece + 1) * KT / sk.d);
    L = sk.nfull + tail;
  } else {
    L = xcd_fold(blk, SK ? sk.nfull : tiles_m * tiles_n);
  }
  const TileCoord tc = tile_coord(L, tiles_m, tiles_n);
  const int m0 = tc.tm * BM;
  const int n0 = tc.tn * TILE_N;

  // ---- direct-to-LDS sources: instruction i of this wave fills LDS bytes
  // [(wave*INST + i) KB, +1 KB) of a stage; lane l fills 16 bytes of it.
  const uint8_t* xsrc[XINST];
#pragma unroll
  for (int i = 0; i < XINST; ++i) {
    const int row = (wave * XINST + i) * XRPI + lane / XCH;
    const int c = (lane % XCH) ^ swz<XROWB>(row);
    const int tok = min(m0 + row, M - 1);
    xsrc[i] = reinterpret_cast<const uint8_t*>(x_row<XT>(xr, tok)) + c * 16;
  }
  const uint8_t* wsrc[WINST];
#pragma unroll
  for (int i = 0; i < WINST; ++i) {
    const int row = (wave * WINST + i) * WRPI + lane / WCH;
    const int c = (lane % WCH) ^ swz<WROWB>(row);
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
  // L2 warm-up one k-tile ahead of the direct loads: each thread touches the
  // 128-byte line of one activation row and one weight row of k-tile kt with a
  // 4-byte direct-to-LDS load into a scratch area nobody reads (no VGPR is
  // written, so nothing waits on it).  The misses of a k-tile are then in
  // flight one k-tile before its own loads, which find the lines in L2.
  // (with 8 waves the upper 256 threads touch the same lines again)
  const int trow = tid & 255;
  const uint8_t* tx = reinterpret_cast<const uint8_t*>(x_row<XT>(xr, min(m0 + (tid & (BM - 1)), M - 1)));
  const uint8_t* tw;
  if constexpr (SWIGLU)
    tw = (trow < BN / 2 ? w0 : w1) + (int64_t)min(n0 + (trow & (BN / 2 - 1)), N - 1) * ldw * EB;
  else
    tw = w0 + (int64_t)min(n0 + trow, N - 1) * ldw * EB;
  uint8_t* tdst = lds + NS * SBYTES + wave * 512;
  auto touch_stage = [&](int kt) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(tx + (int64_t)kt * BK * XE),
                                     (__attribute__((address_space(3))) void*)tdst, 4, 0, 0);
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(tw + (int64_t)kt * BK * EB),
                                     (__attribute__((address_space(3))) void*)(tdst + 256), 4, 0, 0);
  };
  auto issue_stage = [&](int kt, int buf) {
    uint8_t* xdst = lds + buf * SBYTES + wave * XINST * 1024;
    uint8_t* wdst = lds + buf * SBYTES + XBYTES + wave * WINST * 1024;
#pragma unroll
    for (int i = 0; i < XINST; ++i) load_lds16(xsrc[i] + (int64_t)kt * BK * XE, xdst + i * 1024);
#pragma unroll
    for (int i = 0; i < WINST; ++i) load_lds16(wsrc[i] + (int64_t)kt * BK * EB, wdst + i * 1024);
  };
  // ---- fragment rows of this lane inside a stage.  Gate/up: the wave's
  // first CB/2 weight blocks are gate rows of its channels, the last CB/2 the
  // same channels' up rows.
  int wrow[CB], xrow[TB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    if constexpr (SWIGLU)
      wrow[cb] = (cb < CB / 2 ? 0 : BN / 2) + wn * (BN / 2 / WN) + (cb % (CB / 2)) * 32 + r32;
    else
      wrow[cb] = wn * (BN / WN) + cb * 32 + r32;
  }
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) xrow[tb] = wm * (BM / WM) + tb * 32 + r32;

  f32x16 acc[CB][TB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[cb][tb][i] = 0.f;

  // Fragments of sub-step kk (16 k) of a stage.  bf16: lane group g holds
  // chunk 2kk+g of both operands.  fp8: at even kk the weight lane reads
  // 16-byte chunk kk+g (16 codes) once; its low 8 codes serve sub-step kk and
  // its high 8 codes sub-step kk+1, so the activation chunk of 8 elements is
  // 4*(kk/2) + 2g + kk%2.
  u32x4 wq[CB];
  auto read_w = [&](const uint8_t* sw, int kk, int cb, bf16x8 (&wf)[CB]) {
    const int r = wrow[cb];
    if constexpr (WB) {
      if ((kk & 1) == 0) {
        wq[cb] = lds_read16(sw + r * WROWB + (((kk + g) ^ swz<WROWB>(r)) * 16));
        wf[cb] = byte8_to_bf16x8<WB>(wq[cb][0], wq[cb][1]);
      } else {
        wf[cb] = byte8_to_bf16x8<WB>(wq[cb][2], wq[cb][3]);
      }
    } else {
      const int ch = 2 * kk + g;
      wf[cb] = as_bf16x8(lds_read16(sw + r * WROWB + ((ch ^ swz<WROWB>(r)) * 16)));
    }
  };
  auto read_x = [&](const uint8_t* sx, int kk, int tb, bf16x8 (&xf)[TB]) {
    const int r = xrow[tb];
    const int ch = WB ? (4 * (kk >> 1) + 2 * g + (kk & 1)) : (2 * kk + g);
    xf[tb] = as_bf16x8(lds_read16(sx + r * XROWB + ((ch ^ swz<XROWB>(r)) * 16)));
  };
  // Read order = order of first use by the sub-step's MFMAs (cb-major):
  // w0, all x, then the other w.
  auto read_frags = [&](const uint8_t* sx, const uint8_t* sw, int kk, bf16x8 (&wf)[CB], bf16x8 (&xf)[TB]) {
    read_w(sw, kk, 0, wf);
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) read_x(sx, kk, tb, xf);
#pragma unroll
    for (int cb = 1; cb < CB; ++cb) read_w(sw, kk, cb, wf);
  };

  // Main loop, one barrier per k-tile.  Stages 0 .. NS-2 are issued up front;
  // iteration kt waits for stage kt (allowing the NS-2 younger stages to stay
  // in flight), meets the other waves at the barrier (after which stage kt-1's
  // buffer is free), issues stage kt+NS-1 into it and runs its MFMAs.  Past
  // the last k-tile the issue re-loads the last k-tile into the free buffer,
  // so the body stays one basic block with a fixed load count; the
  // scheduling groups thread the fragment reads of sub-step 1 between the
  // MFMAs of sub-step 0.
  {
  #pragma unroll
    for (int s = 0; s < NS - 1; ++s) {
      issue_stage(min(kt0 + s, kt1 - 1), s);
      touch_stage(min(kt0 + s + 1, kt1 - 1));
    }
    int buf = 0;
    for (int kt = kt0; kt < kt1; ++kt) {
      // this wave's loads of stage kt have landed (younger: the touch issued
      // with them and NS-2 later iterations' loads + touches)
      wait_vmcnt<2 + (NS - 2) * (LPS + 2)>();
      lds_barrier();                  // ... and every wave's; stage kt-1 is no longer read
      const int nbuf = buf == 0 ? NS - 1 : buf - 1;   // (kt + NS - 1) % NS
      issue_stage(min(kt + NS - 1, kt1 - 1), nbuf);
      touch_stage(min(kt + NS, kt1 - 1));
      const uint8_t* sx = lds + buf * SBYTES;
      const uint8_t* sw = sx + XBYTES;
      if constexpr (A8) {
        // 64 k per MFMA: lane group g takes bytes [32g, 32g+32) of the
        // sub-step's 64 k of its weight row and of its token row (the same k
        // order on both sides is all the dot product needs)
        v8i wf[2][CB], xf[2][TB];
        auto read8 = [&](const uint8_t* base, int rowb_sel, int r, int kk) {
          const int c0 = 4 * kk + 2 * g;
          u32x4 lo, hi;
          if (rowb_sel == 0) {
            lo = lds_read16(base + r * XROWB + ((c0 ^ swz<XROWB>(r)) * 16));
            hi = lds_read16(base + r * XROWB + (((c0 + 1) ^ swz<XROWB>(r)) * 16));
          } else {
            lo = lds_read16(base + r * WROWB + ((c0 ^ swz<WROWB>(r)) * 16));
            hi = lds_read16(base + r * WROWB + (((c0 + 1) ^ swz<WROWB>(r)) * 16));
          }
          return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        };
        auto frags8 = [&](int kk, v8i (&w_)[CB], v8i (&x_)[TB]) {
          w_[0] = read8(sw, 1, wrow[0], kk);
  #pragma unroll
          for (int tb = 0; tb < TB; ++tb) x_[tb] = read8(sx, 0, xrow[tb], kk);
  #pragma unroll
          for (int cb = 1; cb < CB; ++cb) w_[cb] = read8(sw, 1, wrow[cb], kk);
        };
        frags8(0, wf[0], xf[0]);
  #pragma unroll
        for (int kk = 0; kk < KSUB; ++kk) {
          if (kk + 1 < KSUB) frags8(kk + 1, wf[(kk + 1) & 1], xf[(kk + 1) & 1]);
  #pragma unroll
          for (int cb = 0; cb < CB; ++cb)
  #pragma unroll
            for (int tb = 0; tb < TB; ++tb) acc[cb][tb] = mfma32x64_f8(wf[kk & 1][cb], xf[kk & 1][tb], acc[cb][tb]);
        }
        constexpr int NMF = CB * TB, NRD = 2 * (CB + TB);
        __builtin_amdgcn_sched_group_barrier(0x020, LPS + 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
        sched_substep<NRD, NMF>();
        __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
      } else {
      bf16x8 wf[2][CB], xf[2][TB];
      read_frags(sx, sw, 0, wf[0], xf[0]);
  #pragma unroll
      for (int kk = 0; kk < KSUB; ++kk) {
        if (kk + 1 < KSUB) read_frags(sx, sw, kk + 1, wf[(kk + 1) & 1], xf[(kk + 1) & 1]);
  #pragma unroll
        for (int cb = 0; cb < CB; ++cb)
  #pragma unroll
          for (int tb = 0; tb < TB; ++tb) acc[cb][tb] = mfma32(wf[kk & 1][cb], xf[kk & 1][tb], acc[cb][tb]);
      }
      // scheduling: direct loads of stage kt+NS-1, fragments of sub-step 0,
      // then each sub-step's MFMAs with the next sub-step's reads threaded in
      // (fp8 odd sub-steps read activations only)
      constexpr int NMF = CB * TB, NRD = CB + TB, NRX = WB ? TB : CB + TB;
      __builtin_amdgcn_sched_group_barrier(0x020, LPS + 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
      sched_substep<NRX, NMF>();
      if constexpr (KSUB == 4) {
        sched_substep<NRD, NMF>();
        sched_substep<NRX, NMF>();
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
      }
      buf = buf == NS - 1 ? 0 : buf + 1;
    }
}
  __builtin_amdgcn_s_waitcnt(0);  // no direct load is left in flight at exit

  // ---- a piece of a tail tile: publish the raw sums; the last piece to
  // arrive adds the tile's pieces in k order and writes the tile
  if constexpr (SK) {
    if (tail >= 0 &&
        !sk_handoff<CB, TB, WV * 64, BM>(acc, sk, tail, piece, tid, reinterpret_cast<int*>(lds + NS * SBYTES + WV * 512)))
      return;
  }
  if constexpr (!SWIGLU && rows_epilogue_lds<CB>(WV) <= NS * SBYTES) {
    store_tile_rows<WB, A8, OBF, CB, TB>(acc, M, N, n0 + wn * (BN / WN), m0 + wm * (BM / WM), lane, wave, s0, sx, out,
                                         ld_out, lds);
  } else {
    store_tile<SWIGLU, WB, A8, OBF, CB, TB>(acc, M, N, n0 + (SWIGLU ? wn * (BN / 2 / WN) : wn * (BN / WN)),
                                            m0 + wm * (BM / WM), r32, g, s0, s1, sx, out, ld_out);
  }
}

// ---------------------------------------------------------------------------
// Ping-pong GEMM: bf16 weights and activations, 256 x 256 tiles, eight waves.
//
// What bounds the four-wave kernel above, measured on MI355X: a CU moves
// global memory into LDS at about 35 bytes per clock for this access pattern
// (rows of 128 bytes), which a 64-k stage of a 256 x 256 tile (64 KB) needs
// about 1800 clocks for, close to the 2048 clocks its MFMAs take; and a wave
// that issues direct-to-LDS loads stalls on them at that rate, issuing no
// MFMAs meanwhile.  With one wave per SIMD the loads and the MFMAs therefore
// take turns instead of overlapping.
//
// Here two waves share each SIMD, in two groups of four (A: waves 0-3, B:
// 4-7; a workgroup's waves go to the SIMDs in turn, so each SIMD holds one of
// each).  Each wave alternates a compute phase (the 32 MFMAs of one 64-k
// stage, with that stage's fragment reads from LDS threaded between them)
// and a load phase (issue 8 KB of direct-to-LDS loads), and the groups are
// one phase apart, so on every SIMD one wave issues MFMAs while the other
// waits on its loads, and the loads stream continuously.  Workgroup barriers
// (all eight waves) separate the phases; compute phases run at raised wave
// priority (s_setprio).
//
// Output split: wave q of a group (q = wave % 4) owns 64 weight rows (in a
// gate/up tile: the gate rows of 32 channels and the same channels' up rows)
// and its group's 128 tokens (A: tokens 0-127 of the tile, B: 128-255), 2 x 4
// blocks of 32 x 32 (128 fp32 accumulators per lane).
//
// LDS: a ring of five half-stages of 32 KB (160 KB): the activation half X_s
// (256 token rows x 64 k) of stage s sits in buffer 2s mod 5, its weight half
// W_s in buffer 2s+1 mod 5.  Group A loads the X halves, group B the W
// halves.  In phase slots between barriers (slot 0 = the prologue):
//   slot 2s+1: A computes stage s,  B loads W_{s+1};
//   slot 2s+2: B computes stage s,  A loads X_{s+2}.
// A half-stage's buffer was freed at least one slot before its loads are
// issued, X_s has two slots after its load slot to land and W_s one; each
// wave waits for its own loads (vmcnt) before the barrier after which they
// are read.
template <bool SWIGLU, bool OBF, bool SK, bool A8>
__global__ __launch_bounds__(512, 1) void gemm_pp_kernel(int M, int N, int K, const XRows xr,
                                                         const uint8_t* __restrict__ w0,
                                                         const uint8_t* __restrict__ w1, int64_t ldw,
                                                         const float* __restrict__ s0,
                                                         const float* __restrict__ s1,
                                                         const float* __restrict__ sx,
                                                         void* __restrict__ out, int64_t ld_out, int tiles_m,
                                                         int tiles_n, const SkTail sk) {
  // A8: e4m3fn activations and weights (one byte each, row scales s0 / s1,
  // token scales sx): a stage holds 128 k in the same 128-byte rows, and
  // each 64-k sub-step is one 32x32x64 fp8 MFMA per block pair
  constexpr int BM = 256, BK = A8 ? 128 : 64, WV = 8;
  constexpr int EB = A8 ? 1 : 2;              // bytes per element
  constexpr int WBF = A8 ? kWeightE4M3 : kWeightWide;
  constexpr int CB = 2, TB = 4;               // 32-row weight blocks, 32-token blocks per wave
  constexpr int ROWB = BK * EB;               // bytes per LDS row
  constexpr int HALF = 256 * ROWB;            // one half-stage: 256 rows
  constexpr int NH = 5;                       // half-stages in the ring
  constexpr int LPH = HALF / 1024 / 4;        // 1 KB loads per wave per half-stage
  constexpr int RPI = 1024 / ROWB;            // rows per 1 KB load
  constexpr int CH = ROWB / 16;               // 16-byte chunks per row
  constexpr int KSUB = BK / (A8 ? 64 : 16);   // MFMA sub-steps per stage
  constexpr int TILE_N = SWIGLU ? BN / 2 : BN;
  static_assert(NH * HALF <= 160 * 1024, "LDS");
  // One LDS object (the stream-K flag reuses its first bytes once the ring
  // has drained).
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NH * HALF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool grpB = wave >= 4;
  const int q = wave & 3;
  const int r32 = lane & 31, g = lane >> 5;

  // ---- tile and k-range (as gemm_kernel)
  const int KT = K / BK;
  const int blk = blockIdx.x;
  int L, kt0 = 0, kt1 = KT, tail = -1, piece = 0;
  if (SK && blk >= sk.nfull) {
    const int rem = tiles_m * tiles_n - sk.nfull;
    const int j = xcd_fold(blk - sk.nfull, rem * sk.d);
    piece = j / rem;
    tail = j - piece * rem;
    kt0 = (int)((int64_t)piece * KT / sk.d);
    kt1 = (int)((int64_t)(piece + 1) * KT / sk.d);
    L = sk.nfull + tail;
  } else {
    L = xcd_fold(blk, SK ? sk.nfull : tiles_m * tiles_n);
  }
  const TileCoord tc = tile_coord(L, tiles_m, tiles_n);
  const int m0 = tc.tm * BM;
  const int n0 = tc.tn * TILE_N;

  // ---- this wave's loads: rows q*64 + 8i + lane/8 of its group's half
  // (A: token rows of X, B: weight rows), 128 bytes each, chunk-swizzled
  const uint8_t* src[LPH];
#pragma unroll
  for (int i = 0; i < LPH; ++i) {
    const int row = q * (256 / 4) + i * RPI + lane / CH;
    const int c = (lane % CH) ^ swz<ROWB>(row);
    if (!grpB) {
      src[i] = A8 ? x_row<uint8_t>(xr, min(m0 + row, M - 1)) + c * 16
                  : reinterpret_cast<const uint8_t*>(x_row<uint16_t>(xr, min(m0 + row, M - 1))) + c * 16;
    } else {
      int ch;
      const uint8_t* base;
      if constexpr (SWIGLU) {
        ch = n0 + (row & (BN / 2 - 1));
        base = row < BN / 2 ? w0 : w1;
      } else {
        ch = n0 + row;
        base = w0;
      }
      src[i] = base + (int64_t)min(ch, N - 1) * ldw * EB + c * 16;
    }
  }
  // half-stage of stage kt (clamped to the k-range: past its end the last
  // stage is loaded again, so every load phase issues the same count) into
  // ring buffer `hb`
  auto load_half = [&](int kt, int hb) {
    kt = min(kt, kt1 - 1);
    uint8_t* dst = lds + hb * HALF + q * (HALF / 4);
#pragma unroll
    for (int i = 0; i < LPH; ++i) load_lds16(src[i] + (int64_t)kt * ROWB, dst + i * 1024);
  };

  // ---- fragment rows
  int wrow[CB], xrow[TB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) wrow[cb] = SWIGLU ? cb * (BN / 2) + q * 32 + r32 : q * 64 + cb * 32 + r32;
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) xrow[tb] = (grpB ? 128 : 0) + tb * 32 + r32;

  f32x16 acc[CB][TB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[cb][tb][i] = 0.f;

  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // compute phase of stage kt (ring position s = kt - kt0): fragment reads of
  // sub-step kk+1 threaded between the MFMAs of sub-step kk
  auto compute = [&](int s) {
    const uint8_t* sx = lds + ((2 * s) % NH) * HALF;
    const uint8_t* sw = lds + ((2 * s + 1) % NH) * HALF;
    if constexpr (A8) {
      // lane group g takes bytes [32g, 32g + 32) of the sub-step's 64 k of its
      // weight row and of its token row (chunks 4kk + 2g, +1)
      v8i wf[2][CB], xf[2][TB];
      auto read8 = [&](const uint8_t* base, int r, int kk) {
        const int c0 = 4 * kk + 2 * g;
        const u32x4 lo = lds_read16(base + r * ROWB + ((c0 ^ swz<ROWB>(r)) * 16));
        const u32x4 hi = lds_read16(base + r * ROWB + (((c0 + 1) ^ swz<ROWB>(r)) * 16));
        return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      };
      auto read = [&](int kk, v8i (&w_)[CB], v8i (&x_)[TB]) {
        w_[0] = read8(sw, wrow[0], kk);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) x_[tb] = read8(sx, xrow[tb], kk);
#pragma unroll
        for (int cb = 1; cb < CB; ++cb) w_[cb] = read8(sw, wrow[cb], kk);
      };
      __builtin_amdgcn_s_setprio(1);
      read(0, wf[0], xf[0]);
#pragma unroll
      for (int kk = 0; kk < KSUB; ++kk) {
        if (kk + 1 < KSUB) read(kk + 1, wf[(kk + 1) & 1], xf[(kk + 1) & 1]);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) acc[cb][tb] = mfma32x64_f8(wf[kk & 1][cb], xf[kk & 1][tb], acc[cb][tb]);
      }
      constexpr int NMF = CB * TB, NRD = 2 * (CB + TB);
      __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
      sched_substep<NRD, NMF>();
      __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
      __builtin_amdgcn_s_setprio(0);
    } else {
      bf16x8 wf[2][CB], xf[2][TB];
      auto read = [&](int kk, bf16x8 (&w_)[CB], bf16x8 (&x_)[TB]) {
        const int c = 2 * kk + g;
        w_[0] = as_bf16x8(lds_read16(sw + wrow[0] * ROWB + ((c ^ swz<ROWB>(wrow[0])) * 16)));
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
          x_[tb] = as_bf16x8(lds_read16(sx + xrow[tb] * ROWB + ((c ^ swz<ROWB>(xrow[tb])) * 16)));
#pragma unroll
        for (int cb = 1; cb < CB; ++cb)
          w_[cb] = as_bf16x8(lds_read16(sw + wrow[cb] * ROWB + ((c ^ swz<ROWB>(wrow[cb])) * 16)));
      };
      __builtin_amdgcn_s_setprio(1);
      read(0, wf[0], xf[0]);
#pragma unroll
      for (int kk = 0; kk < KSUB; ++kk) {
        if (kk + 1 < KSUB) read(kk + 1, wf[(kk + 1) & 1], xf[(kk + 1) & 1]);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) acc[cb][tb] = mfma32(wf[kk & 1][cb], xf[kk & 1][tb], acc[cb][tb]);
      }
      // reads of sub-step 0, then per sub-step its MFMAs with the next
      // sub-step's reads threaded one after each of the first MFMAs
      constexpr int NMF = CB * TB, NRD = CB + TB;
      __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
      sched_substep<NRD, NMF>();
      sched_substep<NRD, NMF>();
      sched_substep<NRD, NMF>();
      __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
      __builtin_amdgcn_s_setprio(0);
    }
  };

  // ---- prologue (slot 0): A loads X_0 and X_1, B loads W_0
  if (!grpB) {
    load_half(kt0, 0);
    load_half(kt0 + 1, 2);
    wait_vmcnt<LPH>();
  } else {
    load_half(kt0, 1);
    wait_vmcnt<0>();
  }
  barrier();

  // slots 1 .. 2S: A computes in the odd ones, B in the even ones
  const int S = kt1 - kt0;
  for (int j = 1; j <= 2 * S; ++j) {
    if (((j & 1) != 0) != grpB) {
      compute(grpB ? j / 2 - 1 : j / 2);       // stage s: slot 2s+1 (A), 2s+2 (B)
      if (grpB) wait_vmcnt<0>();                // B: its W_{s+1} has landed
    } else {
      // A, slot 2s+2: X_{s+2} into buffer 2s+4; B, slot 2s+1: W_{s+1} into 2s+3
      const int s = grpB ? j / 2 : j / 2 - 1;
      load_half(kt0 + s + (grpB ? 1 : 2), (2 * s + (grpB ? 3 : 4)) % NH);
      if (!grpB) wait_vmcnt<LPH>();             // A: its X_{s+1} has landed
    }
    barrier();
  }
  __builtin_amdgcn_s_waitcnt(0);  // no direct load is left in flight at exit

  if constexpr (SK) {
    if (tail >= 0 && !sk_handoff<CB, TB, WV * 64, BM>(acc, sk, tail, piece, tid, reinterpret_cast<int*>(lds)))
      return;
  }
  if constexpr (SWIGLU) {
    store_tile<true, WBF, A8, OBF, CB, TB>(acc, M, N, n0 + q * 32, m0 + (grpB ? 128 : 0), r32, g, s0, s1, sx, out,
                                           ld_out);
  } else {
    static_assert(rows_epilogue_lds<CB>(8) <= NH * HALF, "LDS of the row-wise epilogue");
    store_tile_rows<WBF, A8, OBF, CB, TB>(acc, M, N, n0 + q * 64, m0 + (grpB ? 128 : 0), lane, wave, s0, sx, out,
                                          ld_out, lds);
  }
}

// Packed-weight GEMM (bf16 weights in the packed decode layout, bf16
// activations, 256 x 256 tiles).  The packed array stores each 16-row block
// of W as its run of 1 KB fragments, fragment f giving the 16 bytes at
// 16 * L to lane L: row L % 16, k values 32 f + 8 (L / 16) + (0..7).  Two
// consecutive blocks b, b + 1 then form the A operand of two 32x32x16 MFMAs
// per fragment directly: for MFMA h (k values 32 f + 16 h + (0..15)), lane l
// takes row l % 32 (block b + (l / 16) % 2, row l % 16) with k group l / 32,
// i.e. the 16 bytes at 256 (2 h + l / 32) + 16 (l % 16) of that block's
// fragment, and one 16-byte load per lane fetches two 512-byte contiguous
// pieces.  The k order is the one the LDS-staged kernels use (chunk 2 kk + g
// of a 64-k stage), so the activation side is unchanged.
//
// So the weights go from memory straight into registers, each wave loading
// the fragments of its own 64 rows one stage ahead (64 VGPRs, two sets), and
// only the activations pass through LDS: a ring of four 32 KB stages filled
// by direct-to-LDS loads three stages ahead.  Per 64-k stage the LDS moves
// 32 KB of writes and 128 KB of fragment reads (the two-operand kernels: 64 KB
// and 192 KB).
//
// Eight waves, two per SIMD: wave q of group G (q = wave % 4, G = wave / 4)
// owns the tile's blocks 4q .. 4q + 3 (64 weight rows) and tokens 128 G ..
// 128 G + 127, 2 x 4 blocks of 32 x 32 (128 fp32 accumulators per lane).
// Gate/up blocks hold 8 channels' gate rows then their up rows, so in a
// 32-row MFMA block the lane's registers 0-3 / 4-7 are the gate / up sums of
// channels 8 b + 4 g + (0..3) and registers 8-11 / 12-15 those of block b + 1,
// and SiLU(G) * U needs no exchange between lanes.
// One-byte weights (WB: e4m3fn or int8 codes, packed the same way with 64
// k-values per row in a fragment, 16 rows x 64 bytes): lane l loads the
// chunks 2g and 2g + 1 of its row (g = l / 32), 16 codes each, which
// widened to bf16 (exact) give MFMA kk the codes 8 (kk mod 2) .. +7 of chunk
// 2g + kk / 2, i.e. k values 16 (2g + kk / 2) + 8 (kk mod 2) + (0..7) of the
// 64-k stage; the activation side reads the same k values (LDS chunk
// 4g + kk instead of 2kk + g).  Any k assignment shared by both operands
// gives the same products; the row scales multiply the fp32 sums in the
// epilogue, as in the other kernels.
// (wp is deliberately not __restrict__: with it the compiler moved the
// weight loads across the memory-clobbering asm statements that fix their
// place in the schedule.)
template <bool SWIGLU, int WB, bool OBF, bool SK>
__global__ __launch_bounds__(512, 1) void gemm_pk_kernel(int M, int N, int K, const uint8_t* __restrict__ xb,
                                                         int64_t ldx, const uint8_t* wp, int nblk,
                                                         const float* __restrict__ s0,
                                                         const float* __restrict__ s1,
                                                         void* __restrict__ out, int64_t ld_out, int tiles_m,
                                                         int tiles_n, const SkTail sk) {
  constexpr int BM = 256, BK = 64;
  constexpr int CB = 2, TB = 4;               // 32-row weight blocks, 32-token blocks per wave
  constexpr int ROWB = BK * 2;                // bytes per LDS row
  constexpr int STAGE = BM * ROWB;            // 32 KB of activations per stage
  constexpr int NS = 4;                       // stages in the ring (five measured slower)
  constexpr int KSUB = BK / 16;               // MFMA k-steps per stage
  constexpr int BPT = 16;                     // 16-row blocks per tile
  static_assert(NS * STAGE <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int q = wave & 3;
  const int r32 = lane & 31, g = lane >> 5;

  // ---- tile and k-range (as gemm_pp_kernel)
  const int KT = K / BK;
  const int blk = blockIdx.x;
  int L, kt0 = 0, kt1 = KT, tail = -1, piece = 0;
  if (SK && blk >= sk.nfull) {
    const int rem = tiles_m * tiles_n - sk.nfull;
    const int j = xcd_fold(blk - sk.nfull, rem * sk.d);
    piece = j / rem;
    tail = j - piece * rem;
    kt0 = (int)((int64_t)piece * KT / sk.d);
    kt1 = (int)((int64_t)(piece + 1) * KT / sk.d);
    L = sk.nfull + tail;
  } else {
    L = xcd_fold(blk, SK ? sk.nfull : tiles_m * tiles_n);
  }
  const TileCoord tc = tile_coord(L, tiles_m, tiles_n);
  const int m0 = tc.tm * BM;
  const int b0 = tc.tn * BPT;

  // ---- activation loads: this wave's 32 token rows of a stage, four 1 KB
  // direct loads of 8 rows x 128 bytes, chunk-swizzled
  const uint8_t* xsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wave * 32 + i * 8 + lane / 8;
    const int c = (lane % 8) ^ swz<ROWB>(row);
    xsrc[i] = xb + (int64_t)min(m0 + row, M - 1) * ldx * 2 + c * 16;
  }
  // stage kt (clamped to the k-range: every iteration issues the same loads)
  auto load_x = [&](int kt, int buf) {
    kt = min(kt, kt1 - 1);
    uint8_t* dst = lds + buf * STAGE + wave * 4096;
#pragma unroll
    for (int i = 0; i < 4; ++i) load_lds16(xsrc[i] + (int64_t)kt * ROWB, dst + i * 1024);
  };

  // ---- weight fragments: block pair (4q + 2cb, +1) of the tile; blocks past
  // the end read the last block (their outputs are not stored)
  const int64_t fpb = K / (WB ? 64 : 32);     // fragments per block
  const uint8_t* wsrc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int b = min(b0 + 4 * q + 2 * cb + ((lane >> 4) & 1), nblk - 1);
    wsrc[cb] = wp + (int64_t)b * fpb * 1024 + (WB ? 512 : 256) * g + 16 * (lane & 15);
  }
  // 16-byte weight load i (bf16: k-step i; one-byte: chunk 2g + i, i < 2) of
  // MFMA block cb at stage kt
  constexpr int WL = WB ? 2 : KSUB;           // loads per block and stage
  auto load_w = [&](int kt, int cb, int i, u32x4& w) {
    kt = min(kt, kt1 - 1);
    if constexpr (WB)
      w = *reinterpret_cast<const u32x4*>(wsrc[cb] + (int64_t)kt * 1024 + 256 * i);
    else
      w = *reinterpret_cast<const u32x4*>(wsrc[cb] + ((int64_t)kt * 2 + (i >> 1)) * 1024 + 512 * (i & 1));
  };
  // bf16 A operand of k-step kk from the stage's loads
  auto wfrag = [&](const u32x4 (&w)[WL], int kk) -> bf16x8 {
    if constexpr (WB) {
      const u32x4 v = w[kk >> 1];
      return (kk & 1) ? byte8_to_bf16x8<WB>(v[2], v[3]) : byte8_to_bf16x8<WB>(v[0], v[1]);
    } else {
      return as_bf16x8(w[kk]);
    }
  };

  int xrow[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) xrow[tb] = grp * 128 + tb * 32 + r32;

  f32x16 acc[CB][TB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[cb][tb][i] = 0.f;

  // Order of the loads.  The wave holds two sets of weight registers (2 x
  // 32 VGPRs; one-byte weights 2 x 16).  Iteration s (stage kt0 + s): issue
  // the weights of stage s + 1 into the set last read by the MFMAs of stage
  // s - 1 (NWL = eight loads, one-byte weights four); wait
  // until the weights of stage s have arrived, and with them (issued
  // earlier) this wave's activation loads of stage s; barrier (every wave's
  // activations of stage s have landed and every wave is done with stage
  // s - 1); issue the activations of stage s + 3 into the buffer of stage
  // s - 1 (four loads); compute stage s.  So the weights have one stage to
  // arrive and the activations three.  Loads issued after the weights of
  // stage s at the wait: NWL at s = 0 (W1), else NWL + 4 (X of s + 2, W of
  // s + 1).
  // The wait is explicit because the direct-to-LDS loads are FLAT
  // instructions, after which a wait that the compiler inserts itself for a
  // register is widened to vmcnt(0) (it would also drain the prefetch); the
  // empty asm statements with a memory clobber keep the compiler from moving
  // the weight loads next to their first use.  Stage counts are even for
  // whole tiles (K is a multiple of 128); a stream-K piece may end with one
  // odd stage.
  typedef u32x4 WSet[CB][WL];
  auto load_ws = [&](int kt, WSet& w) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int i = 0; i < WL; ++i) load_w(kt, cb, i, w[cb][i]);
  };
  auto compute = [&](int s, const WSet& w) {
    const uint8_t* sx = lds + (s % NS) * STAGE;
    bf16x8 xf[2][TB];
    auto read = [&](int kk, bf16x8 (&x_)[TB]) {
      const int c = WB ? 4 * g + kk : 2 * kk + g;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
        x_[tb] = as_bf16x8(lds_read16(sx + xrow[tb] * ROWB + ((c ^ swz<ROWB>(xrow[tb])) * 16)));
    };
    read(0, xf[0]);
#pragma unroll
    for (int kk = 0; kk < KSUB; ++kk) {
      if (kk + 1 < KSUB) read(kk + 1, xf[(kk + 1) & 1]);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const bf16x8 a = wfrag(w[cb], kk);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[cb][tb] = mfma32(a, xf[kk & 1][tb], acc[cb][tb]);
      }
    }
    constexpr int NMF = CB * TB;
    __builtin_amdgcn_sched_group_barrier(0x100, TB, 0);
    sched_substep<TB, NMF>();
    sched_substep<TB, NMF>();
    sched_substep<TB, NMF>();
    __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
  };
  const int S = kt1 - kt0;
  WSet wa, wb;
#pragma unroll
  for (int i = 0; i < NS - 1; ++i) load_x(kt0 + i, i);
  load_ws(kt0, wa);
  asm volatile("" ::: "memory");
  constexpr int NWL = CB * WL;                // weight loads per stage (8; one-byte weights 4)
  auto iter = [&](int s, const WSet& cur, WSet& nxt) {
    load_ws(kt0 + s + 1, nxt);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (s == 0) wait_vmcnt<NWL>();
    else wait_vmcnt<NWL + 4>();
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    load_x(kt0 + s + NS - 1, (s + NS - 1) % NS);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    compute(s, cur);
  };
  int s = 0;
  for (; s + 1 < S; s += 2) {
    iter(s, wa, wb);
    iter(s + 1, wb, wa);
  }
  if (s < S) iter(s, wa, wb);
  __builtin_amdgcn_s_waitcnt(0);  // no load is left in flight at exit

  if constexpr (SK) {
    if (tail >= 0 && !sk_handoff<CB, TB, 512, BM, 1>(acc, sk, tail, piece, tid, reinterpret_cast<int*>(lds)))
      return;
  }
  const int tok0 = m0 + grp * 128;
  if constexpr (SWIGLU) {
    uint16_t* a_out = reinterpret_cast<uint16_t*>(out);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int ch = (b0 + 4 * q + 2 * cb + hb) * 8 + 4 * g;  // channels ch .. ch+3
        if (ch >= N) continue;
        float sg[4] = {1.f, 1.f, 1.f, 1.f}, su[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (WB) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sg[i] = s0[ch + i];
            su[i] = s1[ch + i];
          }
        }
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          const int tok = tok0 + tb * 32 + r32;
          if (tok >= M) continue;
          float a[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            a[i] = silu(acc[cb][tb][8 * hb + i] * sg[i]) * (acc[cb][tb][8 * hb + 4 + i] * su[i]);
          const u32x2 pk = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
          *reinterpret_cast<u32x2*>(a_out + (int64_t)tok * ld_out + ch) = pk;
        }
      }
  } else {
    static_assert(rows_epilogue_lds<CB>(8) <= NS * STAGE, "LDS of the row-wise epilogue");
    store_tile_rows<WB, false, OBF, CB, TB>(acc, M, N, (b0 + 4 * q) * 16, tok0, lane, wave, s0, nullptr, out, ld_out,
                                            lds);
  }
}

// Stage shape: bf16 weights use two stages of BK = 64 (128 KB of LDS); fp8
// weights, with 48 KB stages, fit three.
constexpr int kBK = 64;
constexpr int kWV = 4;
template <int WB>
constexpr int kNS = WB ? 3 : 2;

// Stream-K plan (see SkTail), sized for MI355X's 256 CUs with one workgroup
// per CU (the 64-token tiles of one-byte weights, 74 KB of LDS, fit two: the
// plan is conservative there).  The pieces run as one round (rem * d <= 256): measured, further
// rounds of pieces lose their gain to the slot stores and arrivals of every
// round.  d minimises a piece's time, ceil(KT / d) k-tiles plus
// kSkSlotCost k-tiles for each other slot its final sum may read, and the
// tail stays whole unless that saves an eighth of the plain last round (KT
// k-tiles); pieces hold at least kSkMinQ k-tiles.
constexpr int kSkCUs = 256;
constexpr int kSkMinQ = 16;
constexpr int kSkSlotCost = 4;

struct SkPlan {
  int nfull = 0, rem = 0, d = 0;
  int64_t cnt_bytes = 0, bytes = 0;   // counters; counters + slots
};

SkPlan sk_plan(int tiles, int KT, int bm) {
  SkPlan p;
  const int rem = tiles % kSkCUs;
  if (rem == 0) return p;
  int best_d = 1;
  int best = KT - KT / 8 + 1;   // a split must cost at most 7/8 of the plain round
  for (int d = 2; d <= KT / kSkMinQ && rem * d <= kSkCUs; ++d) {
    const int cost = (KT + d - 1) / d + kSkSlotCost * (d - 1);
    if (cost < best) {
      best = cost;
      best_d = d;
    }
  }
  if (best_d == 1) return p;
  p.nfull = tiles - rem;
  p.rem = rem;
  p.d = best_d;
  p.cnt_bytes = ((int64_t)rem * 4 + 255) / 256 * 256;
  p.bytes = p.cnt_bytes + (int64_t)rem * best_d * bm * BN * 4;
  return p;
}

int tiles_n_of(bool swiglu, int N) { return swiglu ? (N + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN; }

int gemm_tiles(bool swiglu, int M, int N, int bm) { return ((M + bm - 1) / bm) * tiles_n_of(swiglu, N); }

// Tokens per tile (64, 128 or 256) for M tokens, tiles_n tile columns and
// KT k-tiles.  A tile costs its CU the same time whatever share of its rows
// holds tokens, so at a few hundred tokens the 256-token tiles are mostly
// padding, and too few of them to fill the chip; the smaller tiles (all
// waves across the weight rows) waste less but read more LDS per MFMA.  When
// the 256-token tiles fill three quarters of a round of the CUs or more they
// are kept; otherwise the height with the least modelled time (whole rounds
// of kSkCUs tiles plus the stream-K tail) is taken, the taller one on a tie,
// with a k-tile of a 64- or 128-token tile costing 0.34 or 0.52 of a
// 256-token one (fitted to gate/up and down timings of the 70B shard, bf16
// and fp8 weights, 65 to 2048 tokens: the chosen height's time is 0.6 % above
// the best one's on average, 14 % at most).
int tile_bm(int M, int tiles_n, int KT) {
  if ((int64_t)((M + 255) / 256) * tiles_n * 4 >= kSkCUs * 3) return 256;
  constexpr int kHeights[3] = {256, 128, 64};
  constexpr int kCost[3] = {100, 52, 34};   // per k-tile, relative
  int best_bm = 256;
  int64_t best = -1;
  for (int i = 0; i < 3; ++i) {
    const int bm = kHeights[i];
    const int tiles = ((M + bm - 1) / bm) * tiles_n;
    const SkPlan p = sk_plan(tiles, KT, bm);
    const int64_t tail =
        tiles % kSkCUs == 0 ? 0 : p.d ? (KT + p.d - 1) / p.d + kSkSlotCost * (p.d - 1) : (int64_t)KT;
    const int64_t cost = kCost[i] * ((int64_t)(tiles / kSkCUs) * KT + tail);
    if (best < 0 || cost < best) {
      best = cost;
      best_bm = bm;
    }
  }
  return best_bm;
}

__global__ void sk_clear_kernel(int* __restrict__ cnt, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) cnt[i] = 0;
}

}  // namespace

hipError_t launch_counter_clear(int* cnt, int n, hipStream_t stream) {
  return launch(K_SK_CLEAR, sk_clear_kernel, dim3(1), dim3(256), 0, stream, cnt, n);
}

namespace {

// One GEMM launch: out = epilogue(rows of W (N of them; gate/up: N channels,
// 2N weight rows) times the activation rows).  skws: stream-K scratch of
// sk_plan(...).bytes, or null for whole tiles only.
template <bool SWIGLU, int WB, int BK, int NS, int BM, bool OBF, bool A8>
hipError_t run_gemm_bm(int kind, int M, int N, int K, const XRows& xr, const void* w0, const void* w1, int64_t ldw,
                       const float* s0, const float* s1, const float* sx, void* out, int64_t ldo, void* skws,
                       hipStream_t stream) {
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles = gemm_tiles(SWIGLU, M, N, BM);
  SkTail sk{};
  unsigned grid = (unsigned)tiles;
  const SkPlan p = skws ? sk_plan(tiles, K / BK, BM) : SkPlan{};
  if (p.d) {
    sk.cnt = static_cast<int*>(skws);
    sk.part = reinterpret_cast<float*>(static_cast<uint8_t*>(skws) + p.cnt_bytes);
    sk.nfull = p.nfull;
    sk.d = p.d;
    grid = (unsigned)(p.nfull + p.rem * p.d);
    const hipError_t e = launch(K_SK_CLEAR, sk_clear_kernel, dim3(1), dim3(256), 0, stream, sk.cnt, p.rem);
    if (e != hipSuccess) return e;
  }
  if constexpr (BM == 256 && ((WB == kWeightWide && !A8) || (WB == kWeightE4M3 && A8 && BK == 128))) {
    // bf16 x bf16 and fp8 x fp8 on 256 x 256 tiles: the eight-wave ping-pong kernel
    if (p.d)
      return launch(kind, gemm_pp_kernel<SWIGLU, OBF, true, A8>, dim3(grid), dim3(512), 0, stream, M, N, K, xr,
                    (const uint8_t*)w0, (const uint8_t*)w1, ldw, s0, s1, sx, out, ldo, tiles_m, tiles / tiles_m, sk);
    return launch(kind, gemm_pp_kernel<SWIGLU, OBF, false, A8>, dim3(grid), dim3(512), 0, stream, M, N, K, xr,
                  (const uint8_t*)w0, (const uint8_t*)w1, ldw, s0, s1, sx, out, ldo, tiles_m, tiles / tiles_m, sk);
  }
  if (p.d)
    return launch(kind, gemm_kernel<SWIGLU, WB, BK, NS, kWV, BM, OBF, A8, true>, dim3(grid), dim3(kWV * 64), 0, stream, M,
                  N, K, xr, (const uint8_t*)w0, (const uint8_t*)w1, ldw, s0, s1, sx, out, ldo, tiles_m, tiles / tiles_m,
                  sk);
  return launch(kind, gemm_kernel<SWIGLU, WB, BK, NS, kWV, BM, OBF, A8, false>, dim3(grid), dim3(kWV * 64), 0, stream, M, N,
                K, xr, (const uint8_t*)w0, (const uint8_t*)w1, ldw, s0, s1, sx, out, ldo, tiles_m, tiles / tiles_m, sk);
}

// One GEMM launch with the tile height for M tokens.
template <bool SWIGLU, int WB, int BK, int NS, bool OBF, bool A8>
hipError_t run_gemm(int kind, int M, int N, int K, const XRows& xr, const void* w0, const void* w1, int64_t ldw,
                    const float* s0, const float* s1, const float* sx, void* out, int64_t ldo, void* skws,
                    hipStream_t stream) {
  switch (tile_bm(M, tiles_n_of(SWIGLU, N), K / BK)) {
    case 64:
      return run_gemm_bm<SWIGLU, WB, BK, NS, 64, OBF, A8>(kind, M, N, K, xr, w0, w1, ldw, s0, s1, sx, out, ldo, skws,
                                                         stream);
    case 128:
      return run_gemm_bm<SWIGLU, WB, BK, NS, 128, OBF, A8>(kind, M, N, K, xr, w0, w1, ldw, s0, s1, sx, out, ldo, skws,
                                                          stream);
    default:
      return run_gemm_bm<SWIGLU, WB, BK, NS, 256, OBF, A8>(kind, M, N, K, xr, w0, w1, ldw, s0, s1, sx, out, ldo, skws,
                                                          stream);
  }
}

XRows single_rows(const void* p, int M, int64_t ld) {
  XRows r{};
  r.p[0] = p;
  r.nb = 1;
  r.rows = M;
  r.ld = ld;
  return r;
}

template <int WB>
hipError_t run_gateup(const ShardArgs& a, hipStream_t stream) {
  return run_gemm<true, WB, kBK, kNS<WB>, false, false>(K_GATEUP_PREFILL, a.M, a.I_s, a.h, a.x, a.wg, a.wu,
                                                         a.ldw_gu, a.sg, a.su, nullptr, a.a, a.lda, a.sk, stream);
}

template <int WB, bool OBF>
hipError_t run_rowgemm(const RowGemm& g, hipStream_t stream) {
  return run_gemm<false, WB, kBK, kNS<WB>, OBF, false>(g.kind_prefill, g.M, g.N, g.K, single_rows(g.a, g.M, g.lda),
                                                        g.w, nullptr, g.ldw, g.s, nullptr, nullptr, g.out, g.ldo,
                                                        g.ws, stream);
}

int64_t sk_bytes(bool swiglu, int M, int N, int K, int BK) {
  const int bm = tile_bm(M, tiles_n_of(swiglu, N), K / BK);
  return sk_plan(gemm_tiles(swiglu, M, N, bm), K / BK, bm).bytes;
}

// Packed-weight GEMM launch (256-token tiles): N output channels (gate/up)
// or rows (down) from nblk packed 16-row blocks; skws as in run_gemm_bm.
template <bool SWIGLU, int WB>
hipError_t run_gemm_pk(int kind, int M, int N, int K, const void* x, int64_t ldx, const void* wp, int nblk,
                       const float* s0, const float* s1, void* out, int64_t ldo, void* skws, hipStream_t stream) {
  constexpr int BM = 256;
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles = gemm_tiles(SWIGLU, M, N, BM);
  const SkPlan p = skws ? sk_plan(tiles, K / kBK, BM) : SkPlan{};
  SkTail sk{};
  if (p.d) {
    sk.cnt = static_cast<int*>(skws);
    sk.part = reinterpret_cast<float*>(static_cast<uint8_t*>(skws) + p.cnt_bytes);
    sk.nfull = p.nfull;
    sk.d = p.d;
    const hipError_t e = launch(K_SK_CLEAR, sk_clear_kernel, dim3(1), dim3(256), 0, stream, sk.cnt, p.rem);
    if (e != hipSuccess) return e;
    return launch(kind, gemm_pk_kernel<SWIGLU, WB, false, true>, dim3((unsigned)(p.nfull + p.rem * p.d)), dim3(512),
                  0, stream, M, N, K, (const uint8_t*)x, ldx, (const uint8_t*)wp, nblk, s0, s1, out, ldo, tiles_m,
                  tiles / tiles_m, sk);
  }
  return launch(kind, gemm_pk_kernel<SWIGLU, WB, false, false>, dim3((unsigned)tiles), dim3(512), 0, stream, M, N, K,
                (const uint8_t*)x, ldx, (const uint8_t*)wp, nblk, s0, s1, out, ldo, tiles_m, tiles / tiles_m, sk);
}

}  // namespace

int64_t rowgemm_prefill_workspace_bytes(int M, int N, int K) { return sk_bytes(false, M, N, K, kBK); }

int64_t forward_prefill_sk_bytes(int M, int h, int I_s, bool a8) {
  const int bk = a8 ? 128 : kBK;
  return max(sk_bytes(true, M, I_s, h, bk), sk_bytes(false, M, h, I_s, bk));
}

int64_t forward_prefill_packed_sk_bytes(int M, int h, int I_s) {
  return max(sk_plan(gemm_tiles(true, M, I_s, 256), h / kBK, 256).bytes,
             sk_plan(gemm_tiles(false, M, h, 256), I_s / kBK, 256).bytes);
}

hipError_t launch_rowgemm_prefill(const RowGemm& g, hipStream_t stream) {
  switch (g.wb) {
    case kWeightE4M3:
      return g.out_bf16 ? run_rowgemm<kWeightE4M3, true>(g, stream) : run_rowgemm<kWeightE4M3, false>(g, stream);
    case kWeightI8:
      return g.out_bf16 ? run_rowgemm<kWeightI8, true>(g, stream) : run_rowgemm<kWeightI8, false>(g, stream);
    default:
      return g.out_bf16 ? run_rowgemm<kWeightWide, true>(g, stream) : run_rowgemm<kWeightWide, false>(g, stream);
  }
}

hipError_t launch_forward_w8a8(const ShardArgs& a, const W8A8Bufs& b, hipStream_t stream) {
  constexpr int WB = kWeightE4M3;
  hipError_t e = launch_quant_rows(a.M, a.h, a.x.p[0], a.x.ld, b.xq, a.h, b.sx, stream);
  if (e != hipSuccess) return e;
  e = run_gemm<true, WB, 128, 2, false, true>(K_GATEUP_W8A8, a.M, a.I_s, a.h, single_rows(b.xq, a.M, a.h), a.wg,
                                              a.wu, a.ldw_gu, a.sg, a.su, b.sx, a.a, a.lda, a.sk, stream);
  if (e != hipSuccess) return e;
  e = launch_quant_rows(a.M, a.I_s, a.a, a.lda, b.aq, a.I_s, b.sa, stream);
  if (e != hipSuccess) return e;
  return run_gemm<false, WB, 128, 2, false, true>(K_DOWN_W8A8, a.M, a.h, a.I_s, single_rows(b.aq, a.M, a.I_s), a.wd,
                                                  nullptr, a.ldw_down, a.sd, nullptr, b.sa, a.p, a.ldp, a.sk, stream);
}

// Packed weights (contiguous X: the packed forward has no row-block form).
template <int WB>
hipError_t forward_prefill_packed_wb(const ShardArgs& a, hipStream_t stream) {
  hipError_t e = run_gemm_pk<true, WB>(K_GATEUP_PREFILL, a.M, a.I_s, a.h, a.x.p[0], a.x.ld, a.wg, (a.I_s + 7) / 8,
                                       a.sg, a.su, a.a, a.lda, a.sk, stream);
  if (e != hipSuccess) return e;
  return run_gemm_pk<false, WB>(K_DOWN_PREFILL, a.M, a.h, a.I_s, a.a, a.lda, a.wd, (a.h + 15) / 16, a.sd, nullptr,
                                a.p, a.ldp, a.sk, stream);
}

hipError_t launch_forward_prefill_packed(const ShardArgs& a, hipStream_t stream) {
  if (a.x.nb != 1) return hipErrorInvalidValue;
  switch (a.wb) {
    case kWeightE4M3: return forward_prefill_packed_wb<kWeightE4M3>(a, stream);
    case kWeightI8: return forward_prefill_packed_wb<kWeightI8>(a, stream);
    default: return forward_prefill_packed_wb<kWeightWide>(a, stream);
  }
}

hipError_t launch_forward_prefill(const ShardArgs& a, hipStream_t stream) {
  if (a.packed) return launch_forward_prefill_packed(a, stream);
  hipError_t e;
  switch (a.wb) {
    case kWeightE4M3: e = run_gateup<kWeightE4M3>(a, stream); break;
    case kWeightI8: e = run_gateup<kWeightI8>(a, stream); break;
    default: e = run_gateup<kWeightWide>(a, stream); break;
  }
  if (e != hipSuccess) return e;
  RowGemm g = down_of(a);
  g.ws = static_cast<float*>(a.sk);
  return launch_rowgemm_prefill(g, stream);
}

}  // namespace tpmlp
