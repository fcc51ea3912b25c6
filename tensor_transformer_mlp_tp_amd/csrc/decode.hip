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
// One-byte weights (OCP e4m3fn or int8 codes): each lane's 16-byte load
// carries 16 codes of one row = two MFMA k-groups; they are widened to bf16 in
// registers (exact) and the per-output-channel fp32 scale is applied to the
// fp32 sums.  The activations are read with the same k order, so the dot
// products are exact reorderings of the definition.
//
// The down kernels are generic row GEMMs, out = a * W^T with W in the
// (out, in) layout (RowGemm): they also run the attention block's
// projections, with fp32 or bf16 output, and for narrow outputs (too few row
// blocks to cover the chip) split K over a second grid dimension, the range
// that finishes a tile last adding its ranges in order.

#include "common.h"
#include "internal.h"

namespace tpmlp {

namespace {

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Packed weights (pack_kernel below) store every 16-row block as a run of
// 1 KB MFMA A fragments, block after block: fragment st of block blk, at
// packed_frag(blk, nsteps, st), gives lane l (16 bytes) row l % 16's weight
// bytes [64 st + 16 (l / 16), +16), i.e. 32 bf16 or 64 one-byte k-values of
// the 16 rows.  (Interleaving the fragments of groups of 8 blocks, so that
// a split-K workgroup's 8 blocks read one contiguous range per step, was
// measured no faster there and a third slower for the one-block rings.)
constexpr int kPackStep = 1024;           // bytes between a block's consecutive fragments
constexpr int kPackJS = 4 * kPackStep;    // ... and between its consecutive ring slots (4 fragments)
__host__ __device__ __forceinline__ int64_t packed_frag(int blk, int nsteps, int st) {
  return ((int64_t)blk * nsteps + st) * kPackStep;
}

// Weights are read exactly once per call: non-temporal loads keep them from
// displacing the activations, which every workgroup re-reads from L2.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// A batch of U consecutive k-steps held in registers.  A step is 32 k (bf16
// weights) or 64 k (fp8 weights): one 16-byte weight load per lane per row
// block, plus the matching activation fragments.
template <int NT, int RB, int U, int WB>
struct Batch {
  static constexpr int XJ = WB ? 2 : 1;
  u32x4 wf[U][RB];
  u32x4 xf[U][NT][XJ];
};

// Issue the loads of the batch starting at step s.  wrow[r]: this lane's
// weight bytes of step 0 in row block r; step st adds st * JS bytes.  Steps
// at or past s_end (only in the last, partial batch) re-read step s_end - 1,
// which is valid memory; their products are skipped in mac_batch.
template <int NT, int RB, int U, int WB, int JS>
__device__ __forceinline__ void load_batch(Batch<NT, RB, U, WB>& bt, const uint8_t* const (&wrow)[RB],
                                           const uint16_t* const (&xrow)[NT], int s, int s_end, int grp) {
  constexpr int KSTEP = WB ? 64 : 32;
  constexpr int XJ = WB ? 2 : 1;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t st = min(s + u, s_end - 1);
#pragma unroll
    for (int r = 0; r < RB; ++r) bt.wf[u][r] = ld16_stream(wrow[r] + st * JS);
#pragma unroll
    for (int b = 0; b < NT; ++b)
#pragma unroll
      for (int j = 0; j < XJ; ++j) bt.xf[u][b][j] = ld16(xrow[b] + st * KSTEP + grp * (8 * XJ) + j * 8);
  }
}

// MFMAs of the first n (<= U) steps of a loaded batch.  Token rows past M
// were loaded from a clamped row and are zeroed here.
template <int NT, int RB, int U, int WB>
__device__ __forceinline__ void mac_batch(f32x4 (&acc)[RB][NT], const Batch<NT, RB, U, WB>& bt,
                                          const bool (&xok)[NT], int n) {
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u >= n) break;  // wave-uniform
    bf16x8 xv[NT][WB ? 2 : 1];
#pragma unroll
    for (int b = 0; b < NT; ++b)
#pragma unroll
      for (int j = 0; j < (WB ? 2 : 1); ++j) xv[b][j] = as_bf16x8(xok[b] ? bt.xf[u][b][j] : zero);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      if constexpr (WB) {
        const bf16x8 lo = byte8_to_bf16x8<WB>(bt.wf[u][r][0], bt.wf[u][r][1]);
        const bf16x8 hi = byte8_to_bf16x8<WB>(bt.wf[u][r][2], bt.wf[u][r][3]);
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
template <int NT, int RB, int U, int WB, int JS>
__device__ __forceinline__ void mac_range(f32x4 (&acc)[RB][NT], const uint8_t* const (&wrow)[RB],
                                          const uint16_t* const (&xrow)[NT], const bool (&xok)[NT],
                                          int s_beg, int s_end, int grp) {
  if (s_beg >= s_end) return;
  Batch<NT, RB, U, WB> b0, b1;
  int s = s_beg;
  load_batch<NT, RB, U, WB, JS>(b0, wrow, xrow, s, s_end, grp);
  while (true) {
    int nxt = s + U;
    if (nxt < s_end) load_batch<NT, RB, U, WB, JS>(b1, wrow, xrow, nxt, s_end, grp);
    mac_batch(acc, b0, xok, s_end - s);
    if (nxt >= s_end) break;
    s = nxt;
    nxt = s + U;
    if (nxt < s_end) load_batch<NT, RB, U, WB, JS>(b0, wrow, xrow, nxt, s_end, grp);
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

template <int NT, int RB, int WAVES, int UNROLL, int WB>
__global__ __launch_bounds__(WAVES * 64) void gateup_decode_kernel(
    int M, int h, int I_s, const XRows xr,
    const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu, int64_t ldw,
    const float* __restrict__ sg, const float* __restrict__ su,
    uint16_t* __restrict__ a_out, int64_t lda) {
  constexpr int EB = WB ? 1 : 2;
  constexpr int KSTEP = WB ? 64 : 32;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int row16 = lane & 15;
  const int grp = lane >> 4;
  const int c0 = blockIdx.x * (8 * RB);
  const int nsteps = h / KSTEP;

  const uint8_t* wrow[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int ch = min(c0 + 8 * r + (row16 & 7), I_s - 1);
    wrow[r] = (row16 < 8 ? wg : wu) + (int64_t)ch * ldw * EB + grp * 16;
  }
  const uint16_t* xrow[NT];
  bool xok[NT];
#pragma unroll
  for (int b = 0; b < NT; ++b) {
    const int tok = b * 16 + row16;
    xok[b] = tok < M;
    xrow[b] = x_row<uint16_t>(xr, min(tok, M - 1));
  }

  const int s_beg = (wave * nsteps) / WAVES;
  const int s_end = ((wave + 1) * nsteps) / WAVES;
  f32x4 acc[RB][NT];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[r][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  mac_range<NT, RB, UNROLL, WB, KSTEP * EB>(acc, wrow, xrow, xok, s_beg, s_end, grp);

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
          if constexpr (WB) {
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

// out (M x N) = a_in (M x K) * wd^T, wd N x K; fp32 or bf16 (OBF) output.
template <int NT, int RB, int WAVES, int UNROLL, int WB, bool OBF>
__global__ __launch_bounds__(WAVES * 64) void down_decode_kernel(
    int M, int h, int I_s, const uint16_t* __restrict__ a_in, int64_t lda,
    const uint8_t* __restrict__ wd, int64_t ldw, const float* __restrict__ sd,
    void* __restrict__ p, int64_t ldp) {
  constexpr int EB = WB ? 1 : 2;
  constexpr int KSTEP = WB ? 64 : 32;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int row16 = lane & 15;
  const int grp = lane >> 4;
  const int n0 = blockIdx.x * (16 * RB);
  const int nsteps = I_s / KSTEP;

  const uint8_t* wrow[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int f = min(n0 + 16 * r + row16, h - 1);
    wrow[r] = wd + (int64_t)f * ldw * EB + grp * 16;
  }
  const uint16_t* xrow[NT];
  bool xok[NT];
#pragma unroll
  for (int b = 0; b < NT; ++b) {
    const int tok = b * 16 + row16;
    xok[b] = tok < M;
    xrow[b] = a_in + (int64_t)min(tok, M - 1) * lda;
  }

  const int s_beg = (wave * nsteps) / WAVES;
  const int s_end = ((wave + 1) * nsteps) / WAVES;
  f32x4 acc[RB][NT];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[r][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  mac_range<NT, RB, UNROLL, WB, KSTEP * EB>(acc, wrow, xrow, xok, s_beg, s_end, grp);

  reduce_waves<NT, RB, WAVES>(acc, wave, lane, [&](int r, int b, f32x4 v) {
    const int f = n0 + 16 * r + 4 * grp;  // features f .. f+3
    const int tok = b * 16 + row16;
    if (tok < M && f < h) {
      if constexpr (WB) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] *= sd[f + i];
      }
      store_out4<OBF>(p, (int64_t)tok * ldp + f, v);
    }
  });
}

// ---------------------------------------------------------------------------
// Streaming variant: weights go HBM -> LDS with direct-to-LDS loads into a
// ring private to each wave, then LDS -> MFMA fragments.  Each direct load
// instruction reads 4 weight rows x 256 contiguous bytes (instead of the 16
// rows x 64 bytes a lane-per-row MFMA fragment load touches), which streams
// HBM measurably better, and the ring keeps S-1 slots per wave in flight
// without spending VGPRs.  A slot is RB blocks of 16 rows x 256 bytes (128
// bf16 or 256 fp8 k-values each); its 16-byte chunks are stored XOR-swizzled
// by row so the 16 rows of a fragment read sit in 16 different bank slots.
//
// The activation fragments of a slot come from L2 in registers and serve all
// RB row blocks.  With more than 16 tokens those fragment reads, not the
// weight stream, bound the kernel (every workgroup re-reads the whole
// activation from L2), so the launch gives each wave RB = 2 row blocks there:
// half the activation traffic per weight byte, at half the workgroup count.
//
// The four waves of a workgroup take interleaved slots (wave q: q, q+4, ...),
// so at any moment the workgroup reads a contiguous kilobyte of each row.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void dma16(const void* gsrc, void* lds_dst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gsrc,
                                   (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}

// s_waitcnt vmcnt(N), lgkmcnt/expcnt not waited on.  The counter holds at
// most 63 loads, so a larger N is clamped (which only waits longer).
template <int N0>
__device__ __forceinline__ void wait_vm() {
  constexpr int N = N0 > 63 ? 63 : N0;
  static_assert(N >= 0, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until slot j's D direct loads have landed.  Per iteration the wave
// issues XL activation loads and then the D direct loads of a slot S-1
// ahead; the first S-1 slots were issued up front without activation loads.
template <int S, int XL, int D, int J>
__device__ __forceinline__ void wait_slot_peeled(int j) {
  if constexpr (J >= S - 2) {
    wait_vm<(S - 2) * (XL + D)>();
  } else {
    if (j == J) wait_vm<D * (S - 2 - J) + J * (XL + D)>();
    else wait_slot_peeled<S, XL, D, J + 1>(j);
  }
}

// Byte offset, within one 16-row block of a ring slot, of row r's 16-byte
// chunk q (q = 0..15; 16 weight bytes each).  From the (out, in) layout the
// direct loads carry 4 rows x 256 bytes and the chunks sit XOR-swizzled by
// row; packed weights (PK) arrive in MFMA fragment order: kilobyte q / 4
// holds chunk q % 4 of the 16 rows, row r in lane 16 * (q % 4) + r.
template <bool PK>
__device__ __forceinline__ int ring_chunk(int r, int q) {
  return PK ? (q >> 2) * 1024 + ((q & 3) * 16 + r) * 16 : r * 256 + ((q ^ r) * 16);
}

// Stream slots j_beg, j_beg + jstep, ... (nsl of them) of this wave's RB
// row blocks through its ring and accumulate the MFMAs.  dsrc[rb][i]: this
// lane's source for direct-load instruction i of block rb in slot 0 (row
// 4i + lane/16, pre-swizzled chunk; packed: kilobyte i of the slot); slot j
// adds j*JS bytes (256 in the row-major layout, 4096 in the packed one).
// xrow/xok: activation rows of the NT token blocks.
template <int NT, int RB, int WB, int S, bool PK>
__device__ __forceinline__ void stream_rows(f32x4 (&acc)[RB][NT], uint8_t* ring,
                                            const uint8_t* const (&dsrc)[RB][4],
                                            const uint16_t* const (&xrow)[NT], const bool (&xok)[NT],
                                            int j_beg, int nsl, int jstep, int lane) {
  constexpr int STEPS = WB ? 8 : 4;          // MFMA k-steps (32 k) per slot
  constexpr int KS = WB ? 256 : 128;         // k per slot
  constexpr int XL = STEPS * NT;              // activation loads per slot
  constexpr int D = 4 * RB;                   // direct loads per slot
  constexpr int SLOT = RB * 4096;             // bytes per slot
  constexpr int JS = PK ? kPackJS : 256;
  const int r = lane & 15, g = lane >> 4;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  if (nsl <= 0) return;
  auto issue = [&](int j, int pos) {
    uint8_t* dst = ring + pos * SLOT;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) dma16(dsrc[rb][i] + (int64_t)j * JS, dst + rb * 4096 + i * 1024);
  };
  // (Loading only the lanes of real tokens, exec-masked, measured slower: 70B
  // gate/up at one token 21.4 -> 22.0 us; the clamped rows are L1 hits.)
  auto load_x = [&](int j, u32x4 (&xf)[STEPS][NT]) {
#pragma unroll
    for (int b = 0; b < NT; ++b)
#pragma unroll
      for (int st = 0; st < STEPS; ++st) {
        const int ko = WB ? (64 * (st >> 1) + 16 * g + 8 * (st & 1)) : (32 * st + 8 * g);
        xf[st][b] = *reinterpret_cast<const u32x4*>(xrow[b] + (int64_t)j * KS + ko);
      }
  };
  auto compute = [&](int pos, const u32x4 (&xf)[STEPS][NT]) {
    const uint8_t* sl = ring + pos * SLOT;
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if constexpr (WB) {
          if ((st & 1) == 0) {
            const int q = 4 * (st >> 1) + g;
            const u32x4 v = *reinterpret_cast<const u32x4*>(sl + rb * 4096 + ring_chunk<PK>(r, q));
            const bf16x8 w0 = byte8_to_bf16x8<WB>(v[0], v[1]);
            const bf16x8 w1 = byte8_to_bf16x8<WB>(v[2], v[3]);
#pragma unroll
            for (int b = 0; b < NT; ++b) acc[rb][b] = mfma16(w0, as_bf16x8(xok[b] ? xf[st][b] : zero), acc[rb][b]);
#pragma unroll
            for (int b = 0; b < NT; ++b) acc[rb][b] = mfma16(w1, as_bf16x8(xok[b] ? xf[st + 1][b] : zero), acc[rb][b]);
          }
        } else {
          const int q = 4 * st + g;
          const bf16x8 w = as_bf16x8(*reinterpret_cast<const u32x4*>(sl + rb * 4096 + ring_chunk<PK>(r, q)));
#pragma unroll
          for (int b = 0; b < NT; ++b) acc[rb][b] = mfma16(w, as_bf16x8(xok[b] ? xf[st][b] : zero), acc[rb][b]);
        }
      }
    }
  };
#pragma unroll
  for (int p = 0; p < S - 1; ++p) issue(j_beg + min(p, nsl - 1) * jstep, p);
  // Activation fragments one slot ahead in a second register set: the loads
  // of slot jj+1 (activations and weights) fly while slot jj is computed.
  // Issue order per step: activations of jj+1, then the direct loads of
  // jj+S-1, so the wait before slot jj covers both of its groups.
  static_assert(S == 2, "activation prefetch assumes a two-slot ring");
  u32x4 xa[STEPS][NT], xb[STEPS][NT];
  load_x(j_beg, xa);
  auto step = [&](int jj, u32x4 (&cur)[STEPS][NT], u32x4 (&nxt)[STEPS][NT]) {
    wait_vm<0>();
    load_x(j_beg + min(jj + 1, nsl - 1) * jstep, nxt);
    issue(j_beg + min(jj + 1, nsl - 1) * jstep, (jj + 1) & 1);
    compute(jj & 1, cur);
  };
  int jj = 0;
  for (; jj + 1 < nsl; jj += 2) {
    step(jj, xa, xb);
    step(jj + 1, xb, xa);
  }
  if (jj < nsl) step(jj, xa, xb);
  __builtin_amdgcn_s_waitcnt(0);  // the ring's last (duplicate) loads are done before LDS is reused
}

// Same stream with the activations staged through the ring too: each slot
// also holds the NT token blocks' activation rows for its k range (16 rows x
// 2*KS bytes per block, direct-loaded whole 128-byte lines, 16-byte chunks
// XOR-swizzled by row), and the MFMA fragments are read from LDS.  Register
// fragment loads touch 16 rows x 64 bytes per instruction, half of each line;
// with more than 16 tokens that doubled line traffic, not the weight stream,
// is what bounds the kernel.  xsrc[b][i]: this lane's source for activation
// load i of token block b in slot 0; slot j adds j * 2*KS bytes.
template <int NT, int RB, int WB, int S, bool PK>
__device__ __forceinline__ void stream_rows_xd(f32x4 (&acc)[RB][NT], uint8_t* ring,
                                               const uint8_t* const (&dsrc)[RB][4],
                                               const uint8_t* const (&xsrc)[NT][WB ? 8 : 4],
                                               const bool (&xok)[NT], int j_beg, int nsl, int jstep,
                                               int lane) {
  constexpr int STEPS = WB ? 8 : 4;          // MFMA k-steps (32 k) per slot
  constexpr int KS = WB ? 256 : 128;         // k per slot
  constexpr int XROWB = 2 * KS;               // activation bytes per row per slot
  constexpr int XI = WB ? 8 : 4;             // activation loads per token block
  constexpr int XBLK = 16 * XROWB;
  constexpr int D = 4 * RB + NT * XI;         // direct loads per slot
  constexpr int SLOT = RB * 4096 + NT * XBLK; // bytes per slot
  constexpr int JS = PK ? kPackJS : 256;
  const int r = lane & 15, g = lane >> 4;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  if (nsl <= 0) return;
  auto issue = [&](int j, int pos) {
    uint8_t* dst = ring + pos * SLOT;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) dma16(dsrc[rb][i] + (int64_t)j * JS, dst + rb * 4096 + i * 1024);
#pragma unroll
    for (int b = 0; b < NT; ++b)
#pragma unroll
      for (int i = 0; i < XI; ++i)
        dma16(xsrc[b][i] + (int64_t)j * XROWB, dst + RB * 4096 + b * XBLK + i * 1024);
  };
  auto compute = [&](int pos) {
    const uint8_t* sl = ring + pos * SLOT;
    const uint8_t* xl = ring + pos * SLOT + RB * 4096 + r * XROWB;
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      u32x4 xf[NT];
      const int xc = WB ? (8 * (st >> 1) + 2 * g + (st & 1)) : (4 * st + g);
#pragma unroll
      for (int b = 0; b < NT; ++b) xf[b] = *reinterpret_cast<const u32x4*>(xl + b * XBLK + ((xc ^ r) * 16));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        bf16x8 w;
        if constexpr (WB) {
          const int q = 4 * (st >> 1) + g;
          const u32x4 v = *reinterpret_cast<const u32x4*>(sl + rb * 4096 + ring_chunk<PK>(r, q));
          w = (st & 1) ? byte8_to_bf16x8<WB>(v[2], v[3]) : byte8_to_bf16x8<WB>(v[0], v[1]);
        } else {
          const int q = 4 * st + g;
          w = as_bf16x8(*reinterpret_cast<const u32x4*>(sl + rb * 4096 + ring_chunk<PK>(r, q)));
        }
#pragma unroll
        for (int b = 0; b < NT; ++b) acc[rb][b] = mfma16(w, as_bf16x8(xok[b] ? xf[b] : zero), acc[rb][b]);
      }
    }
  };
#pragma unroll
  for (int p = 0; p < S - 1; ++p) issue(j_beg + min(p, nsl - 1) * jstep, p);
  int pos = 0;
  for (int jj = 0; jj < nsl; ++jj) {
    wait_slot_peeled<S, 0, D, 0>(jj);
    const int npos = pos == 0 ? S - 1 : pos - 1;   // ring slot of j+S-1 (held j-1)
    issue(j_beg + min(jj + S - 1, nsl - 1) * jstep, npos);
    compute(pos);
    pos = pos == S - 1 ? 0 : pos + 1;
  }
  __builtin_amdgcn_s_waitcnt(0);  // the ring's last (duplicate) loads are done before LDS is reused
}

// Activation direct-load sources of this lane: token block b, load i covers
// rows i*RPI + lane/LPR of the block (LPR lanes per row), logical chunk
// (lane % LPR) ^ row.
template <int WB, int NT, typename XPtr>
__device__ __forceinline__ void stream_x_sources(const uint8_t* (&xsrc)[NT][WB ? 8 : 4], int lane, XPtr xptr) {
  constexpr int LPR = WB ? 32 : 16;
  constexpr int RPI = 64 / LPR;
#pragma unroll
  for (int b = 0; b < NT; ++b)
#pragma unroll
    for (int i = 0; i < (WB ? 8 : 4); ++i) {
      const int row = i * RPI + lane / LPR;
      const int c = (lane % LPR) ^ row;
      xsrc[b][i] = reinterpret_cast<const uint8_t*>(xptr(b * 16 + row)) + c * 16;
    }
}

// Direct-load sources of this lane for the 4 instructions of a block in slot
// 0: rows 4i + lane/16 of the block, logical chunk (lane%16) ^ row.
template <typename RowPtr>
__device__ __forceinline__ void stream_sources(const uint8_t* (&dsrc)[4], int lane, RowPtr row_ptr) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * i + (lane >> 4);
    const int c = (lane & 15) ^ row;
    dsrc[i] = row_ptr(row) + c * 16;
  }
}

// Packed ring sources: load i of slot j of block blk is the block's fragment
// 4 j + i, lane l taking bytes [16 l, 16 l + 16).
__device__ __forceinline__ void packed_sources(const uint8_t* (&dsrc)[4], const uint8_t* packed, int blk,
                                               int nslots, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) dsrc[i] = packed + packed_frag(blk, 4 * nslots, i) + lane * 16;
}

// Cross-wave sum for the streaming kernels: like reduce_waves, but through
// the (no longer needed) ring memory instead of a separate LDS array.
template <int NT, int RB, int WAVES, typename Epi>
__device__ __forceinline__ void reduce_waves_ring(f32x4 (&acc)[RB][NT], f32x4* buf, int wave, int lane,
                                                  Epi epi) {
  __syncthreads();  // every wave is done with its ring
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int b = 0; b < NT; ++b) buf[(wave * RB * NT + r * NT + b) * 64 + lane] = acc[r][b];
  __syncthreads();
  for (int q = wave; q < RB * NT; q += WAVES) {
    f32x4 s = buf[q * 64 + lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) s = s + buf[(w * RB * NT + q) * 64 + lane];
    epi(q / NT, q % NT, s);
  }
}

constexpr int kSlots = 2;   // the register-activation stream's ring (its prefetch assumes two)
constexpr int kSWaves = 4;

// Slots of this wave: interleaved over the workgroup's WV waves.
template <int WV>
__device__ __forceinline__ void wave_slots(int nslots, int wave, int& j_beg, int& nsl, int& jstep) {
  j_beg = wave;
  jstep = WV;
  nsl = (nslots - wave + WV - 1) / WV;
}

// Ring geometry of a streaming kernel: slot bytes and ring depth.  With the
// activations in the ring (XD) the slots are larger, so those kernels run two
// waves per workgroup with three slots each.
template <int NT, int RB, int WB, bool XD>
struct StreamShape {
  static constexpr int WV = XD ? 2 : kSWaves;
  static constexpr int SLOT = RB * 4096 + (XD ? NT * 16 * 2 * (WB ? 256 : 128) : 0);
  static constexpr int S = XD ? (WV * 3 * SLOT <= 160 * 1024 ? 3 : 2) : kSlots;
  static constexpr int RING = WV * S * SLOT;
  static_assert(WV * RB * NT * 1024 <= RING, "the cross-wave sums fit the ring");
  static_assert(RING <= 160 * 1024, "LDS");
};

// PK: wg is the packed gate/up array (wu, ldw unused).
template <int NT, int RB, int WB, bool XD, bool PK>
__global__ __launch_bounds__((StreamShape<NT, RB, WB, XD>::WV * 64)) void gateup_stream_kernel(
    int M, int h, int I_s, const XRows xr,
    const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu, int64_t ldw,
    const float* __restrict__ sg, const float* __restrict__ su,
    uint16_t* __restrict__ a_out, int64_t lda) {
  using SS = StreamShape<NT, RB, WB, XD>;
  constexpr int EB = WB ? 1 : 2;
  constexpr int KS = WB ? 256 : 128;
  __shared__ __attribute__((aligned(1024))) uint8_t ring_all[SS::RING];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row16 = lane & 15, grp = lane >> 4;
  const int c0 = blockIdx.x * 8 * RB;
  // row block rb: rows 0-7 gate channels c0+8rb..+7, rows 8-15 the same channels' up rows
  const uint8_t* dsrc[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if constexpr (PK)
      packed_sources(dsrc[rb], wg, min(c0 / 8 + rb, (I_s + 7) / 8 - 1), h / KS, lane);
    else
      stream_sources(dsrc[rb], lane, [&](int row) {
        const int ch = min(c0 + 8 * rb + (row & 7), I_s - 1);
        return (row < 8 ? wg : wu) + (int64_t)ch * ldw * EB;
      });
  }
  int j_beg, nsl, jstep;
  wave_slots<SS::WV>(h / KS, wave, j_beg, nsl, jstep);
  bool xok[NT];
#pragma unroll
  for (int b = 0; b < NT; ++b) xok[b] = b * 16 + row16 < M;
  f32x4 acc[RB][NT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[rb][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint8_t* ring = ring_all + wave * SS::S * SS::SLOT;
  if constexpr (XD) {
    const uint8_t* xsrc[NT][WB ? 8 : 4];
    stream_x_sources<WB, NT>(xsrc, lane, [&](int tok) { return x_row<uint16_t>(xr, min(tok, M - 1)); });
    stream_rows_xd<NT, RB, WB, SS::S, PK>(acc, ring, dsrc, xsrc, xok, j_beg, nsl, jstep, lane);
  } else {
    const uint16_t* xrow[NT];
#pragma unroll
    for (int b = 0; b < NT; ++b) xrow[b] = x_row<uint16_t>(xr, min(b * 16 + row16, M - 1));
    stream_rows<NT, RB, WB, SS::S, PK>(acc, ring, dsrc, xrow, xok, j_beg, nsl, jstep, lane);
  }

  reduce_waves_ring<NT, RB, SS::WV>(acc, reinterpret_cast<f32x4*>(ring_all), wave, lane,
                                    [&](int rb, int b, f32x4 v) {
    f32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __shfl_xor(v[i], 32);
    if (grp < 2) {
      const int ch = c0 + 8 * rb + 4 * grp;
      const int tok = b * 16 + row16;
      if (tok < M && ch < I_s) {
        float a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float gv = v[i], uv = o[i];
          if constexpr (WB) {
            gv *= sg[ch + i];
            uv *= su[ch + i];
          }
          a[i] = silu(gv) * uv;
        }
        u32x2 packed = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
        *reinterpret_cast<u32x2*>(a_out + (int64_t)tok * lda + ch) = packed;
      }
    }
  });
}

// Split K (SPLIT, gridDim.y = nseg > 1): workgroup (x, y) streams the y-th of
// nseg contiguous ranges of the K slots, stores its unscaled fp32 sums in its
// slot of `part` (RB x NT x 1 KB per tile and range) and counts itself in the
// tile's arrival counter (zero at launch); the range that arrives last adds
// the tile's nseg slots in range order (the same sum whichever range is
// last), applies the row scales and writes the output.  No workgroup waits
// for another.  Skinny outputs (few 16-row blocks, long K) need the split to
// keep enough loads in flight across the chip.
// PK: wd is the packed array of the N x K weights (ldw unused).
template <int NT, int RB, int WB, bool XD, bool OBF, bool PK, bool SPLIT>
__global__ __launch_bounds__((StreamShape<NT, RB, WB, XD>::WV * 64)) void down_stream_kernel(
    int M, int h, int I_s, const uint16_t* __restrict__ a_in, int64_t lda,
    const uint8_t* __restrict__ wd, int64_t ldw, const float* __restrict__ sd,
    void* __restrict__ p, int64_t ldp, int nseg, float* __restrict__ part, int* __restrict__ cnt) {
  using SS = StreamShape<NT, RB, WB, XD>;
  constexpr int EB = WB ? 1 : 2;
  constexpr int KS = WB ? 256 : 128;
  __shared__ __attribute__((aligned(1024))) uint8_t ring_all[SS::RING];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row16 = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * 16 * RB;
  const int nslots = I_s / KS;
  const uint8_t* dsrc[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if constexpr (PK)
      packed_sources(dsrc[rb], wd, min(n0 / 16 + rb, (h + 15) / 16 - 1), nslots, lane);
    else
      stream_sources(dsrc[rb], lane,
                     [&](int row) { return wd + (int64_t)min(n0 + 16 * rb + row, h - 1) * ldw * EB; });
  }
  int j_beg, nsl, jstep;
  const int seg = blockIdx.y;
  const int s0 = (int)((int64_t)seg * nslots / nseg);
  const int s1 = (int)((int64_t)(seg + 1) * nslots / nseg);
  wave_slots<SS::WV>(s1 - s0, wave, j_beg, nsl, jstep);
  j_beg += s0;
  bool xok[NT];
#pragma unroll
  for (int b = 0; b < NT; ++b) xok[b] = b * 16 + row16 < M;
  f32x4 acc[RB][NT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[rb][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint8_t* ring = ring_all + wave * SS::S * SS::SLOT;
  if constexpr (XD) {
    const uint8_t* xsrc[NT][WB ? 8 : 4];
    stream_x_sources<WB, NT>(xsrc, lane, [&](int tok) { return a_in + (int64_t)min(tok, M - 1) * lda; });
    stream_rows_xd<NT, RB, WB, SS::S, PK>(acc, ring, dsrc, xsrc, xok, j_beg, nsl, jstep, lane);
  } else {
    const uint16_t* xrow[NT];
#pragma unroll
    for (int b = 0; b < NT; ++b) xrow[b] = a_in + (int64_t)min(b * 16 + row16, M - 1) * lda;
    stream_rows<NT, RB, WB, SS::S, PK>(acc, ring, dsrc, xrow, xok, j_beg, nsl, jstep, lane);
  }

  // the tile's slots (SPLIT): slot of range r at r * SLOT, position (rb, b)
  // of lane l at ((rb * NT + b) * 64 + l) * 16
  constexpr int SLOT = RB * NT * 1024;
  constexpr int kDeviceScope = 16;   // buffer cache policy: sc1
  const __amdgpu_buffer_rsrc_t slots = __builtin_amdgcn_make_buffer_rsrc(
      SPLIT ? part + (int64_t)blockIdx.x * nseg * (SLOT / 4) : part, 0, SPLIT ? nseg * SLOT : 0, 0x00020000);
  auto finish = [&](int rb, int b, f32x4 v) {
    const int f = n0 + 16 * rb + 4 * grp;
    const int tok = b * 16 + row16;
    if (tok < M && f < h) {
      if constexpr (WB) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] *= sd[f + i];
      }
      store_out4<OBF>(p, (int64_t)tok * ldp + f, v);
    }
  };
  reduce_waves_ring<NT, RB, SS::WV>(acc, reinterpret_cast<f32x4*>(ring_all), wave, lane,
                                    [&](int rb, int b, f32x4 v) {
    if constexpr (SPLIT)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), slots,
                                             seg * SLOT + ((rb * NT + b) * 64 + lane) * 16, 0, kDeviceScope);
    else
      finish(rb, b, v);
  });
  if constexpr (SPLIT) {
    // The ordering argument is the prefill stream-K tail's: every slot store
    // and load carries sc1 (they go to the point of coherence shared by the
    // XCDs), vmcnt(0) completes this range's stores at agent scope, the
    // barrier orders all lanes before the counter increment, and the last
    // range's loads are issued only once the increment's result is known.
    // The flag lives in the ring's memory (the cross-wave sums above are read
    // before the barrier).
    int* flag = reinterpret_cast<int*>(ring_all);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
      *flag = __hip_atomic_fetch_add(cnt + blockIdx.x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (*flag != nseg - 1) return;
    if (threadIdx.x == 0) __hip_atomic_store(cnt + blockIdx.x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // Wave w sums positions w, w + WV, ... (QPW of them), every range in
    // order; the loads of all its positions for FB ranges are issued
    // together (one memory round trip per FB ranges: the last range's sum
    // is the tail of the launch).
    constexpr int QPW = (RB * NT + SS::WV - 1) / SS::WV;
    constexpr int FB = 8;
    f32x4 sum[QPW];
    for (int r0 = 0; r0 < nseg; r0 += FB) {
      f32x4 t[FB][QPW];
#pragma unroll
      for (int j = 0; j < FB; ++j)
#pragma unroll
        for (int i = 0; i < QPW; ++i) {
          const int q = wave + SS::WV * i;
          if (r0 + j < nseg && q < RB * NT)
            t[j][i] = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(slots, (r0 + j) * SLOT + (q * 64 + lane) * 16, 0,
                                                             kDeviceScope));
        }
#pragma unroll
      for (int j = 0; j < FB; ++j)
#pragma unroll
        for (int i = 0; i < QPW; ++i)
          if (r0 + j < nseg) sum[i] = r0 + j == 0 ? t[j][i] : sum[i] + t[j][i];
    }
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      const int q = wave + SS::WV * i;
      if (q < RB * NT) finish(q / NT, q % NT, sum[i]);
    }
  }
}

// ---------------------------------------------------------------------------
// Split-K streams for 17 to 64 tokens.
//
// Above 16 tokens a stream whose workgroups each own a few rows is bound by
// its activation reads: every workgroup re-reads the activations of its K
// range, M / R bytes per weight byte for R rows per workgroup (two at 64
// tokens and 32 rows), and staged through the ring they also take the LDS
// that would hold weight bytes in flight.  Here a workgroup owns R = 16 W RB
// rows (W waves of RB 16-row blocks) and one of nseg contiguous K ranges,
// so the grid still covers the chip while each activation byte serves R
// rows:
//  - the activation fragments of a step (16 tokens x 32 k each, in MFMA B
//    order) are loaded once per workgroup, the W waves sharing the loads,
//    D - 1 steps ahead into registers, and written to one of two LDS
//    stages just before the step, where all W waves read them;
//  - each wave streams its own weight fragments (packed layout: one
//    contiguous kilobyte per load; (out, in) layout: 16 rows x 64 bytes)
//    straight into registers, D - 1 steps ahead;
//  - one barrier per step, between the stage writes and the reads.
// Every load goes to registers, so the compiler counts them all and places
// the waits (direct-to-LDS loads would make it wait for all of them before
// each LDS read).  The step loop is unrolled completely (ranges of at most
// NSTEP steps): in a loop the wait counting drains every load at the loop
// head.
// A step is one weight fragment: 32 k (bf16) or 64 k (one-byte weights).
//
// The nseg range sums of a tile meet as in the prefill stream-K tail: each
// range stores its fp32 sums with agent-scope (sc1) buffer stores, counts
// itself in the tile's arrival counter, and the range that arrives last adds
// the nseg sums in range order (the same sum whichever arrives last), sets
// the counter back to zero and runs the epilogue.  The counters are zeroed
// by a one-workgroup kernel before the first split GEMM of a call.
// ---------------------------------------------------------------------------

// f(std::integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <int NT, int WB, int W>
struct SkShape {
  static constexpr int XJ = WB ? 2 : 1;          // activation fragments per token block and step
  static constexpr int NF = NT * XJ;             // activation fragments per step
  static constexpr int AF = (NF + W - 1) / W;    // ... loaded by each of the W waves (padded)
  static constexpr int STAGE = W * AF * 1024;    // LDS bytes per stage
};

// Bytes of one range's fp32 sums of a tile (W waves x RB x NT fragments).
template <int NT, int RB, int W>
constexpr int kSkSlot = W * RB * NT * 1024;

// GU: gate/up (N = I_s channels, w0/w1 = W_gate/W_up or the packed array in
// w0, out = A in bf16 with SiLU(gate) * up applied); else a row GEMM
// (N output rows, out fp32 or bf16 (OBF)).  s0/s1: row scales of one-byte
// weights.  part/cnt: split scratch (nseg > 1).  Each of the nseg K ranges
// is at most NSTEP steps.
template <int NT, int RB, int W, int WB, int D, int NSTEP, bool PK, bool GU, bool OBF>
__global__ __launch_bounds__(W * 64) void sk_stream_kernel(
    int M, int N, int K, const XRows xr, const uint8_t* __restrict__ w0, const uint8_t* __restrict__ w1,
    int64_t ldw, const float* __restrict__ s0, const float* __restrict__ s1, void* __restrict__ out,
    int64_t ldo, int nseg, float* __restrict__ part, int* __restrict__ cnt) {
  using SS = SkShape<NT, WB, W>;
  constexpr int XJ = SS::XJ, AF = SS::AF;
  constexpr int EB = WB ? 1 : 2;
  constexpr int KSTEP = WB ? 64 : 32;           // k per step
  constexpr int JS = PK ? kPackStep : 64;       // weight bytes between steps
  __shared__ __attribute__((aligned(1024))) uint8_t stage_buf[2][SS::STAGE];
  __shared__ int flag;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int tile = blockIdx.x, seg = blockIdx.y;
  const int nsteps = K / KSTEP;
  const int sb = (int)((int64_t)seg * nsteps / nseg);
  const int n = (int)((int64_t)(seg + 1) * nsteps / nseg) - sb;

  // Weight sources of this wave's blocks at step sb.
  const int nblk = GU ? (N + 7) / 8 : (N + 15) / 16;
  const int blk0 = (tile * W + wave) * RB;
  const uint8_t* wsrc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int blk = min(blk0 + rb, nblk - 1);
    if constexpr (PK) {
      wsrc[rb] = w0 + packed_frag(blk, nsteps, sb) + lane * 16;
    } else if constexpr (GU) {
      const int ch = min(blk * 8 + (r16 & 7), N - 1);
      wsrc[rb] = (r16 < 8 ? w0 : w1) + (int64_t)ch * ldw * EB + g * 16 + (int64_t)sb * 64;
    } else {
      const int row = min(blk * 16 + r16, N - 1);
      wsrc[rb] = w0 + (int64_t)row * ldw * EB + g * 16 + (int64_t)sb * 64;
    }
  }
  // Activation fragments this wave loads: f = wave + W a (token block f / XJ,
  // part f % XJ); the padding fragments (f >= NF) repeat fragment 0 into
  // stage positions nobody reads.  Lane l loads token (l % 16) of the block,
  // which is the MFMA B order.
  const uint8_t* xsrc[AF];
#pragma unroll
  for (int a = 0; a < AF; ++a) {
    const int f = wave + W * a < SS::NF ? wave + W * a : 0;
    const int b = f / XJ, j = f % XJ;
    const int tok = min(b * 16 + r16, M - 1);
    const int k0 = sb * KSTEP + (WB ? 16 * g + 8 * j : 8 * g);
    xsrc[a] = reinterpret_cast<const uint8_t*>(x_row<uint16_t>(xr, tok) + k0);
  }

  // Steps past the range (j >= n, the pipeline's last D - 1 iterations)
  // still issue their loads, from the range's last activation fragment (an
  // L2 hit), into registers no step reads: every path through the unrolled
  // iterations then issues the same loads, so the compiler's wait counts
  // need no worst case over the range length.
  const uint8_t* spare = xsrc[0] + (int64_t)(n - 1) * (2 * KSTEP);
  // (A wave whose share of the step's fragments runs past NF loads and
  // stages nothing there: the CU's load bytes per step set the pace here, so
  // the three idle fragment loads of a 7-wave gate/up tile at 64 tokens cost
  // 5 % of its time.)
  auto issue_x = [&](int i, u32x4 (&dst)[AF]) {
#pragma unroll
    for (int a = 0; a < AF; ++a)
      if (wave + W * a < SS::NF) dst[a] = ld16(i < n ? xsrc[a] + (int64_t)i * (2 * KSTEP) : spare);
  };
  auto stage_x = [&](int stage, const u32x4 (&src)[AF]) {
#pragma unroll
    for (int a = 0; a < AF; ++a)
      if (wave + W * a < SS::NF)
        *reinterpret_cast<u32x4*>(stage_buf[stage] + (wave + W * a) * 1024 + lane * 16) = src[a];
  };
  auto issue_w = [&](int i, u32x4 (&dst)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) dst[rb] = ld16_stream(i < n ? wsrc[rb] + (int64_t)i * JS : spare);
  };
  f32x4 acc[RB][NT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[rb][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int stage, const u32x4 (&w)[RB]) {
    const uint8_t* st = stage_buf[stage] + lane * 16;
    u32x4 xf[NT][XJ];
#pragma unroll
    for (int b = 0; b < NT; ++b)
#pragma unroll
      for (int j = 0; j < XJ; ++j) xf[b][j] = *reinterpret_cast<const u32x4*>(st + (b * XJ + j) * 1024);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if constexpr (WB) {
        const bf16x8 lo = byte8_to_bf16x8<WB>(w[rb][0], w[rb][1]);
        const bf16x8 hi = byte8_to_bf16x8<WB>(w[rb][2], w[rb][3]);
#pragma unroll
        for (int b = 0; b < NT; ++b) {
          acc[rb][b] = mfma16(lo, as_bf16x8(xf[b][0]), acc[rb][b]);
          acc[rb][b] = mfma16(hi, as_bf16x8(xf[b][1]), acc[rb][b]);
        }
      } else {
#pragma unroll
        for (int b = 0; b < NT; ++b) acc[rb][b] = mfma16(as_bf16x8(w[rb]), as_bf16x8(xf[b][0]), acc[rb][b]);
      }
    }
  };

  // Iteration j (0 <= j < n + D - 1), with i = j - D + 1: once step i is
  // due, write its activation fragments (registers xv[i % D]) to stage i % 2
  // (step i - 2 read it; the previous barrier saw every wave finish those
  // reads), barrier (every wave's fragments are in), and compute it from the
  // stage and registers wf[i % D]; then issue step j (activations into
  // xv[j % D], weights into wf[j % D], both last used by step i - 1).
  // (Staging two or four steps per barrier measured no faster.)
  // The iterations are unrolled at compile time (static_for; n <= NSTEP):
  // every stage and register set is a constant, and the compiler's wait
  // counting stays exact (at the head of a loop it drains every load).
  u32x4 wf[D][RB], xv[D][AF];
  static_for<0, NSTEP + D - 1>([&](auto J) {
    constexpr int j = J, i = j - (D - 1);
    if constexpr (i >= 0) {
      if (i < n) {
        stage_x(i % 2, xv[i % D]);
        lds_barrier();
        compute(i % 2, wf[i % D]);
      }
    }
    if constexpr (j < NSTEP) {
      issue_x(j, xv[j % D]);
      issue_w(j, wf[j % D]);
    }
  });

  if (nseg > 1) {
    constexpr int SLOT = kSkSlot<NT, RB, W>;
    constexpr int kDeviceScope = 16;   // buffer cache policy: sc1
    const __amdgpu_buffer_rsrc_t slots = __builtin_amdgcn_make_buffer_rsrc(
        part + (int64_t)tile * nseg * (SLOT / 4), 0, nseg * SLOT, 0x00020000);
    auto off = [&](int p, int rb, int b) { return p * SLOT + ((wave * RB + rb) * NT + b) * 1024 + lane * 16; };
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int b = 0; b < NT; ++b)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[rb][b]), slots, off(seg, rb, b), 0,
                                               kDeviceScope);
    // The ordering argument is the prefill stream-K tail's (sk_handoff):
    // every slot store and load carries sc1, vmcnt(0) completes this range's
    // stores at agent scope, the barrier orders all lanes before the
    // counter increment, and the last range's loads depend on its result.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) flag = __hip_atomic_fetch_add(cnt + tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (flag != nseg - 1) return;
    if (threadIdx.x == 0) __hip_atomic_store(cnt + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // Ranges in order, FB at a time with all their loads in flight together
    // (one memory round trip per FB ranges); this range's own sums in place.
    constexpr int FB = 2;
    f32x4 sum[RB][NT];
    for (int p0 = 0; p0 < nseg; p0 += FB) {
      f32x4 v[FB][RB][NT];
#pragma unroll
      for (int q = 0; q < FB; ++q)
        if (p0 + q < nseg && p0 + q != seg)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int b = 0; b < NT; ++b)
              v[q][rb][b] = __builtin_bit_cast(
                  f32x4, __builtin_amdgcn_raw_buffer_load_b128(slots, off(p0 + q, rb, b), 0, kDeviceScope));
#pragma unroll
      for (int q = 0; q < FB; ++q) {
        const int p = p0 + q;
        if (p < nseg)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int b = 0; b < NT; ++b) {
              const f32x4 x = p == seg ? acc[rb][b] : v[q][rb][b];
              sum[rb][b] = p == 0 ? x : sum[rb][b] + x;
            }
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int b = 0; b < NT; ++b) acc[rb][b] = sum[rb][b];
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int b = 0; b < NT; ++b) {
      f32x4 v = acc[rb][b];
      const int tok = b * 16 + r16;
      if constexpr (GU) {
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = __shfl_xor(v[i], 32);
        const int ch = (blk0 + rb) * 8 + 4 * g;   // four channels ch .. ch+3 (lanes g < 2)
        if (g < 2 && tok < M && ch < N) {
          float a[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float gv = v[i], uv = o[i];
            if constexpr (WB) {
              gv *= s0[ch + i];
              uv *= s1[ch + i];
            }
            a[i] = silu(gv) * uv;
          }
          const u32x2 packed = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + (int64_t)tok * ldo + ch) = packed;
        }
      } else {
        const int f = (blk0 + rb) * 16 + 4 * g;   // rows f .. f+3
        if (tok < M && f < N) {
          if constexpr (WB) {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] *= s0[f + i];
          }
          store_out4<OBF>(out, (int64_t)tok * ldo + f, v);
        }
      }
    }
}

// Split-K streams: which token counts take them, their shape (W waves of
// RB row blocks, D steps in flight) and their grid: tiles of 16 * W * RB
// weight rows, K cut into nseg balanced ranges so that about kSkWgs
// workgroups run, with ranges of at most 64 steps; the kernel is compiled
// for ranges of up to 32 and up to 64 steps (nstep).
//
// Measured on the 70B TP = 8 shard (whole forward, packed weights, six
// rotating weight sets): 64 tokens 53.4 -> 48.6 us against the rings, 48
// tokens 44.7 -> 44.5, 32 tokens 38.5 -> 41.9; fp8 at TP = 4, 32 tokens
// 52.0 -> 44.5.  So they take bf16 weights at 49-64 tokens and one-byte
// weights at 17-32.  The workgroup target is one per CU: a CU that holds two
// finishes last (gate/up at 64 tokens in 128-row tiles: 56 tiles x 4 ranges
// = 224 workgroups 28.3 us, x 5 = 280 workgroups 47.6 us, x 9 = 504 33.6
// us; in 112-row tiles, 64 x 4 = 256 workgroups, 29.2 -> 28.3 us on one
// box against the 128-row tiles), and more ranges
// cost more range sums (a round trip through memory each) and shorter
// streams.  Pipelines of 12 or 16 steps instead of 8 measured no faster.  For the same reason they lose on a narrow output
// such as the attention block's QKV projection (1280 rows: 10 tiles, 22
// ranges of 11-12 steps): 13.2 us plus a 2 us finishing kernel on the
// rings (then a separate launch) against 26.3 us at 64 tokens.
template <int NT, int WB>
constexpr bool kSkStream = WB ? NT == 2 : NT == 4;

// Tiles: gate/up seven waves of one 16-row block (112 rows = 56 channels),
// so the 70B shards' gate/up rows (7168 and 14336) make whole multiples of
// 64 tiles and their ranges fill the 256 CUs; the down projection eight
// waves of one block (128 rows; against four waves of two blocks the decode
// step at 8192 x 3584 went 4.30 -> 4.33 TB/s, the fp8 down at 32 tokens
// 16.8-17.2 -> 16.1-16.4 us).  Wider tiles, so that each activation fragment
// serves more rows, measured slower at 64 tokens (70B TP = 8, gate/up 26.8
// us: 14 waves 30.6, 7 waves of two blocks 31.2; down: 256-row tiles 17.8
// and 18.1 against 18.1 us for the M = 64 launch), and so did 64-row down
// tiles (two ranges of 56 steps): the longer tiles need more, shorter
// ranges, the shorter ones reread the activations more often.
template <int NT, int WB, bool GU>
struct SkPlan {
  static constexpr int W = GU ? 7 : 8;
  static constexpr int RB = 1;
  static constexpr int D = 8;
  static constexpr int ROWS = 16 * W * RB;
};
constexpr int kSkWgs = 256;

struct SkGrid {
  int tiles, nseg, nstep;
};

template <int NT, int WB, bool GU>
SkGrid sk_grid(int N, int K) {
  using P = SkPlan<NT, WB, GU>;
  const int rows = P::ROWS;
  const int tiles = GU ? (2 * N + rows - 1) / rows : (N + rows - 1) / rows;
  const int nsteps = K / (WB ? 64 : 32);
  int nseg = max(1, (kSkWgs + tiles / 2) / tiles);
  nseg = min(max(nseg, (nsteps + 63) / 64), nsteps);
  const int longest = (nsteps + nseg - 1) / nseg;
  return SkGrid{tiles, nseg, longest <= 32 ? 32 : 64};
}

template <int NT, int WB, bool GU>
int64_t sk_part_bytes(const SkGrid& g) {
  using P = SkPlan<NT, WB, GU>;
  return g.nseg > 1 ? (int64_t)g.tiles * g.nseg * kSkSlot<NT, P::RB, P::W> : 0;
}

inline int64_t sk_cnt_bytes(int tiles) { return ((int64_t)tiles * 4 + 255) / 256 * 256; }

// One split-K GEMM.  scratch: arrival counters (zero) then the range slots.
template <int NT, int WB, bool GU, bool OBF>
hipError_t sk_launch(int kind, int M, int N, int K, const XRows& xr, const void* w0, const void* w1, int64_t ldw,
                     const float* s0, const float* s1, void* out, int64_t ldo, bool packed, void* scratch,
                     int cnt_tiles, hipStream_t stream) {
  using P = SkPlan<NT, WB, GU>;
  const SkGrid gr = sk_grid<NT, WB, GU>(N, K);
  int* cnt = static_cast<int*>(scratch);
  float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(scratch) + sk_cnt_bytes(cnt_tiles));
  const dim3 grid(gr.tiles, gr.nseg), block(P::W * 64);
  auto go = [&](auto kern) {
    return launch(kind, kern, grid, block, 0, stream, M, N, K, xr, (const uint8_t*)w0, (const uint8_t*)w1, ldw, s0,
                  s1, out, ldo, gr.nseg, part, cnt);
  };
  if (gr.nstep == 32)
    return packed ? go(sk_stream_kernel<NT, P::RB, P::W, WB, P::D, 32, true, GU, OBF>)
                  : go(sk_stream_kernel<NT, P::RB, P::W, WB, P::D, 32, false, GU, OBF>);
  return packed ? go(sk_stream_kernel<NT, P::RB, P::W, WB, P::D, 64, true, GU, OBF>)
                : go(sk_stream_kernel<NT, P::RB, P::W, WB, P::D, 64, false, GU, OBF>);
}

template <int NT, int WB>
int64_t forward_sk_bytes(int h, int I_s) {
  const SkGrid g1 = sk_grid<NT, WB, true>(I_s, h), g2 = sk_grid<NT, WB, false>(h, I_s);
  const int64_t part = max(sk_part_bytes<NT, WB, true>(g1), sk_part_bytes<NT, WB, false>(g2));
  return part ? sk_cnt_bytes(max(g1.tiles, g2.tiles)) + part : 0;
}

// The forward on the split-K streams: clear the counters, gate/up, down.
// Both GEMMs use the same counters (each range that finishes a tile sets
// its counter back to zero) and the same range slots.
template <int NT, int WB>
hipError_t forward_sk(const ShardArgs& a, hipStream_t stream) {
  const SkGrid g1 = sk_grid<NT, WB, true>(a.I_s, a.h), g2 = sk_grid<NT, WB, false>(a.h, a.I_s);
  const int ct = max(g1.tiles, g2.tiles);
  if (g1.nseg > 1 || g2.nseg > 1) {
    const hipError_t e = launch_counter_clear(static_cast<int*>(a.sk), ct, stream);
    if (e != hipSuccess) return e;
  }
  hipError_t e = sk_launch<NT, WB, true, false>(K_GATEUP_DECODE, a.M, a.I_s, a.h, a.x, a.wg, a.wu, a.ldw_gu, a.sg,
                                                a.su, a.a, a.lda, a.packed, a.sk, ct, stream);
  if (e != hipSuccess) return e;
  XRows ax{};
  ax.p[0] = a.a;
  ax.nb = 1;
  ax.rows = a.M;
  ax.ld = a.lda;
  return sk_launch<NT, WB, false, false>(K_DOWN_DECODE, a.M, a.h, a.I_s, ax, a.wd, nullptr, a.ldw_down, a.sd,
                                         nullptr, a.p, a.ldp, a.packed, a.sk, ct, stream);
}

// Whether the forward takes the split-K streams (M tokens, weight format
// wb), and its scratch bytes (0 if it does not or needs none).
template <int WB>
int64_t forward_sk_bytes_wb(int M, int h, int I_s) {
  if (h % (WB ? 64 : 32) || I_s % (WB ? 64 : 32)) return -1;
  switch ((M + 15) / 16) {
    case 2: return kSkStream<2, WB> ? forward_sk_bytes<2, WB>(h, I_s) : -1;
    case 3: return kSkStream<3, WB> ? forward_sk_bytes<3, WB>(h, I_s) : -1;
    case 4: return kSkStream<4, WB> ? forward_sk_bytes<4, WB>(h, I_s) : -1;
    default: return -1;
  }
}

template <int WB>
hipError_t forward_sk_wb(const ShardArgs& a, hipStream_t stream) {
  switch ((a.M + 15) / 16) {
    case 2: if constexpr (kSkStream<2, WB>) return forward_sk<2, WB>(a, stream); break;
    case 3: if constexpr (kSkStream<3, WB>) return forward_sk<3, WB>(a, stream); break;
    case 4: if constexpr (kSkStream<4, WB>) return forward_sk<4, WB>(a, stream); break;
    default: break;
  }
  return hipErrorInvalidValue;
}

// Launch shape (waves per workgroup splitting K; steps per register batch).
constexpr int kWaves = 4;
constexpr int kUnroll = 8;

template <int NT, int WB>
hipError_t gateup_v1(const ShardArgs& a, hipStream_t stream) {
  // Row blocks per workgroup: with more token blocks, two weight blocks share
  // each activation fragment load.  Batches shrink as fragments per step grow.
  constexpr int RB = NT >= 3 ? 2 : 1;
  constexpr int UN = WB ? (NT >= 3 ? kUnroll / 4 : kUnroll / 2) : (NT >= 3 ? kUnroll / 2 : kUnroll);
  return launch(K_GATEUP_DECODE, gateup_decode_kernel<NT, RB, kWaves, UN, WB>,
                dim3((a.I_s + 8 * RB - 1) / (8 * RB)), dim3(kWaves * 64), 0, stream, a.M, a.h, a.I_s, a.x,
                (const uint8_t*)a.wg, (const uint8_t*)a.wu, a.ldw_gu, a.sg, a.su, (uint16_t*)a.a, a.lda);
}

template <int NT, int WB, bool OBF>
hipError_t rowgemm_v1(const RowGemm& g, hipStream_t stream) {
  constexpr int UN = WB ? (NT >= 3 ? kUnroll / 4 : kUnroll / 2) : (NT >= 3 ? kUnroll / 2 : kUnroll);
  return launch(g.kind_decode, down_decode_kernel<NT, 1, kWaves, UN, WB, OBF>, dim3((g.N + 15) / 16),
                dim3(kWaves * 64), 0, stream, g.M, g.N, g.K, (const uint16_t*)g.a, g.lda,
                (const uint8_t*)g.w, g.ldw, g.s, g.out, g.ldo);
}

// Row blocks per wave of the activation-staged streams: two (bf16 weights),
// four for the one-byte gate/up and two for the one-byte down projection.
constexpr int kRbWide = 2;
constexpr int kRbXdByteGu = 4;
constexpr int kRbXdByteDn = 2;

// One-byte weights put 256 k in a slot, so up to 16 tokens their activation
// fragments per weight byte are twice bf16's; two row blocks per wave share
// them in gate/up (measured: fp8 M = 8 32.0 -> 26.0 us, int8 59.9 -> 55.4 us
// at the 70B TP = 4 / TP = 2 shards; the down projection, with a quarter of
// the rows, kept one).
constexpr int kRbNt1Byte = 2;

// bf16 weights, up to 16 tokens: the activation fragments of a slot are
// M x 256 bytes against 4 KB of weights per row block, so from about 8
// tokens two row blocks per wave pay for their halved workgroup count.
// Measured on the 70B TP = 8 shard (whole forward, packed weights): gate/up
// with two blocks 1 token 33.6 -> 34.2 us, 4: 33.9 -> 34.4, 8: 35.0 -> 34.7,
// 12: 37.7 -> 35.4, 16: 42.0 -> 36.8; the down projection as well, over
// that: 12 tokens 35.5 -> 35.4, 16: 36.8 -> 35.8, 8: 34.7 -> 35.2.
constexpr int kRb2MinMGateUp = 8;
constexpr int kRb2MinMDown = 13;

// Up to 16 tokens: one 16-row block per wave, activations from registers
// (most workgroups).  More tokens: RB row blocks per wave share each
// activation fragment, and the activations come through the ring (where its
// slots fit the LDS: fp8 weights have twice the k per slot).
template <int NT, int WB>
constexpr bool kStreamXD = NT >= 2 && (!WB || NT == 2);

template <int NT, int WB, int RB>
hipError_t gateup_stream_rb(const ShardArgs& a, hipStream_t stream) {
  constexpr bool XD = kStreamXD<NT, WB>;
  const dim3 grid((a.I_s + 8 * RB - 1) / (8 * RB)), block(StreamShape<NT, RB, WB, XD>::WV * 64);
  if (a.packed)
    return launch(K_GATEUP_DECODE, gateup_stream_kernel<NT, RB, WB, XD, true>, grid, block, 0, stream, a.M, a.h,
                  a.I_s, a.x, (const uint8_t*)a.wg, (const uint8_t*)a.wu, a.ldw_gu, a.sg, a.su, (uint16_t*)a.a,
                  a.lda);
  return launch(K_GATEUP_DECODE, gateup_stream_kernel<NT, RB, WB, XD, false>, grid, block, 0, stream, a.M, a.h,
                a.I_s, a.x, (const uint8_t*)a.wg, (const uint8_t*)a.wu, a.ldw_gu, a.sg, a.su, (uint16_t*)a.a, a.lda);
}

template <int NT, int WB>
hipError_t gateup_stream(const ShardArgs& a, hipStream_t stream) {
  if constexpr (NT == 1 && !WB) {
    if (a.M >= kRb2MinMGateUp) return gateup_stream_rb<1, WB, 2>(a, stream);
    return gateup_stream_rb<1, WB, 1>(a, stream);
  } else {
    constexpr int RB = NT == 1 ? kRbNt1Byte : (kStreamXD<NT, WB> && WB ? kRbXdByteGu : kRbWide);
    return gateup_stream_rb<NT, WB, RB>(a, stream);
  }
}

template <int NT, int WB>
constexpr int kRowRB = NT == 1 ? 1 : (kStreamXD<NT, WB> && WB ? kRbXdByteDn : kRbWide);

// A narrow row GEMM that splits K (below) runs three 16-row blocks per wave
// on the bf16 activation-staged path instead of two: each staged activation
// fragment serves 48 rows, and the split keeps the workgroup count up.
// Measured on the 70B TP = 8 QKV projection (1280 rows): M = 64 17.3 ->
// 13.4 us, M = 32 13.0 -> 10.7 us; the wide outputs (MLP, o_proj) are
// faster with two.
template <int NT, int WB>
constexpr int kRowRBSplit = kStreamXD<NT, WB> && !WB ? 3 : kRowRB<NT, WB>;

// K split of a streaming row GEMM.  A narrow output (few 16-row blocks, e.g.
// a rank's QKV projection: 80 blocks for 1280 rows) keeps too few loads in
// flight across the chip; its K slots are then split into nseg contiguous
// ranges over a second grid dimension (the range that finishes a tile last
// adds its ranges: a clear of the arrival counters, then one launch), aiming
// at about four waves per CU, with each wave keeping at least two slots.  (Sixteen waves per row block instead of a
// split was measured slower: per-CU streaming rate, not wave count, is the
// limit.)
constexpr int kSplitTargetWaves = 1024;

template <int NT, int WB, int RB = kRowRBSplit<NT, WB>>
int stream_splits(int N, int K) {
  constexpr int WV = StreamShape<NT, RB, WB, kStreamXD<NT, WB>>::WV;
  const int blocks = (N + 16 * RB - 1) / (16 * RB);
  const int want = (kSplitTargetWaves + blocks * WV - 1) / (blocks * WV);
  const int cap = K / (WB ? 256 : 128) / (2 * WV);
  return max(1, min(want, cap));
}

// Split scratch of a streaming row GEMM with nseg > 1 ranges: one arrival
// counter per tile (256-byte rounded), then RB x NT KB per tile and range.
template <int NT, int RB>
constexpr int64_t split_cnt_bytes(int tiles) { return ((int64_t)tiles * 4 + 255) / 256 * 256; }

template <int NT, int RB, int WB, bool OBF>
hipError_t rowgemm_stream_launch(const RowGemm& g, int nseg, hipStream_t stream) {
  constexpr bool XD = kStreamXD<NT, WB>;
  const int tiles = (g.N + 16 * RB - 1) / (16 * RB);
  const dim3 grid(tiles, nseg), block(StreamShape<NT, RB, WB, XD>::WV * 64);
  const uint16_t* a = (const uint16_t*)g.a;
  const uint8_t* w = (const uint8_t*)g.w;
  if (nseg > 1) {
    int* cnt = reinterpret_cast<int*>(g.ws);
    float* part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(g.ws) + split_cnt_bytes<NT, RB>(tiles));
    const hipError_t e = launch_counter_clear(cnt, tiles, stream);
    if (e != hipSuccess) return e;
    if (g.packed)
      return launch(g.kind_decode, down_stream_kernel<NT, RB, WB, XD, OBF, true, true>, grid, block, 0, stream, g.M,
                    g.N, g.K, a, g.lda, w, g.ldw, g.s, g.out, g.ldo, nseg, part, cnt);
    return launch(g.kind_decode, down_stream_kernel<NT, RB, WB, XD, OBF, false, true>, grid, block, 0, stream, g.M,
                  g.N, g.K, a, g.lda, w, g.ldw, g.s, g.out, g.ldo, nseg, part, cnt);
  }
  if (g.packed)
    return launch(g.kind_decode, down_stream_kernel<NT, RB, WB, XD, OBF, true, false>, grid, block, 0, stream, g.M,
                  g.N, g.K, a, g.lda, w, g.ldw, g.s, g.out, g.ldo, 1, (float*)nullptr, (int*)nullptr);
  return launch(g.kind_decode, down_stream_kernel<NT, RB, WB, XD, OBF, false, false>, grid, block, 0, stream, g.M,
                g.N, g.K, a, g.lda, w, g.ldw, g.s, g.out, g.ldo, 1, (float*)nullptr, (int*)nullptr);
}

template <int NT, int WB, bool OBF>
hipError_t rowgemm_stream(const RowGemm& g, hipStream_t stream) {
  // nseg is planned for kRowRBSplit row blocks per wave; when it comes out 1
  // the output is wide enough for kRowRB without a split (kRowRB's larger
  // block count would not split either).
  const int nseg = g.ws ? stream_splits<NT, WB>(g.N, g.K) : 1;
  if constexpr (NT == 1 && !WB) {
    if (nseg == 1 && g.M >= kRb2MinMDown) return rowgemm_stream_launch<1, 2, WB, OBF>(g, 1, stream);
  }
  if (nseg == 1) return rowgemm_stream_launch<NT, kRowRB<NT, WB>, WB, OBF>(g, 1, stream);
  return rowgemm_stream_launch<NT, kRowRBSplit<NT, WB>, WB, OBF>(g, nseg, stream);
}

// The streaming kernels move whole 16-row x 256-byte slots along K: they need
// K to be a multiple of 128 (bf16) / 256 (fp8) k-values; other shapes use the
// register-batch kernels, which step 32 / 64 k-values at a time.
template <int WB>
constexpr bool streams(int K) {
  return K % (WB ? 256 : 128) == 0;
}

template <int WB>
hipError_t run_gateup(const ShardArgs& a, hipStream_t stream) {
  const bool st = streams<WB>(a.h);
  if (a.packed && !st) return hipErrorInvalidValue;   // packed weights are read by the streams only
  switch ((a.M + 15) / 16) {
    case 1: return st ? gateup_stream<1, WB>(a, stream) : gateup_v1<1, WB>(a, stream);
    case 2: return st ? gateup_stream<2, WB>(a, stream) : gateup_v1<2, WB>(a, stream);
    case 3: return st ? gateup_stream<3, WB>(a, stream) : gateup_v1<3, WB>(a, stream);
    case 4: return st ? gateup_stream<4, WB>(a, stream) : gateup_v1<4, WB>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int WB, bool OBF>
hipError_t run_rowgemm(const RowGemm& g, hipStream_t stream) {
  const bool st = streams<WB>(g.K);
  if (g.packed && !st) return hipErrorInvalidValue;
  switch ((g.M + 15) / 16) {
    case 1: return st ? rowgemm_stream<1, WB, OBF>(g, stream) : rowgemm_v1<1, WB, OBF>(g, stream);
    case 2: return st ? rowgemm_stream<2, WB, OBF>(g, stream) : rowgemm_v1<2, WB, OBF>(g, stream);
    case 3: return st ? rowgemm_stream<3, WB, OBF>(g, stream) : rowgemm_v1<3, WB, OBF>(g, stream);
    case 4: return st ? rowgemm_stream<4, WB, OBF>(g, stream) : rowgemm_v1<4, WB, OBF>(g, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

namespace {

template <int NT, int WB>
int64_t workspace_bytes_nt(int M, int N, int K) {
  constexpr int RB = kRowRBSplit<NT, WB>;
  const int nseg = stream_splits<NT, WB>(N, K);
  if (nseg == 1) return 0;
  const int tiles = (N + 16 * RB - 1) / (16 * RB);
  return split_cnt_bytes<NT, RB>(tiles) + (int64_t)tiles * nseg * RB * NT * 1024;
}

template <int WB>
int64_t workspace_bytes_wb(int M, int N, int K) {
  if (!streams<WB>(K)) return 0;
  switch ((M + 15) / 16) {
    case 1: return workspace_bytes_nt<1, WB>(M, N, K);
    case 2: return workspace_bytes_nt<2, WB>(M, N, K);
    case 3: return workspace_bytes_nt<3, WB>(M, N, K);
    default: return workspace_bytes_nt<4, WB>(M, N, K);
  }
}

template <int WB>
hipError_t rowgemm_wb(const RowGemm& g, hipStream_t stream) {
  return g.out_bf16 ? run_rowgemm<WB, true>(g, stream) : run_rowgemm<WB, false>(g, stream);
}

}  // namespace

// A narrow row GEMM that the matrix-core stream would split along K (the
// QKV projection) goes, at up to kGemvMaxM tokens with bf16 weights, to the
// row-streaming VALU kernel of gemv.hip: no split and no arrival counters.
static bool use_gemv(int M, int N, int K, int wb) {
  return gemv_supported(M, K, wb) && stream_splits<1, kWeightWide>(N, K) > 1;
}

int64_t rowgemm_decode_workspace_bytes(int M, int N, int K, int wb) {
  if (M < 1 || M > kDecodeMaxM || use_gemv(M, N, K, wb)) return 0;
  switch (wb) {
    case kWeightE4M3: return workspace_bytes_wb<kWeightE4M3>(M, N, K);
    case kWeightI8: return workspace_bytes_wb<kWeightI8>(M, N, K);
    default: return workspace_bytes_wb<kWeightWide>(M, N, K);
  }
}

hipError_t launch_rowgemm_decode(const RowGemm& g, hipStream_t stream) {
  if (!g.packed && use_gemv(g.M, g.N, g.K, g.wb)) return launch_rowgemm_gemv(g, stream);
  switch (g.wb) {
    case kWeightE4M3: return rowgemm_wb<kWeightE4M3>(g, stream);
    case kWeightI8: return rowgemm_wb<kWeightI8>(g, stream);
    default: return rowgemm_wb<kWeightWide>(g, stream);
  }
}

// Split-K scratch of the decode forward (-1: the forward does not take the
// split-K streams).
static int64_t forward_sk_need(int M, int h, int I_s, int wb) {
  if (M < 1 || M > kDecodeMaxM) return -1;
  switch (wb) {
    case kWeightE4M3: return forward_sk_bytes_wb<kWeightE4M3>(M, h, I_s);
    case kWeightI8: return forward_sk_bytes_wb<kWeightI8>(M, h, I_s);
    default: return forward_sk_bytes_wb<kWeightWide>(M, h, I_s);
  }
}

int64_t forward_decode_sk_bytes(int M, int h, int I_s, int wb) { return max((int64_t)0, forward_sk_need(M, h, I_s, wb)); }

hipError_t launch_forward_decode(const ShardArgs& a, hipStream_t stream) {
  const int64_t skb = forward_sk_need(a.M, a.h, a.I_s, a.wb);
  if (skb >= 0 && (skb == 0 || a.sk)) {
    switch (a.wb) {
      case kWeightE4M3: return forward_sk_wb<kWeightE4M3>(a, stream);
      case kWeightI8: return forward_sk_wb<kWeightI8>(a, stream);
      default: return forward_sk_wb<kWeightWide>(a, stream);
    }
  }
  hipError_t e;
  switch (a.wb) {
    case kWeightE4M3: e = run_gateup<kWeightE4M3>(a, stream); break;
    case kWeightI8: e = run_gateup<kWeightI8>(a, stream); break;
    default: e = run_gateup<kWeightWide>(a, stream); break;
  }
  if (e != hipSuccess) return e;
  return launch_rowgemm_decode(down_of(a), stream);
}

// ---------------------------------------------------------------- packed weights
// The streams read each 16-row block of W slot by slot (256 bytes of each of
// the 16 rows per slot), which in the (out, in) layout is 16 pieces 16 KB
// apart (70B shard); a read pattern like that runs at about 4.9 TB/s on
// MI355X against 6.3 TB/s for the same bytes read in address order.  The
// packed array stores every 16-row block as its run of 1 KB MFMA A fragments
// (packed_frag above), block after block, so each block streams one
// contiguous range.  Gate/up blocks hold 8 gate rows then the same 8
// channels' up rows; rows past the end repeat the last row, as the row-major
// streams clamp.

namespace {

// One thread per 16 bytes of the packed array (blocks x nsteps fragments);
// GU: rows 0-7 of block blk from w0 (channels 8 blk + r), 8-15 from w1.
template <bool GU>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ w0, const uint8_t* __restrict__ w1,
                                                   int64_t ld_bytes, int nrows, int nsteps, int64_t nchunks,
                                                   uint8_t* __restrict__ out) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= nchunks) return;
  const int64_t blk = q / ((int64_t)nsteps * 64);
  const int within = (int)(q - blk * nsteps * 64);
  const int st = within >> 6, lane = within & 63;   // fragment st of the block, lane
  const int row = lane & 15;
  const uint8_t* src;
  if constexpr (GU)
    src = (row < 8 ? w0 : w1) + min(8 * blk + (row & 7), (int64_t)nrows - 1) * ld_bytes;
  else
    src = w0 + min(16 * blk + row, (int64_t)nrows - 1) * ld_bytes;
  *reinterpret_cast<u32x4*>(out + q * 16) = *reinterpret_cast<const u32x4*>(src + (int64_t)st * 64 + (lane >> 4) * 16);
}

}  // namespace

bool decode_packable(int h, int I_s, int wb) {
  const int ks = wb ? 256 : 128;
  return h % ks == 0 && I_s % ks == 0;
}

// One fragment (1 KB) per 64 weight bytes of a block's rows.
int64_t packed_gateup_bytes(int h, int I_s, int wb) {
  return (int64_t)((I_s + 7) / 8) * (h * (wb ? 1 : 2) / 64) * 1024;
}

int64_t packed_down_bytes(int h, int I_s, int wb) {
  return (int64_t)((h + 15) / 16) * (I_s * (wb ? 1 : 2) / 64) * 1024;
}

hipError_t launch_pack_weights(const ShardArgs& a, void* packed, hipStream_t stream) {
  const int eb = a.wb ? 1 : 2;
  uint8_t* gu = static_cast<uint8_t*>(packed);
  uint8_t* dn = gu + packed_gateup_bytes(a.h, a.I_s, a.wb);
  const int64_t c_gu = packed_gateup_bytes(a.h, a.I_s, a.wb) / 16, c_dn = packed_down_bytes(a.h, a.I_s, a.wb) / 16;
  hipError_t e = launch(-1, pack_kernel<true>, dim3((unsigned)((c_gu + 255) / 256)), dim3(256), 0, stream,
                        (const uint8_t*)a.wg, (const uint8_t*)a.wu, a.ldw_gu * eb, a.I_s, a.h * eb / 64, c_gu, gu);
  if (e != hipSuccess) return e;
  return launch(-1, pack_kernel<false>, dim3((unsigned)((c_dn + 255) / 256)), dim3(256), 0, stream,
                (const uint8_t*)a.wd, (const uint8_t*)nullptr, a.ldw_down * eb, a.h, a.I_s * eb / 64, c_dn, dn);
}

}  // namespace tpmlp
