// Internal interface between the C ABI layer (abi.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

// Kernel kinds for the timing record (kept in sync with kKindNames in abi.cpp).
enum KernelKind : int {
  K_GATEUP_DECODE = 0,
  K_DOWN_DECODE = 1,
  K_GATEUP_PREFILL = 2,
  K_DOWN_PREFILL = 3,
  K_PARTIAL_REDUCE = 4,
  K_GATEUP_F32 = 5,
  K_DOWN_F32 = 6,
  K_QKV_DECODE = 7,
  K_QKV_PREFILL = 8,
  K_OPROJ_DECODE = 9,
  K_OPROJ_PREFILL = 10,
  K_QKV_F32 = 11,
  K_OPROJ_F32 = 12,
  K_QUANT_ROWS = 13,
  K_GATEUP_W8A8 = 14,
  K_DOWN_W8A8 = 15,
  K_SK_CLEAR = 16,
  K_NUM_KINDS = 17
};

constexpr int kMaxPartials = 64;

// Weight storage formats of the bf16-activation kernels: 2-byte bf16, or one
// byte per weight with an fp32 scale per output row (e4m3fn codes or int8).
constexpr int kWeightWide = 0;
constexpr int kWeightE4M3 = 1;
constexpr int kWeightI8 = 2;

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
  int wb;                   // weight format: kWeightWide / kWeightE4M3 / kWeightI8
  void* sk;                 // prefill stream-K scratch (forward_prefill_sk_bytes), or null
  bool packed = false;      // decode only: wg = packed gate/up array, wd = packed down array
};

// out (M x N) = A (M x K) * W^T with W (N x K, (out, in) layout), fp32
// accumulation, fp8 W scaled per output row, out fp32 or bf16: the down
// projection of the MLP and the attention block's projections.
struct RowGemm {
  int M, N, K;
  const void* a;            // M x K, bf16 (fp32 on the fp32 path)
  int64_t lda;
  const void* w;            // N x K, bf16 / fp8 codes / fp32
  int64_t ldw;
  const float* s;           // fp8 only: N per-row scales
  void* out;                // M x N
  int64_t ldo;
  bool out_bf16;            // else fp32
  int wb;                   // weight format (kWeight*)
  float* ws;                // decode: split-K sums; prefill: stream-K scratch (null: neither), 256-byte aligned
  int kind_decode, kind_prefill, kind_f32;  // timing kinds of the three paths
  bool packed = false;      // decode streams only: w is a packed array
};

// Packed decode weights (decode.hip): both GEMMs' K a multiple of the
// streams' slot (128 k bf16, 256 k one-byte); the gate/up array, then the
// down array; one pass of pack kernels from the (out, in) weights.
bool decode_packable(int h, int I_s, int wb);
int64_t packed_gateup_bytes(int h, int I_s, int wb);
int64_t packed_down_bytes(int h, int I_s, int wb);
hipError_t launch_pack_weights(const ShardArgs& a, void* packed, hipStream_t stream);

// Largest M served by the weight-streaming (decode) kernels.
constexpr int kDecodeMaxM = 64;
// ... in the MLP forward: with one-byte weights the streams stage the
// activations through LDS up to 32 tokens only, and beyond that the 64-token
// prefill tiles are faster (70B shard, fp8, TP = 4: 48 tokens 88 -> 82 us,
// 64 tokens 113 -> 84 us; the same at 33 tokens: 73 against 79).
inline int forward_decode_max_m(int wb) { return wb == kWeightWide ? kDecodeMaxM : 32; }
// Largest M served by the row-streaming VALU kernel (gemv.hip), bf16 weights.
constexpr int kGemvMaxM = 2;

hipError_t launch_partial_reduce(const PartialPtrs& ptrs, int t, float* out, int64_t n,
                                 hipStream_t stream);
// The MLP's down projection of a shard: partial (M x h fp32) = a (M x I_s) * wd^T.
inline RowGemm down_of(const ShardArgs& s) {
  RowGemm g;
  g.M = s.M; g.N = s.h; g.K = s.I_s;
  g.a = s.a; g.lda = s.lda;
  g.w = s.wd; g.ldw = s.ldw_down; g.s = s.sd;
  g.out = s.p; g.ldo = s.ldp;
  g.out_bf16 = false; g.wb = s.wb; g.ws = nullptr; g.packed = s.packed;
  g.kind_decode = K_DOWN_DECODE; g.kind_prefill = K_DOWN_PREFILL; g.kind_f32 = K_DOWN_F32;
  return g;
}

// Scratch of the fp8 x fp8 forward beyond A (a.a): the activations' e4m3fn
// codes and per-token scales, and the same for A.
struct W8A8Bufs {
  void* xq;                 // M x h codes
  float* sx;                // M
  void* aq;                 // M x I_s codes
  float* sa;                // M
};

hipError_t launch_forward_decode(const ShardArgs& a, hipStream_t stream);
// Split-K scratch of a decode forward (a.sk; 0: none needed).
int64_t forward_decode_sk_bytes(int M, int h, int I_s, int wb);
// Zero n arrival counters (one workgroup).
hipError_t launch_counter_clear(int* cnt, int n, hipStream_t stream);
hipError_t launch_forward_prefill(const ShardArgs& a, hipStream_t stream);
hipError_t launch_forward_f32(const ShardArgs& a, hipStream_t stream);
hipError_t launch_rowgemm_decode(const RowGemm& g, hipStream_t stream);
// Split-K scratch bytes launch_rowgemm_decode uses for this shape (0: none).
int64_t rowgemm_decode_workspace_bytes(int M, int N, int K, int wb);
// Stream-K scratch bytes launch_rowgemm_prefill uses for this shape (0: none).
int64_t rowgemm_prefill_workspace_bytes(int M, int N, int K);
// Stream-K scratch of a prefill forward's two GEMMs (they run one after the
// other and share it); a8: the fp8 x fp8 forward.
int64_t forward_prefill_sk_bytes(int M, int h, int I_s, bool a8);
// Stream-K scratch of the packed-weight prefill forward (bf16, 256-token tiles).
int64_t forward_prefill_packed_sk_bytes(int M, int h, int I_s);
hipError_t launch_rowgemm_prefill(const RowGemm& g, hipStream_t stream);
// Row-streaming VALU row GEMM (M <= kGemvMaxM, bf16 weights, K a multiple of
// 512 up to 16384): whether it can take this shape, and the launch.
bool gemv_supported(int M, int K, int wb);
hipError_t launch_rowgemm_gemv(const RowGemm& g, hipStream_t stream);
hipError_t launch_rowgemm_f32(const RowGemm& g, hipStream_t stream);
// rows x K bf16 -> e4m3fn codes (ldq bytes per row) and one fp32 scale per row.
hipError_t launch_quant_rows(int M, int K, const void* x, int64_t ldx, void* q, int64_t ldq, float* scales,
                             hipStream_t stream);
// The fp8 x fp8 forward (contiguous X, e4m3fn weights with row scales).
hipError_t launch_forward_w8a8(const ShardArgs& a, const W8A8Bufs& b, hipStream_t stream);

}  // namespace tpmlp
