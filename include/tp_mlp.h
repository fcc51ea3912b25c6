/*
 * tp_mlp.h -- C ABI of the MI355X (gfx950) tensor-parallel MLP shard library.
 *
 * One tensor-parallel rank's share of a Llama-style MLP under the Megatron
 * split, and the local sum of the t ranks' partial outputs.
 *
 * The operation (sources are web pages; section names given so a reader can
 * find the passage):
 *
 *   - "Build a model sharding system for serving 70B+ parameter models"
 *     (scalablesystem.dev), section "The Tensor-Parallel Shard Group":
 *     gate_proj and up_proj are column-parallel (each rank holds a slice of
 *     the intermediate dimension, weight layout (local_out, in)); down_proj is
 *     row-parallel (weight layout (out, local_in)); each rank's down output is
 *     a partial that an all-reduce sums; out/in features must divide by the
 *     group size.
 *   - "Tensor, Pipeline and Expert Parallelism: One Model, Many GPUs"
 *     (vidyal.ai), section "Step 1: tensor parallelism slices every layer":
 *     the activation is applied locally after the column split; Llama's MLP
 *     adds a second input matrix split the same way.
 *   - "Chapter 12 Parallelism Strategies" (arunshar.com), section 12.2.1:
 *     A = [A_1 | ... | A_t] by columns, B by rows, Z = sum_k Z_k.
 *
 * With S_k = [k*I_s, (k+1)*I_s), I_s = I_full / t, rank k computes
 *
 *     G = X * W_gate_k^T,  U = X * W_up_k^T          (M x I_s, fp32 accumulate)
 *     A = SiLU(G) (.) U,   SiLU(z) = z / (1 + e^-z)   (elementwise)
 *     P_k = A * W_down_k^T                            (M x h, fp32)
 *
 * and tp_partial_reduce computes Y = (((P_0 + P_1) + P_2) + ...) + P_{t-1}
 * elementwise in fp32, always in that order (the pages note that the
 * all-reduce's summation order changes the bits: scalablesystem.dev,
 * "Quality, Evaluation, and Guardrails").
 *
 * Conventions for every entry point:
 *   - All matrices are row-major.  Leading dimensions are in elements.
 *   - Device pointers are HIP device addresses on the current device; the
 *     caller owns every buffer.  The library never allocates, frees or
 *     synchronises device memory on these paths; work is enqueued on `stream`
 *     (a hipStream_t, NULL = the null stream) and the call returns at once.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     any error nothing is launched and a status other than TP_OK is
 *     returned.  tp_last_error() then gives a message (thread-local).
 *   - Nothing is thrown across the ABI.
 */
#ifndef TP_MLP_H
#define TP_MLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TP_F32 = 0,         /* IEEE binary32                                       */
  TP_BF16 = 1,        /* bfloat16 (upper half of binary32)                   */
  TP_FP8_E4M3FN = 2,  /* OCP FP8 E4M3 (bias 7, max 448, no inf); weights only */
  TP_INT8 = 3         /* two's-complement int8 code; weights only            */
} tp_dtype;

typedef enum {
  TP_OK = 0,
  TP_ERR_INVALID_ARG = 1,  /* shapes, indices, pointers inconsistent        */
  TP_ERR_UNSUPPORTED = 2,  /* valid but not implemented (dtype pair, shape
                              alignment, pointer alignment)                 */
  TP_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required    */
  TP_ERR_HIP = 4           /* a HIP runtime call failed (launch, device)    */
} tp_status;

/*
 * Workspace bytes tp_mlp_shard_forward needs for these arguments (0 if the
 * arguments are invalid).  The workspace holds the intermediate activation A
 * (M x I_s, in the activation dtype) plus alignment padding, and
 *  - for a bf16 prefill (M > 64; M > 32 with one-byte weights) whose output
 *    tiles do not fill whole rounds of the 256 CUs, the stream-K scratch of
 *    the two GEMMs: arrival counters and one fp32 tile (256 weight rows by
 *    64, 128 or 256 tokens) per piece of the tiles cut along K (at most 256
 *    pieces, 64 MiB);
 *  - for a decode forward on the split-K streams (bf16 weights and
 *    49 <= M <= 64, one-byte weights and 17 <= M <= 32), arrival counters
 *    and one fp32 slot (112 or 128 weight rows by 16 * ceil(M / 16)
 *    tokens) per tile and K range (about 256 slots, 8 MiB for the 70B
 *    shard at TP = 8).
 */
size_t tp_mlp_workspace_bytes(int64_t M, int64_t h, int64_t I_full, int32_t t,
                              int32_t act_dtype, int32_t w_dtype);

/*
 * Rank k's partial P_k (definition above).
 *
 *   M        tokens (rows of X and P), M >= 1.
 *   h        hidden size, h >= 1.
 *   I_full   full (unsharded) intermediate size; I_full % t == 0.
 *   t, k     TP degree (1..64) and this rank's index (0..t-1).  k selects no
 *            data: the caller passes rank k's shard pointers.  It is
 *            validated, and the result for given shard bytes does not depend
 *            on it.
 *   act_dtype  dtype of X and of the intermediate A: TP_BF16 or TP_F32.
 *   w_dtype    dtype of the three weight shards.  Supported pairs:
 *              (TP_BF16, TP_BF16), (TP_BF16, TP_FP8_E4M3FN),
 *              (TP_BF16, TP_INT8), (TP_F32, TP_F32).  The one-byte formats
 *              are weight-only quantisation ("Build a model sharding system
 *              ...", the planner's bytes per parameter for fp8 and int8):
 *              the codes are widened to bf16 exactly in the kernels and the
 *              activations stay bf16.
 *   x        M x h, leading dimension ldx >= h.
 *   w_gate, w_up   I_s x h each ((out, in) layout: row j is intermediate
 *            channel k*I_s + j of the full matrix), leading dimension
 *            ldw_gu >= h.  A caller holding the full matrix passes the
 *            pointer to row k*I_s.
 *   w_down   h x I_s ((out, in) layout, the rank's column block of the full
 *            W_down), leading dimension ldw_down >= I_s.  A caller holding
 *            the full h x I_full matrix passes the pointer to column k*I_s
 *            and ldw_down = I_full.
 *   s_gate, s_up, s_down   fp32 per-output-channel scales, required for
 *            one-byte weights (TP_FP8_E4M3FN, TP_INT8; lengths I_s, I_s, h;
 *            the dequantised weight is code value * scale of its row) and
 *            must be NULL otherwise.
 *   partial  M x h fp32 output, leading dimension ldp >= h; overwritten.
 *            Must not overlap any input or the workspace.
 *   workspace, workspace_bytes   device scratch of at least
 *            tp_mlp_workspace_bytes(...) bytes, 256-byte aligned; its
 *            contents on entry are ignored.  Concurrent calls must not share
 *            a workspace.
 *   stream   hipStream_t or NULL.
 *
 * Requirements beyond validity (else TP_ERR_UNSUPPORTED): with bf16
 * activations (bf16 or one-byte weights) h % 64 == 0 and I_s % 64 == 0, all tensor
 * pointers 16-byte aligned and every row 16-byte aligned (leading dimension
 * times element size a multiple of 16 bytes), scales 4-byte aligned; with
 * fp32 activations and weights any h and I_s, 4-byte alignment.  The
 * workspace is 256-byte aligned in both cases.
 *
 * Numerics: fp32 accumulation; SiLU and the gate/up product in fp32; A is
 * rounded to the activation dtype (bf16, round-to-nearest-even) before the
 * down projection.  Results are deterministic (no atomics in the sums).
 */
tp_status tp_mlp_shard_forward(int64_t M, int64_t h, int64_t I_full,
                               int32_t t, int32_t k,
                               int32_t act_dtype, int32_t w_dtype,
                               const void* x, int64_t ldx,
                               const void* w_gate, const void* w_up, int64_t ldw_gu,
                               const void* w_down, int64_t ldw_down,
                               const float* s_gate, const float* s_up,
                               const float* s_down,
                               float* partial, int64_t ldp,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * tp_mlp_shard_forward without its workspace argument.  The forward's
 * scratch (the intermediate A and, for a prefill with a stream-K tail or a
 * decode on the split-K streams, their arrival counters and slots) lives in
 * a static device array of TP_NOALLOC_SCRATCH_BYTES bytes, one per device
 * the library runs on, held until the process ends.  The call allocates nothing and calls no
 * allocating routine (its first call on a device looks up that device's
 * array address once).  Every call on a device shares the array and it keeps
 * the last call's contents (the counters are cleared by a kernel of the
 * call itself): calls that overlap in time on one device (several streams
 * or host threads) race and give undefined results; calls on one stream are
 * ordered and safe.  With kernel timing on, only launches with events made
 * beforehand by tp_profile_reserve are timed.
 *
 * Arguments, requirements, errors and results (bit for bit) are those of
 * tp_mlp_shard_forward.  A forward whose tp_mlp_workspace_bytes(...) is
 * larger than TP_NOALLOC_SCRATCH_BYTES returns TP_ERR_UNSUPPORTED and
 * launches nothing (the 70B shard at TP = 8 needs 7 KB per token for A, so a
 * 4096-token prefill fits).
 */
#define TP_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

tp_status tp_mlp_shard_forward_noalloc(int64_t M, int64_t h, int64_t I_full,
                                       int32_t t, int32_t k,
                                       int32_t act_dtype, int32_t w_dtype,
                                       const void* x, int64_t ldx,
                                       const void* w_gate, const void* w_up, int64_t ldw_gu,
                                       const void* w_down, int64_t ldw_down,
                                       const float* s_gate, const float* s_up,
                                       const float* s_down,
                                       float* partial, int64_t ldp, void* stream);

/*
 * out[i] = (((partials[0][i] + partials[1][i]) + partials[2][i]) + ...)
 *          + partials[t-1][i]   for 0 <= i < n, fp32 round-to-nearest-even,
 * no fused operations and no flush of subnormals: bit-exact against that
 * left fold.  This is the sum the all-reduce after the row-parallel
 * projection computes, run locally over t buffers on one device.
 *
 *   n          elements per buffer (n >= 0; n == 0 is a no-op that reads no
 *              pointer, so any of them may then be NULL).
 *   t          number of partials, 1..64.
 *   partials   HOST array of t device pointers, each 16-byte aligned (the
 *              array itself is read during the call only).
 *   out        n fp32, 16-byte aligned.  May be equal to partials[0] (in
 *              place); must not otherwise overlap a partial.
 */
tp_status tp_partial_reduce(int64_t n, int32_t t, const float* const* partials,
                            float* out, void* stream);

/* ------------------------------------------------------------------------
 * Sequence-parallel forms ("Chapter 12 Parallelism Strategies",
 * arunshar.com, section 12.3.1: with sequence parallelism the all-reduce
 * after the row-parallel projection becomes a reduce-scatter, rank k keeping
 * the fully reduced rows of sequence positions [k*s/t, (k+1)*s/t), and the
 * column-parallel projection that follows runs on the all-gathered
 * sequence).  The tokens M play the role of the sequence positions.
 * ---------------------------------------------------------------------- */

/*
 * tp_mlp_shard_forward with the activation given as the t ranks' row blocks
 * instead of one gathered matrix: x_blocks is a HOST array of t device
 * pointers, block j holding rows [j*M/t, (j+1)*M/t) of X (M/t x h, leading
 * dimension ldx).  The kernels read the rows from the blocks in place, so
 * the gathered X is never formed.  Requires M % t == 0; every other argument,
 * requirement and the result (bit for bit) are those of tp_mlp_shard_forward
 * on the row-concatenated X.
 */
tp_status tp_mlp_shard_forward_sp(int64_t M, int64_t h, int64_t I_full,
                                  int32_t t, int32_t k,
                                  int32_t act_dtype, int32_t w_dtype,
                                  const void* const* x_blocks, int64_t ldx,
                                  const void* w_gate, const void* w_up, int64_t ldw_gu,
                                  const void* w_down, int64_t ldw_down,
                                  const float* s_gate, const float* s_up,
                                  const float* s_down,
                                  float* partial, int64_t ldp,
                                  void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * Rank k's share of the reduce-scatter: for the t partials, each `rows` x
 * row_len contiguous fp32 (row-major, no padding), out receives rows
 * [k*rows/t, (k+1)*rows/t) of their left-fold sum, i.e. tp_partial_reduce
 * over the n = rows/t * row_len elements starting at element k*n of every
 * partial (same order, same bits).
 *
 *   rows, row_len   rows % t == 0; rows/t * row_len a multiple of 4 (else
 *              TP_ERR_UNSUPPORTED); a zero count is a no-op.
 *   t, k       1 <= t <= 64, 0 <= k < t.
 *   partials   HOST array of t device pointers (16-byte aligned).
 *   out        rows/t x row_len fp32, 16-byte aligned.  May be rank k's
 *              slice of partials[0] (partials[0] + k*n, in place); must not
 *              otherwise overlap the slices read.
 */
tp_status tp_partial_reduce_scatter(int64_t rows, int64_t row_len, int32_t t, int32_t k,
                                    const float* const* partials, float* out,
                                    void* stream);

/* ------------------------------------------------------------------------
 * fp8 x fp8 (W8A8) forward.  The pages' fp8 mode is one byte per weight
 * ("Build a model sharding system for serving 70B+ parameter models",
 * scalablesystem.dev, the shard planner); quantising the activations too
 * puts both GEMM operands on gfx950's fp8 matrix instructions (twice the
 * bf16 rate) and changes the numerics.  Activation rows are quantised per
 * token:
 *
 *   s_m = amax_m / 448 (fp32; 1 for an all-zero row),
 *   q[m][j] = e4m3fn(x[m][j] / s_m)   (fp32 quotient, nearest code, ties to
 *                                      even, magnitudes >= 448 saturate)
 *
 * and the rank forward becomes: Xq, s_x = quant(X); G, U = (Xq Wq^T) * s_x *
 * s_w (fp32 accumulation); A = SiLU(G) (.) U rounded to bf16; Aq, s_a =
 * quant(A); P_k = (Aq W_down_q^T) * s_a * s_down.  It runs on the MFMA GEMM
 * kernels for every M (meant for prefill; at decode sizes the fp8-weight
 * tp_mlp_shard_forward reads the same weight bytes).
 * ---------------------------------------------------------------------- */

/*
 * Workspace bytes of tp_mlp_shard_forward_w8a8 (0 if the arguments are
 * invalid): A in bf16, the codes of X and A, their per-token scales, and
 * the GEMMs' stream-K scratch as for tp_mlp_shard_forward.
 */
size_t tp_mlp_w8a8_workspace_bytes(int64_t M, int64_t h, int64_t I_full, int32_t t);

/*
 * Rank k's partial with fp8 activations and fp8 (e4m3fn) weights.  Arguments
 * as tp_mlp_shard_forward with act_dtype = TP_BF16 (x is bf16) and w_dtype =
 * TP_FP8_E4M3FN (scales required); contiguous X only.  Requires h % 128 == 0
 * and I_s % 128 == 0 (else TP_ERR_UNSUPPORTED), 16-byte aligned pointers and
 * rows, a 256-byte aligned workspace of tp_mlp_w8a8_workspace_bytes(...)
 * bytes whose contents on entry are ignored.  Deterministic.
 *
 * When the work has completed, the workspace holds the forward's
 * intermediates, each starting at the next multiple of 256 bytes after the
 * previous one (offset 0 first): A (M x I_s bf16), X's codes (M x h bytes),
 * X's scales (M fp32), A's codes (M x I_s bytes), A's scales (M fp32).
 */
tp_status tp_mlp_shard_forward_w8a8(int64_t M, int64_t h, int64_t I_full,
                                    int32_t t, int32_t k,
                                    const void* x, int64_t ldx,
                                    const void* w_gate, const void* w_up, int64_t ldw_gu,
                                    const void* w_down, int64_t ldw_down,
                                    const float* s_gate, const float* s_up,
                                    const float* s_down,
                                    float* partial, int64_t ldp,
                                    void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * The per-token quantisation above on its own: rows x cols bf16 (leading
 * dimension ldx, rows 16-byte aligned) -> e4m3fn codes (leading dimension
 * ldq bytes, rows 8-byte aligned) and one fp32 scale per row.  cols % 8 == 0
 * (else TP_ERR_UNSUPPORTED); rows == 0 is a no-op.  Buffers must not overlap.
 * The rows must be finite: a row holding an infinity or a NaN gets
 * unspecified codes.
 */
tp_status tp_quantize_rows_e4m3(int64_t rows, int64_t cols, const void* x, int64_t ldx,
                                void* codes, int64_t ldq, float* scales, void* stream);

/* ------------------------------------------------------------------------
 * Attention-block projections of one rank.  "Build a model sharding system
 * for serving 70B+ parameter models" (scalablesystem.dev), section "The
 * Tensor-Parallel Shard Group", class TPAttentionBlock: the QKV projection is
 * column-parallel (each rank computes the projections of its own attention
 * heads, no communication), attention runs locally over those heads, and the
 * output projection is row-parallel, its partials summed by an all-reduce.
 * "Chapter 12 Parallelism Strategies" (arunshar.com), section 12.2.1: rank k
 * handles n_heads/t heads.  Grouped-query attention: the KV-head count must
 * divide by the TP degree (scalablesystem.dev, the interview question on
 * uneven division); when the degree is a multiple of the KV-head count, each
 * rank keeps one KV head and the heads are replicated ("Tensor, Pipeline and
 * Expert Parallelism: One Model, Many GPUs", vidyal.ai, section "The KV
 * cache splits too, until it doesn't").
 *
 * With q_loc = n_heads/t and kv_loc = n_kv_heads/t (or 1 when t is a multiple
 * of n_kv_heads), rank k's QKV width is n_loc = (q_loc + 2*kv_loc)*head_dim and
 *
 *     QKV_k = X * W_qkv_k^T      (M x n_loc, fp32 accumulate, stored in the
 *                                 activation dtype: bf16 RNE, or fp32)
 *     P_k   = O_k * W_o_k^T      (M x h, fp32), O_k = the rank's attention
 *                                 output, M x q_loc*head_dim
 *
 * and the t partials P_k sum (tp_partial_reduce) to O * W_o^T.  The attention
 * core between the two is not part of this library.
 * ---------------------------------------------------------------------- */

/*
 * n_loc, the width of one rank's QKV output (and the row count of its
 * W_qkv_k), or -1 if the heads do not split over t (see tp_attn_qkv_forward).
 */
int64_t tp_attn_qkv_width(int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, int32_t t);

/*
 * Rank k's column-parallel QKV projection.
 *
 *   M          tokens, M >= 1.
 *   h          hidden size (the projection's input features).
 *   n_heads, n_kv_heads, head_dim   query heads, key/value heads (grouped
 *              query attention: n_heads % n_kv_heads == 0) and head size.
 *              n_heads % t == 0, and n_kv_heads % t == 0 or t % n_kv_heads
 *              == 0; else TP_ERR_INVALID_ARG.
 *   t, k       TP degree (1..64), rank index (validated; selects no data).
 *   act_dtype, w_dtype   as tp_mlp_shard_forward: (bf16, bf16),
 *              (bf16, fp8 e4m3fn), (bf16, int8), (fp32, fp32).
 *   x          M x h, leading dimension ldx >= h.
 *   w_qkv      n_loc x h ((out, in) layout), leading dimension ldw >= h: the
 *              rank's rows in the order [its q_loc query heads | its kv_loc
 *              key heads | its kv_loc value heads], head_dim rows per head,
 *              heads in their global order.  Rank k holds query heads
 *              [k*q_loc, (k+1)*q_loc) and key/value heads [k*kv_loc,
 *              (k+1)*kv_loc), or, replicated, head k / (t / n_kv_heads).
 *   s_qkv      one-byte weights only: n_loc fp32 per-row scales (weight = code * scale of
 *              its row); NULL otherwise.
 *   qkv        M x n_loc output in the activation dtype, leading dimension
 *              ldq >= n_loc, same column order as w_qkv's rows; overwritten;
 *              must not overlap an input.
 *   workspace, workspace_bytes   device scratch of at least
 *              tp_attn_qkv_workspace_bytes(...) bytes, 256-byte aligned, not
 *              overlapping any argument; may be NULL when that size is 0.
 *              It holds fp32 sums over ranges of h when the projection is
 *              split along h across workgroups: decode with a narrow output
 *              (few rows of W to spread over the chip), prefill with output
 *              tiles that do not fill whole rounds of the CUs (stream-K
 *              pieces and their arrival counters).  Contents on entry are
 *              ignored; concurrent calls must not share it.
 *
 * Requirements (else TP_ERR_UNSUPPORTED): with bf16 activations h % 64 == 0
 * and n_loc % 16 == 0, pointers and rows 16-byte aligned, scales 4-byte
 * aligned; with fp32, 4-byte alignment.  Deterministic: the split and the
 * order of the partial sums depend on the shape only (not on which workgroup
 * finishes first).
 */
tp_status tp_attn_qkv_forward(int64_t M, int64_t h, int64_t n_heads, int64_t n_kv_heads,
                              int64_t head_dim, int32_t t, int32_t k,
                              int32_t act_dtype, int32_t w_dtype,
                              const void* x, int64_t ldx,
                              const void* w_qkv, int64_t ldw, const float* s_qkv,
                              void* qkv, int64_t ldq,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes tp_attn_qkv_forward needs for these arguments (0 if none
 * is needed or the arguments are invalid).
 */
size_t tp_attn_qkv_workspace_bytes(int64_t M, int64_t h, int64_t n_heads, int64_t n_kv_heads,
                                   int64_t head_dim, int32_t t, int32_t act_dtype, int32_t w_dtype);

/*
 * Rank k's row-parallel output projection: partial P_k (M x h fp32).
 *
 *   n_heads, head_dim   q_loc = n_heads / t query heads per rank
 *              (n_heads % t == 0, else TP_ERR_INVALID_ARG); the input width
 *              is K = q_loc * head_dim.
 *   attn       M x K, the rank's attention output (its heads in global
 *              order), activation dtype, leading dimension lda >= K.
 *   w_o        h x K ((out, in) layout: the rank's column block of the full
 *              h x n_heads*head_dim matrix), leading dimension ldw >= K.  A
 *              caller holding the full matrix passes the pointer to column
 *              k*K and ldw = n_heads*head_dim.
 *   s_o        one-byte weights only: h fp32 per-row scales; NULL otherwise.
 *   partial    M x h fp32, leading dimension ldp >= h; overwritten; must not
 *              overlap an input.
 *
 * Other arguments and requirements as tp_attn_qkv_forward, with K in place
 * of h (K % 64 == 0) and h in place of n_loc (h % 16 == 0).  No workspace.
 */
tp_status tp_attn_out_forward(int64_t M, int64_t h, int64_t n_heads, int64_t head_dim,
                              int32_t t, int32_t k,
                              int32_t act_dtype, int32_t w_dtype,
                              const void* attn, int64_t lda,
                              const void* w_o, int64_t ldw, const float* s_o,
                              float* partial, int64_t ldp, void* stream);

/* Static text for a status code. */
const char* tp_status_string(int32_t status);

/* Message describing the last non-OK status returned on this thread. */
const char* tp_last_error(void);

/* ------------------------------------------------------------------------
 * Kernel timing (for benchmarks).  While enabled, every kernel the library
 * launches records its own start and end timestamps on the stream it runs on
 * (HIP extended launch with a start and a stop event).  tp_profile_collect
 * waits for those events, adds the durations per kernel kind and clears the
 * record.  Not thread-safe; intended for a single benchmarking thread.
 * ---------------------------------------------------------------------- */

/* Number of kernel kinds (indices 0 .. n-1 for the calls below). */
int32_t tp_kernel_kind_count(void);

/* Static name of a kernel kind (NULL if out of range). */
const char* tp_kernel_kind_name(int32_t kind);

/*
 * Select the kernel kinds to time: bit i of `kinds` times the kernels of
 * kind i, 0 turns timing off, -1 times every kind.  A timed launch costs the
 * host noticeably more than a plain one (on the order of 20 us against 3 us
 * here), so a throughput loop should time only the kinds it reports.
 */
tp_status tp_profile_enable(int32_t kinds);

/*
 * Create event pairs up front for at least `records` timed launches, so
 * that timing does not create events (a slow host call) inside a measured
 * loop; without it the record grows on demand.  Synchronous.
 */
tp_status tp_profile_reserve(int64_t records);

/*
 * Synchronise the recorded events and add, for each kind i < n_kinds,
 * the summed duration in milliseconds to total_ms[i] and the number of
 * launches to counts[i].  Clears the record.  Both arrays are host memory.
 */
tp_status tp_profile_collect(double* total_ms, int64_t* counts, int32_t n_kinds);

/*
 * Durations in milliseconds of the recorded launches of kernel kind `kind`,
 * in launch order, without clearing the record (call before
 * tp_profile_collect): the first min(count, capacity) go to ms (host
 * memory, may be NULL when capacity is 0) and the count to *n.  Waits for
 * those launches' events.
 */
tp_status tp_profile_durations(int32_t kind, float* ms, int64_t capacity, int64_t* n);

/* ------------------------------------------------------------------------
 * Packed weights.
 *
 * The same forward as tp_mlp_shard_forward, reading the rank's three weight
 * matrices from one array in the order the weight-streaming decode kernels
 * consume them: each workgroup then reads one contiguous range of memory
 * instead of 16 rows side by side (on MI355X the gate/up launches of the 70B
 * shard measured 5 to 14 % shorter).  The same array also serves every
 * larger M: MFMA GEMMs on 256-token tiles that load the packed fragments
 * straight into the matrix instruction's operand registers (one-byte codes
 * widened to bf16 there), so a server keeps one copy of the weights for
 * decode and prefill.  Packing is a permutation of the weight bytes, done once per
 * weight set on the GPU.  At decode sizes the packed forward's partial is
 * bit-identical to tp_mlp_shard_forward's on the same weights; above them
 * too when both add the products in the same order (256-token tiles with
 * the same stream-K plan, e.g. 4096 tokens of the 70B TP = 8 shard), and
 * otherwise within the bf16 tolerance.  The projections are those of "The
 * Tensor-Parallel Shard Group" (scalablesystem.dev): the rank's column
 * shards of W_gate and W_up and its row shard of W_down.
 *
 * Layout (opaque to callers; for the record): gate/up blocks of 8 channels
 * (their 8 gate rows, then their 8 up rows), then down blocks of 16 rows of
 * W_down; each block is a run of 4 KB slots (128 k-values of bf16 or 256 of
 * one-byte weights for each of the 16 rows, 16-byte chunks permuted within
 * a row); rows past the end repeat the last row.
 * ------------------------------------------------------------------------ */

/*
 * Bytes of the packed array for these shapes (w_dtype TP_BF16, TP_FP8_E4M3FN
 * or TP_INT8): the size of the three weight matrices when I_s is a multiple
 * of 8.  Requires h and I_s = I_full / t multiples of 128 (bf16) or 256
 * (one-byte weights); 0 if the arguments are invalid or unsupported.
 */
size_t tp_mlp_packed_weights_bytes(int64_t h, int64_t I_full, int32_t t, int32_t w_dtype);

/*
 * Writes the packed array of one rank's weights (device pointers, the layout
 * and dtypes of tp_mlp_shard_forward: w_gate, w_up I_s x h with leading
 * dimension ldw_gu; w_down h x I_s with ldw_down) to packed (device, 16-byte
 * aligned, at least tp_mlp_packed_weights_bytes(...) bytes, not overlapping
 * the weights), asynchronously on stream.  The scales are not part of it.
 * Errors: TP_ERR_INVALID_ARG (null pointer, leading dimension, size,
 * overlap), TP_ERR_UNSUPPORTED (shapes, alignment, dtype), TP_ERR_HIP.
 */
tp_status tp_mlp_pack_weights(int64_t h, int64_t I_full, int32_t t, int32_t w_dtype,
                              const void* w_gate, const void* w_up, int64_t ldw_gu,
                              const void* w_down, int64_t ldw_down,
                              void* packed, size_t packed_bytes, void* stream);

/*
 * Workspace bytes of tp_mlp_shard_forward_packed for these shapes (bf16
 * activations): A (M x I_s bf16) plus the split scratch of the decode
 * streams or, above the decode sizes, the stream-K scratch of the packed
 * 256-token GEMMs (this can exceed tp_mlp_workspace_bytes for a few hundred
 * tokens).  0 if the shapes are invalid or not packable.
 */
size_t tp_mlp_packed_workspace_bytes(int64_t M, int64_t h, int64_t I_full, int32_t t, int32_t w_dtype);

/*
 * tp_mlp_shard_forward with the weights given as a packed array (above)
 * instead of w_gate, w_up, w_down and their leading dimensions; bf16
 * activations only; any M >= 1.  packed_bytes is the size of the
 * caller's packed array; fewer than tp_mlp_packed_weights_bytes(h, I_full,
 * t, w_dtype) bytes (an array packed for other shapes) is
 * TP_ERR_INVALID_ARG.  The workspace needs tp_mlp_packed_workspace_bytes(...)
 * bytes (TP_ERR_WORKSPACE if smaller); its contents on entry do not matter.
 * s_gate, s_up, s_down, partial and the other errors are as for
 * tp_mlp_shard_forward; the packed array must not overlap the partial or
 * the workspace.
 */
tp_status tp_mlp_shard_forward_packed(int64_t M, int64_t h, int64_t I_full, int32_t t, int32_t k,
                                      int32_t act_dtype, int32_t w_dtype, const void* x, int64_t ldx,
                                      const void* packed, size_t packed_bytes,
                                      const float* s_gate, const float* s_up,
                                      const float* s_down, float* partial, int64_t ldp,
                                      void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TP_MLP_H */
