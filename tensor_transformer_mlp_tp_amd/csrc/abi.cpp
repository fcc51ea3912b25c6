// C ABI of the TP-MLP shard library: argument validation, dispatch, status
// strings and the kernel timing record.  The operation and the calling
// conventions are documented in include/tp_mlp.h.
//
// Validation follows the pages' statement of the layers: out_features and
// in_features must divide by the group size (ColumnParallelLinear /
// RowParallelLinear in "The Tensor-Parallel Shard Group", scalablesystem.dev),
// a rank holds only its own shard, and its forward returns a partial that the
// all-reduce sums.  Everything is checked on the host before any HIP call.
#include "tp_mlp.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "common.h"
#include "internal.h"

#define TP_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[512] = "no error";

tp_status fail(tp_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

tp_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return TP_OK;
  return fail(TP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int elem_bytes(int32_t dt) {
  switch (dt) {
    case TP_F32: return 4;
    case TP_BF16: return 2;
    case TP_FP8_E4M3FN: return 1;
    case TP_INT8: return 1;
    default: return 0;
  }
}

// One-byte weight formats (fp32 scale per output row) and the kernels' code.
bool scaled_weights(int32_t w) { return w == TP_FP8_E4M3FN || w == TP_INT8; }

int weight_format(int32_t w) {
  return w == TP_FP8_E4M3FN ? tpmlp::kWeightE4M3 : w == TP_INT8 ? tpmlp::kWeightI8 : tpmlp::kWeightWide;
}

// Supported (activation, weight) pairs; fills an error message otherwise.
tp_status check_pair(int32_t act, int32_t w) {
  if (elem_bytes(act) == 0 || elem_bytes(w) == 0)
    return fail(TP_ERR_INVALID_ARG, "unknown dtype code (act=%d, w=%d)", act, w);
  if (act == TP_FP8_E4M3FN || act == TP_INT8)
    return fail(TP_ERR_UNSUPPORTED, "one-byte activations are not supported");
  const bool ok = (act == TP_BF16 && (w == TP_BF16 || scaled_weights(w))) || (act == TP_F32 && w == TP_F32);
  if (!ok) return fail(TP_ERR_UNSUPPORTED, "unsupported dtype pair (act=%d, w=%d)", act, w);
  return TP_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte extent of a rows x cols matrix with leading dimension ld.
struct Extent {
  uintptr_t lo, hi;  // [lo, hi)
};

Extent extent(const void* p, int64_t rows, int64_t cols, int64_t ld, int eb) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  const uintptr_t len = (uintptr_t)(((rows - 1) * ld + cols) * eb);
  return Extent{lo, lo + len};
}

bool overlap(Extent a, Extent b) { return a.lo < b.hi && b.lo < a.hi; }

constexpr int64_t kMaxDim = (int64_t)1 << 30;

int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Shape checks shared by the workspace query and the forward.
tp_status check_shapes(int64_t M, int64_t h, int64_t I_full, int32_t t, int32_t k, int32_t act,
                       int32_t w) {
  if (M < 1 || h < 1 || I_full < 1)
    return fail(TP_ERR_INVALID_ARG, "M, h and I_full must be >= 1 (got %lld, %lld, %lld)",
                (long long)M, (long long)h, (long long)I_full);
  if (t < 1 || t > tpmlp::kMaxPartials)
    return fail(TP_ERR_INVALID_ARG, "t must be in [1, %d] (got %d)", tpmlp::kMaxPartials, t);
  if (k < 0 || k >= t) return fail(TP_ERR_INVALID_ARG, "k must be in [0, t) (got k=%d, t=%d)", k, t);
  if (I_full % t != 0)
    return fail(TP_ERR_INVALID_ARG, "I_full (%lld) must be divisible by t (%d)", (long long)I_full, t);
  {
    const tp_status st = check_pair(act, w);
    if (st != TP_OK) return st;
  }
  const int64_t I_s = I_full / t;
  if (M > kMaxDim || h > kMaxDim || I_s > kMaxDim)
    return fail(TP_ERR_UNSUPPORTED, "dimension above 2^30");
  if (act == TP_BF16 && (h % 64 != 0 || I_s % 64 != 0))
    return fail(TP_ERR_UNSUPPORTED, "bf16 paths need h %% 64 == 0 and I_s %% 64 == 0 (h=%lld, I_s=%lld)",
                (long long)h, (long long)I_s);
  return TP_OK;
}

// The forward's workspace: A (M x I_s, the activation dtype), then for a
// bf16 prefill the two GEMMs' stream-K scratch.
int64_t workspace_a_bytes(int64_t M, int64_t I_s, int32_t act) { return round_up(M * I_s * elem_bytes(act), 256); }

int64_t workspace_need(int64_t M, int64_t h, int64_t I_s, int32_t act, int32_t w) {
  const int wb = weight_format(w);
  const int64_t sk = act != TP_BF16 ? 0
                     : M > tpmlp::forward_decode_max_m(wb)
                         ? tpmlp::forward_prefill_sk_bytes((int)M, (int)h, (int)I_s, false)
                         : tpmlp::forward_decode_sk_bytes((int)M, (int)h, (int)I_s, wb);
  return workspace_a_bytes(M, I_s, act) + round_up(sk, 256);
}

// Workspace of the packed forward (bf16 activations): the decode streams'
// split scratch, or above the decode sizes that of the packed-weight GEMMs.
int64_t packed_workspace_need(int64_t M, int64_t h, int64_t I_s, int32_t w) {
  const int wb = weight_format(w);
  const int64_t sk = M > tpmlp::forward_decode_max_m(wb)
                         ? tpmlp::forward_prefill_packed_sk_bytes((int)M, (int)h, (int)I_s)
                         : tpmlp::forward_decode_sk_bytes((int)M, (int)h, (int)I_s, wb);
  return workspace_a_bytes(M, I_s, TP_BF16) + round_up(sk, 256);
}

// ------------------------------------------------------------------ timing

struct ProfRec {
  hipEvent_t start, stop;
  int kind;
};

uint32_t g_prof_mask = 0;   // bit i: time kernels of kind i
std::vector<ProfRec> g_prof_pool;
size_t g_prof_used = 0;
// Set during an allocation-free call: timing then uses reserved events only.
thread_local bool g_no_alloc = false;

const char* const kKindNames[tpmlp::K_NUM_KINDS] = {
    "gateup_decode", "down_decode", "gateup_prefill", "down_prefill",
    "partial_reduce", "gateup_f32", "down_f32", "qkv_decode", "qkv_prefill",
    "oproj_decode", "oproj_prefill", "qkv_f32", "oproj_f32", "quant_rows",
    "gateup_w8a8", "down_w8a8", "sk_clear"};

// Appends one start/stop event pair to the timing pool.  The events only
// time launches (read after the caller synchronises), so they skip the
// system-scope fence on record: its L2 write-back and invalidate would add to
// the timed interval and slow the launch that follows.
bool prof_grow() {
  ProfRec r{};
  if (hipEventCreateWithFlags(&r.start, hipEventDisableSystemFence) != hipSuccess) return false;
  if (hipEventCreateWithFlags(&r.stop, hipEventDisableSystemFence) != hipSuccess) {
    (void)hipEventDestroy(r.start);
    return false;
  }
  g_prof_pool.push_back(r);
  return true;
}

}  // namespace

namespace tpmlp {

void profile_events_for_launch(int kind, hipEvent_t* start, hipEvent_t* stop) {
  *start = nullptr;
  *stop = nullptr;
  if (kind < 0 || kind >= 32 || !((g_prof_mask >> kind) & 1u)) return;
  if (g_prof_used == g_prof_pool.size() && (g_no_alloc || !prof_grow())) return;
  ProfRec& r = g_prof_pool[g_prof_used++];
  r.kind = kind;
  *start = r.start;
  *stop = r.stop;
}

}  // namespace tpmlp

TP_API size_t tp_mlp_workspace_bytes(int64_t M, int64_t h, int64_t I_full, int32_t t,
                                     int32_t act_dtype, int32_t w_dtype) {
  if (check_shapes(M, h, I_full, t, 0, act_dtype, w_dtype) != TP_OK) return 0;
  return (size_t)workspace_need(M, h, I_full / t, act_dtype, w_dtype);
}

namespace {

// Checks and launch shared by the contiguous and the row-block forms of the
// forward.  x_blocks[0..nb): the activation row blocks, rows_per_block rows
// each (nb * rows_per_block == M).
tp_status forward_impl(int64_t M, int64_t h, int64_t I_full, int32_t t, int32_t k, int32_t act_dtype,
                       int32_t w_dtype, const void* const* x_blocks, int nb, int64_t rows_per_block,
                       int64_t ldx, const void* w_gate, const void* w_up, int64_t ldw_gu, const void* w_down,
                       int64_t ldw_down, const float* s_gate, const float* s_up, const float* s_down,
                       float* partial, int64_t ldp, void* workspace, size_t workspace_bytes, void* stream) {
  tp_status st = check_shapes(M, h, I_full, t, k, act_dtype, w_dtype);
  if (st != TP_OK) return st;
  const int64_t I_s = I_full / t;
  if (!x_blocks || !w_gate || !w_up || !w_down || !partial)
    return fail(TP_ERR_INVALID_ARG, "null tensor pointer");
  for (int b = 0; b < nb; ++b)
    if (!x_blocks[b]) return fail(TP_ERR_INVALID_ARG, "null activation pointer (block %d)", b);
  const bool fp8 = scaled_weights(w_dtype);   // one-byte weights with row scales
  if (fp8 && (!s_gate || !s_up || !s_down))
    return fail(TP_ERR_INVALID_ARG, "one-byte weights need s_gate, s_up and s_down");
  if (!fp8 && (s_gate || s_up || s_down))
    return fail(TP_ERR_INVALID_ARG, "scales are only accepted with one-byte weights");
  if (ldx < h || ldw_gu < h || ldw_down < I_s || ldp < h)
    return fail(TP_ERR_INVALID_ARG, "leading dimension smaller than the row length "
                "(ldx=%lld ldw_gu=%lld ldw_down=%lld ldp=%lld)", (long long)ldx, (long long)ldw_gu,
                (long long)ldw_down, (long long)ldp);
  const int64_t need = workspace_need(M, h, I_s, act_dtype, w_dtype);
  if (!workspace || (int64_t)workspace_bytes < need)
    return fail(TP_ERR_WORKSPACE, "workspace of %lld bytes needed (got %llu)", (long long)need,
                (unsigned long long)workspace_bytes);
  const int ea = elem_bytes(act_dtype), ew = elem_bytes(w_dtype);
  const size_t amin = act_dtype == TP_BF16 ? 16 : 4;
  for (int b = 0; b < nb; ++b)
    if (!aligned(x_blocks[b], amin))
      return fail(TP_ERR_UNSUPPORTED, "activation pointers must be %d-byte aligned", (int)amin);
  if (act_dtype == TP_BF16) {
    if (!aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(w_down, 16) || !aligned(partial, 16))
      return fail(TP_ERR_UNSUPPORTED, "tensor pointers must be 16-byte aligned");
    if ((ldx * ea) % 16 || (ldw_gu * ew) % 16 || (ldw_down * ew) % 16 || (ldp * 4) % 16)
      return fail(TP_ERR_UNSUPPORTED, "rows must start 16-byte aligned (leading dimensions)");
    if (fp8 && (!aligned(s_gate, 4) || !aligned(s_up, 4) || !aligned(s_down, 4)))
      return fail(TP_ERR_UNSUPPORTED, "scale pointers must be 4-byte aligned");
  } else {
    if (!aligned(w_gate, 4) || !aligned(w_up, 4) || !aligned(w_down, 4) || !aligned(partial, 4))
      return fail(TP_ERR_UNSUPPORTED, "fp32 pointers must be 4-byte aligned");
  }
  if (!aligned(workspace, 256)) return fail(TP_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");

  const Extent ep = extent(partial, M, h, ldp, 4);
  const Extent ewk{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + (uintptr_t)need};
  const Extent ins[4] = {extent(w_gate, I_s, h, ldw_gu, ew), extent(w_up, I_s, h, ldw_gu, ew),
                         extent(w_down, h, I_s, ldw_down, ew), ewk};
  for (const Extent& e : ins)
    if (overlap(ep, e)) return fail(TP_ERR_INVALID_ARG, "partial overlaps an input or the workspace");
  for (int i = 0; i < 3; ++i)
    if (overlap(ewk, ins[i])) return fail(TP_ERR_INVALID_ARG, "workspace overlaps an input");
  for (int b = 0; b < nb; ++b) {
    const Extent ex = extent(x_blocks[b], rows_per_block, h, ldx, ea);
    if (overlap(ep, ex)) return fail(TP_ERR_INVALID_ARG, "partial overlaps the activations");
    if (overlap(ewk, ex)) return fail(TP_ERR_INVALID_ARG, "workspace overlaps the activations");
  }

  tpmlp::ShardArgs a;
  a.M = (int)M;
  a.h = (int)h;
  a.I_s = (int)I_s;
  a.x = tpmlp::XRows{};
  for (int b = 0; b < nb; ++b) a.x.p[b] = x_blocks[b];
  a.x.nb = nb;
  a.x.rows = (int)rows_per_block;
  a.x.ld = ldx;
  a.wg = w_gate;
  a.wu = w_up;
  a.ldw_gu = ldw_gu;
  a.wd = w_down;
  a.ldw_down = ldw_down;
  a.sg = s_gate;
  a.su = s_up;
  a.sd = s_down;
  a.p = partial;
  a.ldp = ldp;
  a.a = workspace;
  a.lda = I_s;
  a.wb = weight_format(w_dtype);
  a.sk = need > workspace_a_bytes(M, I_s, act_dtype)
             ? static_cast<uint8_t*>(workspace) + workspace_a_bytes(M, I_s, act_dtype) : nullptr;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (act_dtype == TP_F32)
    e = tpmlp::launch_forward_f32(a, s);
  else if (M <= tpmlp::forward_decode_max_m(a.wb))
    e = tpmlp::launch_forward_decode(a, s);
  else
    e = tpmlp::launch_forward_prefill(a, s);
  return from_hip(e, "kernel launch");
}

}  // namespace

TP_API tp_status tp_mlp_shard_forward(int64_t M, int64_t h, int64_t I_full, int32_t t, int32_t k,
                                      int32_t act_dtype, int32_t w_dtype, const void* x, int64_t ldx,
                                      const void* w_gate, const void* w_up, int64_t ldw_gu,
                                      const void* w_down, int64_t ldw_down, const float* s_gate,
                                      const float* s_up, const float* s_down, float* partial,
                                      int64_t ldp, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  const void* blocks[1] = {x};
  return forward_impl(M, h, I_full, t, k, act_dtype, w_dtype, blocks, 1, M, ldx, w_gate, w_up, ldw_gu, w_down,
                      ldw_down, s_gate, s_up, s_down, partial, ldp, workspace, workspace_bytes, stream);
}

// ------------------------------------------------------------ allocation-free forward

namespace {

// The allocation-free forward's scratch: one array per device (each device
// that loads the library's code object holds its own copy until the process
// ends).  In host code `noalloc_scratch` names a host-side stand-in, not the
// device array: device code reaches the array only through the address
// hipGetSymbolAddress returns for the current device, kept per device.
static __device__ __align__(256) uint8_t noalloc_scratch[TP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mu;
void* g_noalloc_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up on the
// first call on that device.
tp_status noalloc_scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return from_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(TP_ERR_UNSUPPORTED, "device index %d is not below %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch));
    if (e != hipSuccess) return from_hip(e, "hipGetSymbolAddress (allocation-free scratch)");
    if (!p || !aligned(p, 256)) return fail(TP_ERR_HIP, "allocation-free scratch has no 256-byte aligned address");
    g_noalloc_ptr[dev] = p;
  }
  *out = g_noalloc_ptr[dev];
  return TP_OK;
}

}  // namespace

TP_API tp_status tp_mlp_shard_forward_noalloc(int64_t M, int64_t h, int64_t I_full, int32_t t, int32_t k,
                                              int32_t act_dtype, int32_t w_dtype, const void* x, int64_t ldx,
                                              const void* w_gate, const void* w_up, int64_t ldw_gu,
                                              const void* w_down, int64_t ldw_down, const float* s_gate,
                                              const float* s_up, const float* s_down, float* partial,
                                              int64_t ldp, void* stream) {
  const tp_status st = check_shapes(M, h, I_full, t, k, act_dtype, w_dtype);
  if (st != TP_OK) return st;
  const int64_t need = workspace_need(M, h, I_full / t, act_dtype, w_dtype);
  if (need > (int64_t)TP_NOALLOC_SCRATCH_BYTES)
    return fail(TP_ERR_UNSUPPORTED, "this forward needs %lld bytes of scratch; the allocation-free entry point "
                "holds %llu (use tp_mlp_shard_forward with a workspace)", (long long)need,
                (unsigned long long)TP_NOALLOC_SCRATCH_BYTES);
  void* scratch = nullptr;
  const tp_status sp = noalloc_scratch_ptr(&scratch);
  if (sp != TP_OK) return sp;
  const void* blocks[1] = {x};
  g_no_alloc = true;
  const tp_status r = forward_impl(M, h, I_full, t, k, act_dtype, w_dtype, blocks, 1, M, ldx, w_gate, w_up, ldw_gu,
                                   w_down, ldw_down, s_gate, s_up, s_down, partial, ldp, scratch,
                                   TP_NOALLOC_SCRATCH_BYTES, stream);
  g_no_alloc = false;
  return r;
}

// ------------------------------------------------------------ packed decode weights

namespace {

// Packed size for valid arguments, else 0 with the error message set.
int64_t packed_need(int64_t h, int64_t I_full, int32_t t, int32_t w_dtype) {
  if (check_shapes(1, h, I_full, t, 0, TP_BF16, w_dtype) != TP_OK) return 0;
  const int wb = weight_format(w_dtype);
  const int64_t I_s = I_full / t;
  if (!tpmlp::decode_packable((int)h, (int)I_s, wb)) {
    fail(TP_ERR_UNSUPPORTED, "packed weights need h and I_s multiples of %d (h=%lld, I_s=%lld)", wb ? 256 : 128,
         (long long)h, (long long)I_s);
    return 0;
  }
  return tpmlp::packed_gateup_bytes((int)h, (int)I_s, wb) + tpmlp::packed_down_bytes((int)h, (int)I_s, wb);
}

}  // namespace

TP_API size_t tp_mlp_packed_weights_bytes(int64_t h, int64_t I_full, int32_t t, int32_t w_dtype) {
  return (size_t)packed_need(h, I_full, t, w_dtype);
}

TP_API tp_status tp_mlp_pack_weights(int64_t h, int64_t I_full, int32_t t, int32_t w_dtype, const void* w_gate,
                                     const void* w_up, int64_t ldw_gu, const void* w_down, int64_t ldw_down,
                                     void* packed, size_t packed_bytes, void* stream) {
  const tp_status st = check_shapes(1, h, I_full, t, 0, TP_BF16, w_dtype);
  if (st != TP_OK) return st;
  const int64_t need = packed_need(h, I_full, t, w_dtype);
  if (need == 0) return TP_ERR_UNSUPPORTED;
  const int64_t I_s = I_full / t;
  if (!w_gate || !w_up || !w_down || !packed) return fail(TP_ERR_INVALID_ARG, "null pointer");
  if (ldw_gu < h || ldw_down < I_s)
    return fail(TP_ERR_INVALID_ARG, "leading dimension smaller than the row length (ldw_gu=%lld ldw_down=%lld)",
                (long long)ldw_gu, (long long)ldw_down);
  const int ew = elem_bytes(w_dtype);
  if (!aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(w_down, 16) || !aligned(packed, 16) ||
      (ldw_gu * ew) % 16 || (ldw_down * ew) % 16)
    return fail(TP_ERR_UNSUPPORTED, "weights, their rows and the packed array must be 16-byte aligned");
  if ((int64_t)packed_bytes < need)
    return fail(TP_ERR_INVALID_ARG, "packed array of %lld bytes needed (got %llu)", (long long)need,
                (unsigned long long)packed_bytes);
  const Extent ek{reinterpret_cast<uintptr_t>(packed), reinterpret_cast<uintptr_t>(packed) + (uintptr_t)need};
  if (overlap(ek, extent(w_gate, I_s, h, ldw_gu, ew)) || overlap(ek, extent(w_up, I_s, h, ldw_gu, ew)) ||
      overlap(ek, extent(w_down, h, I_s, ldw_down, ew)))
    return fail(TP_ERR_INVALID_ARG, "the packed array overlaps the weights");
  tpmlp::ShardArgs a{};
  a.h = (int)h;
  a.I_s = (int)I_s;
  a.wg = w_gate;
  a.wu = w_up;
  a.ldw_gu = ldw_gu;
  a.wd = w_down;
  a.ldw_down = ldw_down;
  a.wb = weight_format(w_dtype);
  return from_hip(tpmlp::launch_pack_weights(a, packed, reinterpret_cast<hipStream_t>(stream)), "kernel launch");
}

TP_API size_t tp_mlp_packed_workspace_bytes(int64_t M, int64_t h, int64_t I_full, int32_t t, int32_t w_dtype) {
  if (check_shapes(M, h, I_full, t, 0, TP_BF16, w_dtype) != TP_OK) return 0;
  if (packed_need(h, I_full, t, w_dtype) == 0) return 0;
  return (size_t)packed_workspace_need(M, h, I_full / t, w_dtype);
}

TP_API tp_status tp_mlp_shard_forward_packed(int64_t M, int64_t h, int64_t I_full, int32_t t, int32_t k,
                                             int32_t act_dtype, int32_t w_dtype, const void* x, int64_t ldx,
                                             const void* packed, size_t packed_bytes, const float* s_gate,
                                             const float* s_up, const float* s_down, float* partial, int64_t ldp,
                                             void* workspace, size_t workspace_bytes, void* stream) {
  tp_status st = check_shapes(M, h, I_full, t, k, act_dtype, w_dtype);
  if (st != TP_OK) return st;
  if (act_dtype != TP_BF16) return fail(TP_ERR_UNSUPPORTED, "packed weights take bf16 activations");
  const int wb = weight_format(w_dtype);
  const bool prefill = M > tpmlp::forward_decode_max_m(wb);
  const int64_t pbytes = packed_need(h, I_full, t, w_dtype);
  if (pbytes == 0) return TP_ERR_UNSUPPORTED;
  const int64_t I_s = I_full / t;
  if (!x || !packed || !partial) return fail(TP_ERR_INVALID_ARG, "null tensor pointer");
  if ((int64_t)packed_bytes < pbytes)
    return fail(TP_ERR_INVALID_ARG, "packed array of %lld bytes needed for these shapes (got %llu)",
                (long long)pbytes, (unsigned long long)packed_bytes);
  const bool fp8 = scaled_weights(w_dtype);
  if (fp8 && (!s_gate || !s_up || !s_down))
    return fail(TP_ERR_INVALID_ARG, "one-byte weights need s_gate, s_up and s_down");
  if (!fp8 && (s_gate || s_up || s_down))
    return fail(TP_ERR_INVALID_ARG, "scales are only accepted with one-byte weights");
  if (ldx < h || ldp < h)
    return fail(TP_ERR_INVALID_ARG, "leading dimension smaller than the row length (ldx=%lld ldp=%lld)",
                (long long)ldx, (long long)ldp);
  const int64_t need = packed_workspace_need(M, h, I_s, w_dtype);
  if (!workspace || (int64_t)workspace_bytes < need)
    return fail(TP_ERR_WORKSPACE, "workspace of %lld bytes needed (got %llu)", (long long)need,
                (unsigned long long)workspace_bytes);
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(partial, 16) || (ldx * 2) % 16 || (ldp * 4) % 16)
    return fail(TP_ERR_UNSUPPORTED, "tensor pointers and rows must be 16-byte aligned");
  if (fp8 && (!aligned(s_gate, 4) || !aligned(s_up, 4) || !aligned(s_down, 4)))
    return fail(TP_ERR_UNSUPPORTED, "scale pointers must be 4-byte aligned");
  if (!aligned(workspace, 256)) return fail(TP_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  const Extent ep = extent(partial, M, h, ldp, 4), ex = extent(x, M, h, ldx, 2);
  const Extent ek{reinterpret_cast<uintptr_t>(packed), reinterpret_cast<uintptr_t>(packed) + (uintptr_t)pbytes};
  const Extent ewk{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + (uintptr_t)need};
  if (overlap(ep, ex) || overlap(ep, ek) || overlap(ep, ewk))
    return fail(TP_ERR_INVALID_ARG, "partial overlaps an input or the workspace");
  if (overlap(ewk, ex) || overlap(ewk, ek)) return fail(TP_ERR_INVALID_ARG, "workspace overlaps an input");

  tpmlp::ShardArgs a{};
  a.M = (int)M;
  a.h = (int)h;
  a.I_s = (int)I_s;
  a.x.p[0] = x;
  a.x.nb = 1;
  a.x.rows = (int)M;
  a.x.ld = ldx;
  a.wb = wb;
  a.packed = true;
  a.wg = packed;
  a.wu = nullptr;
  a.ldw_gu = h;
  a.wd = static_cast<const uint8_t*>(packed) + tpmlp::packed_gateup_bytes((int)h, (int)I_s, wb);
  a.ldw_down = I_s;
  a.sg = s_gate;
  a.su = s_up;
  a.sd = s_down;
  a.p = partial;
  a.ldp = ldp;
  a.a = workspace;
  a.lda = I_s;
  a.sk = need > workspace_a_bytes(M, I_s, act_dtype)
             ? static_cast<uint8_t*>(workspace) + workspace_a_bytes(M, I_s, act_dtype) : nullptr;
  if (prefill)
    return from_hip(tpmlp::launch_forward_prefill(a, reinterpret_cast<hipStream_t>(stream)), "kernel launch");
  return from_hip(tpmlp::launch_forward_decode(a, reinterpret_cast<hipStream_t>(stream)), "kernel launch");
}

TP_API tp_status tp_mlp_shard_forward_sp(int64_t M, int64_t h, int64_t I_full, int32_t t, int32_t k,
                                         int32_t act_dtype, int32_t w_dtype, const void* const* x_blocks,
                                         int64_t ldx, const void* w_gate, const void* w_up, int64_t ldw_gu,
                                         const void* w_down, int64_t ldw_down, const float* s_gate,
                                         const float* s_up, const float* s_down, float* partial, int64_t ldp,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  if (t < 1 || t > tpmlp::kMaxPartials)
    return fail(TP_ERR_INVALID_ARG, "t must be in [1, %d] (got %d)", tpmlp::kMaxPartials, t);
  if (M < 1 || M % t != 0)
    return fail(TP_ERR_INVALID_ARG, "M (%lld) must be a positive multiple of t (%d)", (long long)M, t);
  if (!x_blocks) return fail(TP_ERR_INVALID_ARG, "null x_blocks array");
  return forward_impl(M, h, I_full, t, k, act_dtype, w_dtype, x_blocks, t, M / t, ldx, w_gate, w_up, ldw_gu,
                      w_down, ldw_down, s_gate, s_up, s_down, partial, ldp, workspace, workspace_bytes, stream);
}

TP_API tp_status tp_partial_reduce(int64_t n, int32_t t, const float* const* partials, float* out,
                                   void* stream) {
  if (n < 0) return fail(TP_ERR_INVALID_ARG, "n must be >= 0");
  if (t < 1 || t > tpmlp::kMaxPartials)
    return fail(TP_ERR_INVALID_ARG, "t must be in [1, %d] (got %d)", tpmlp::kMaxPartials, t);
  if (n == 0) return TP_OK;  // nothing is read or written; pointers may be null
  if (!partials || !out) return fail(TP_ERR_INVALID_ARG, "null pointer");
  if (n > ((int64_t)1 << 40)) return fail(TP_ERR_UNSUPPORTED, "n above 2^40");
  tpmlp::PartialPtrs ptrs{};
  const Extent eo = extent(out, 1, n > 0 ? n : 1, n, 4);
  for (int j = 0; j < t; ++j) {
    if (!partials[j]) return fail(TP_ERR_INVALID_ARG, "partials[%d] is null", j);
    if (!aligned(partials[j], 16)) return fail(TP_ERR_UNSUPPORTED, "partials[%d] not 16-byte aligned", j);
    const Extent ej = extent(partials[j], 1, n > 0 ? n : 1, n, 4);
    const bool in_place = (j == 0 && partials[0] == out);
    if (!in_place && overlap(eo, ej))
      return fail(TP_ERR_INVALID_ARG, "out overlaps partials[%d] (only out == partials[0] is allowed)", j);
    ptrs.p[j] = partials[j];
  }
  if (!aligned(out, 16)) return fail(TP_ERR_UNSUPPORTED, "out not 16-byte aligned");
  return from_hip(tpmlp::launch_partial_reduce(ptrs, t, out, n, reinterpret_cast<hipStream_t>(stream)),
                  "kernel launch");
}

TP_API tp_status tp_partial_reduce_scatter(int64_t rows, int64_t row_len, int32_t t, int32_t k,
                                           const float* const* partials, float* out, void* stream) {
  if (t < 1 || t > tpmlp::kMaxPartials)
    return fail(TP_ERR_INVALID_ARG, "t must be in [1, %d] (got %d)", tpmlp::kMaxPartials, t);
  if (k < 0 || k >= t) return fail(TP_ERR_INVALID_ARG, "k must be in [0, t) (got k=%d, t=%d)", k, t);
  if (rows < 0 || row_len < 0 || rows % t != 0)
    return fail(TP_ERR_INVALID_ARG, "rows (%lld) must be a non-negative multiple of t (%d)", (long long)rows, t);
  if (!partials) return fail(TP_ERR_INVALID_ARG, "null partials array");
  const int64_t n = rows / t * row_len;
  if (n == 0) return TP_OK;
  if ((n * 4) % 16) return fail(TP_ERR_UNSUPPORTED, "rows/t * row_len must be a multiple of 4");
  const float* shifted[tpmlp::kMaxPartials];
  for (int j = 0; j < t; ++j) {
    if (!partials[j]) return fail(TP_ERR_INVALID_ARG, "partials[%d] is null", j);
    shifted[j] = partials[j] + (int64_t)k * n;
  }
  return tp_partial_reduce(n, t, shifted, out, stream);
}

// ------------------------------------------------------------ fp8 x fp8

namespace {

struct W8A8Layout {
  int64_t a, xq, sx, aq, sa, sk, total;   // byte offsets in the workspace
};

W8A8Layout w8a8_layout(int64_t M, int64_t h, int64_t I_s) {
  W8A8Layout l;
  l.a = 0;
  l.xq = l.a + round_up(M * I_s * 2, 256);
  l.sx = l.xq + round_up(M * h, 256);
  l.aq = l.sx + round_up(M * 4, 256);
  l.sa = l.aq + round_up(M * I_s, 256);
  l.sk = l.sa + round_up(M * 4, 256);
  l.total = l.sk + round_up(tpmlp::forward_prefill_sk_bytes((int)M, (int)h, (int)I_s, true), 256);
  return l;
}

tp_status check_w8a8(int64_t M, int64_t h, int64_t I_full, int32_t t, int32_t k) {
  tp_status st = check_shapes(M, h, I_full, t, k, TP_BF16, TP_FP8_E4M3FN);
  if (st != TP_OK) return st;
  if (h % 128 != 0 || (I_full / t) % 128 != 0)
    return fail(TP_ERR_UNSUPPORTED, "the fp8 x fp8 forward needs h %% 128 == 0 and I_s %% 128 == 0");
  return TP_OK;
}

}  // namespace

TP_API size_t tp_mlp_w8a8_workspace_bytes(int64_t M, int64_t h, int64_t I_full, int32_t t) {
  if (check_w8a8(M, h, I_full, t, 0) != TP_OK) return 0;
  return (size_t)w8a8_layout(M, h, I_full / t).total;
}

TP_API tp_status tp_mlp_shard_forward_w8a8(int64_t M, int64_t h, int64_t I_full, int32_t t, int32_t k,
                                           const void* x, int64_t ldx, const void* w_gate, const void* w_up,
                                           int64_t ldw_gu, const void* w_down, int64_t ldw_down,
                                           const float* s_gate, const float* s_up, const float* s_down,
                                           float* partial, int64_t ldp, void* workspace, size_t workspace_bytes,
                                           void* stream) {
  tp_status st = check_w8a8(M, h, I_full, t, k);
  if (st != TP_OK) return st;
  const int64_t I_s = I_full / t;
  if (!x || !w_gate || !w_up || !w_down || !partial) return fail(TP_ERR_INVALID_ARG, "null tensor pointer");
  if (!s_gate || !s_up || !s_down) return fail(TP_ERR_INVALID_ARG, "e4m3fn weights need s_gate, s_up and s_down");
  if (ldx < h || ldw_gu < h || ldw_down < I_s || ldp < h)
    return fail(TP_ERR_INVALID_ARG, "leading dimension smaller than the row length");
  const W8A8Layout l = w8a8_layout(M, h, I_s);
  if (!workspace || (int64_t)workspace_bytes < l.total)
    return fail(TP_ERR_WORKSPACE, "workspace of %lld bytes needed (got %llu)", (long long)l.total,
                (unsigned long long)workspace_bytes);
  if (!aligned(workspace, 256)) return fail(TP_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  if (!aligned(x, 16) || !aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(w_down, 16) || !aligned(partial, 16))
    return fail(TP_ERR_UNSUPPORTED, "tensor pointers must be 16-byte aligned");
  if ((ldx * 2) % 16 || ldw_gu % 16 || ldw_down % 16 || (ldp * 4) % 16)
    return fail(TP_ERR_UNSUPPORTED, "rows must start 16-byte aligned (leading dimensions)");
  if (!aligned(s_gate, 4) || !aligned(s_up, 4) || !aligned(s_down, 4))
    return fail(TP_ERR_UNSUPPORTED, "scale pointers must be 4-byte aligned");
  const Extent ep = extent(partial, M, h, ldp, 4);
  const Extent ew{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + (uintptr_t)l.total};
  const Extent ins[5] = {extent(w_gate, I_s, h, ldw_gu, 1), extent(w_up, I_s, h, ldw_gu, 1),
                         extent(w_down, h, I_s, ldw_down, 1), extent(x, M, h, ldx, 2), ew};
  for (const Extent& e : ins)
    if (overlap(ep, e)) return fail(TP_ERR_INVALID_ARG, "partial overlaps an input or the workspace");
  for (int i = 0; i < 4; ++i)
    if (overlap(ew, ins[i])) return fail(TP_ERR_INVALID_ARG, "workspace overlaps an input");

  uint8_t* wsb = static_cast<uint8_t*>(workspace);
  tpmlp::ShardArgs a;
  a.M = (int)M;
  a.h = (int)h;
  a.I_s = (int)I_s;
  a.x = tpmlp::XRows{};
  a.x.p[0] = x;
  a.x.nb = 1;
  a.x.rows = (int)M;
  a.x.ld = ldx;
  a.wg = w_gate;
  a.wu = w_up;
  a.ldw_gu = ldw_gu;
  a.wd = w_down;
  a.ldw_down = ldw_down;
  a.sg = s_gate;
  a.su = s_up;
  a.sd = s_down;
  a.p = partial;
  a.ldp = ldp;
  a.a = wsb + l.a;
  a.lda = I_s;
  a.wb = tpmlp::kWeightE4M3;
  a.sk = l.total > l.sk ? wsb + l.sk : nullptr;
  tpmlp::W8A8Bufs b;
  b.xq = wsb + l.xq;
  b.sx = reinterpret_cast<float*>(wsb + l.sx);
  b.aq = wsb + l.aq;
  b.sa = reinterpret_cast<float*>(wsb + l.sa);
  return from_hip(tpmlp::launch_forward_w8a8(a, b, reinterpret_cast<hipStream_t>(stream)), "kernel launch");
}

TP_API tp_status tp_quantize_rows_e4m3(int64_t rows, int64_t cols, const void* x, int64_t ldx, void* codes,
                                       int64_t ldq, float* scales, void* stream) {
  if (rows < 0 || cols < 1) return fail(TP_ERR_INVALID_ARG, "rows must be >= 0 and cols >= 1");
  if (rows == 0) return TP_OK;
  if (rows > kMaxDim || cols > kMaxDim) return fail(TP_ERR_UNSUPPORTED, "dimension above 2^30");
  if (!x || !codes || !scales) return fail(TP_ERR_INVALID_ARG, "null pointer");
  if (ldx < cols || ldq < cols) return fail(TP_ERR_INVALID_ARG, "leading dimension smaller than the row length");
  if (cols % 8 != 0) return fail(TP_ERR_UNSUPPORTED, "cols must be a multiple of 8");
  if (!aligned(x, 16) || (ldx * 2) % 16 || !aligned(codes, 8) || ldq % 8 || !aligned(scales, 4))
    return fail(TP_ERR_UNSUPPORTED, "x rows must be 16-byte aligned, code rows 8-byte aligned");
  const Extent ex = extent(x, rows, cols, ldx, 2), eq = extent(codes, rows, cols, ldq, 1),
               es = extent(scales, 1, rows, rows, 4);
  if (overlap(ex, eq) || overlap(ex, es) || overlap(eq, es))
    return fail(TP_ERR_INVALID_ARG, "buffers overlap");
  return from_hip(tpmlp::launch_quant_rows((int)rows, (int)cols, x, ldx, codes, ldq, scales,
                                           reinterpret_cast<hipStream_t>(stream)),
                  "kernel launch");
}

// ------------------------------------------------------------ attention

namespace {

// Local heads of one rank: query heads split evenly; KV heads split evenly,
// or, when the group is a multiple of the KV-head count, one KV head per rank
// (replicated over t / n_kv_heads ranks).  Returns false if neither holds.
bool attn_local_heads(int64_t n_heads, int64_t n_kv_heads, int32_t t, int64_t* q_loc, int64_t* kv_loc) {
  if (t < 1 || n_heads < 1 || n_kv_heads < 1 || n_heads % t != 0) return false;
  if (n_heads % n_kv_heads != 0) return false;  // grouped-query: whole groups
  if (n_kv_heads % t == 0)
    *kv_loc = n_kv_heads / t;
  else if (t % n_kv_heads == 0)
    *kv_loc = 1;
  else
    return false;
  *q_loc = n_heads / t;
  return true;
}

// Checks and launch shared by the attention projections:
// out (M x N) = a (M x K) * w^T, w N x K, out in the activation dtype
// (out_f32 forces fp32).
// Scratch the projection needs (bytes, before rounding): split-K sums for
// decode, stream-K counters and partial tiles for prefill.
int64_t linear_workspace_need(int64_t M, int64_t N, int64_t K, int32_t act_dtype, int32_t w_dtype) {
  if (act_dtype != TP_BF16) return 0;
  if (M > tpmlp::kDecodeMaxM) return tpmlp::rowgemm_prefill_workspace_bytes((int)M, (int)N, (int)K);
  return tpmlp::rowgemm_decode_workspace_bytes((int)M, (int)N, (int)K, weight_format(w_dtype));
}

tp_status linear_impl(int64_t M, int64_t N, int64_t K, int32_t act_dtype, int32_t w_dtype, const void* a,
                      int64_t lda, const void* w, int64_t ldw, const float* s, void* out, int64_t ldo,
                      bool out_f32, void* workspace, size_t workspace_bytes, bool has_workspace,
                      int kind_decode, int kind_prefill, int kind_f32, void* stream) {
  {
    const tp_status st = check_pair(act_dtype, w_dtype);
    if (st != TP_OK) return st;
  }
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return fail(TP_ERR_UNSUPPORTED, "dimension above 2^30");
  if (act_dtype == TP_BF16 && (K % 64 != 0 || N % 16 != 0))
    return fail(TP_ERR_UNSUPPORTED, "bf16 paths need K %% 64 == 0 and N %% 16 == 0 (K=%lld, N=%lld)",
                (long long)K, (long long)N);
  if (!a || !w || !out) return fail(TP_ERR_INVALID_ARG, "null tensor pointer");
  const bool fp8 = scaled_weights(w_dtype);   // one-byte weights with row scales
  if (fp8 && !s) return fail(TP_ERR_INVALID_ARG, "one-byte weights need their scales");
  if (!fp8 && s) return fail(TP_ERR_INVALID_ARG, "scales are only accepted with one-byte weights");
  if (lda < K || ldw < K || ldo < N)
    return fail(TP_ERR_INVALID_ARG, "leading dimension smaller than the row length (lda=%lld ldw=%lld ldo=%lld)",
                (long long)lda, (long long)ldw, (long long)ldo);
  const int ea = elem_bytes(act_dtype), ew = elem_bytes(w_dtype);
  const int eo = out_f32 ? 4 : ea;
  if (act_dtype == TP_BF16) {
    if (!aligned(a, 16) || !aligned(w, 16) || !aligned(out, 16))
      return fail(TP_ERR_UNSUPPORTED, "tensor pointers must be 16-byte aligned");
    if ((lda * ea) % 16 || (ldw * ew) % 16 || (ldo * eo) % 16)
      return fail(TP_ERR_UNSUPPORTED, "rows must start 16-byte aligned (leading dimensions)");
    if (fp8 && !aligned(s, 4)) return fail(TP_ERR_UNSUPPORTED, "scale pointer must be 4-byte aligned");
  } else if (!aligned(a, 4) || !aligned(w, 4) || !aligned(out, 4)) {
    return fail(TP_ERR_UNSUPPORTED, "fp32 pointers must be 4-byte aligned");
  }
  const Extent e_out = extent(out, M, N, ldo, eo);
  if (overlap(e_out, extent(a, M, K, lda, ea)) || overlap(e_out, extent(w, N, K, ldw, ew)) ||
      (s && overlap(e_out, extent(s, 1, N, N, 4))))
    return fail(TP_ERR_INVALID_ARG, "output overlaps an input");
  const int64_t need = has_workspace ? linear_workspace_need(M, N, K, act_dtype, w_dtype) : 0;
  if (need > 0) {
    if (!workspace || (int64_t)workspace_bytes < need)
      return fail(TP_ERR_WORKSPACE, "workspace of %lld bytes needed (got %llu)", (long long)need,
                  (unsigned long long)workspace_bytes);
    if (!aligned(workspace, 256)) return fail(TP_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
    const Extent ew_ = {reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + (uintptr_t)need};
    if (overlap(ew_, e_out) || overlap(ew_, extent(a, M, K, lda, ea)) || overlap(ew_, extent(w, N, K, ldw, ew)) ||
        (s && overlap(ew_, extent(s, 1, N, N, 4))))
      return fail(TP_ERR_INVALID_ARG, "workspace overlaps an input or the output");
  }

  tpmlp::RowGemm g;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.a = a;
  g.lda = lda;
  g.w = w;
  g.ldw = ldw;
  g.s = s;
  g.out = out;
  g.ldo = ldo;
  g.out_bf16 = act_dtype == TP_BF16 && !out_f32;
  g.wb = weight_format(w_dtype);
  g.ws = need > 0 ? static_cast<float*>(workspace) : nullptr;
  g.kind_decode = kind_decode;
  g.kind_prefill = kind_prefill;
  g.kind_f32 = kind_f32;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (act_dtype == TP_F32)
    e = tpmlp::launch_rowgemm_f32(g, st);
  else if (M <= tpmlp::kDecodeMaxM)
    e = tpmlp::launch_rowgemm_decode(g, st);
  else
    e = tpmlp::launch_rowgemm_prefill(g, st);
  return from_hip(e, "kernel launch");
}

tp_status check_attn(int64_t M, int64_t h, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, int32_t t,
                     int32_t k, int64_t* q_loc, int64_t* kv_loc) {
  if (M < 1 || h < 1 || head_dim < 1)
    return fail(TP_ERR_INVALID_ARG, "M, h and head_dim must be >= 1 (got %lld, %lld, %lld)", (long long)M,
                (long long)h, (long long)head_dim);
  if (t < 1 || t > tpmlp::kMaxPartials)
    return fail(TP_ERR_INVALID_ARG, "t must be in [1, %d] (got %d)", tpmlp::kMaxPartials, t);
  if (k < 0 || k >= t) return fail(TP_ERR_INVALID_ARG, "k must be in [0, t) (got k=%d, t=%d)", k, t);
  if (!attn_local_heads(n_heads, n_kv_heads, t, q_loc, kv_loc))
    return fail(TP_ERR_INVALID_ARG,
                "heads do not split over t=%d (n_heads=%lld must divide by t and by n_kv_heads=%lld; "
                "n_kv_heads must divide by t or t by n_kv_heads)",
                t, (long long)n_heads, (long long)n_kv_heads);
  if (n_heads * head_dim > kMaxDim) return fail(TP_ERR_UNSUPPORTED, "dimension above 2^30");
  return TP_OK;
}

}  // namespace

TP_API int64_t tp_attn_qkv_width(int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, int32_t t) {
  int64_t q_loc = 0, kv_loc = 0;
  if (head_dim < 1 || head_dim > kMaxDim || t > tpmlp::kMaxPartials ||
      !attn_local_heads(n_heads, n_kv_heads, t, &q_loc, &kv_loc))
    return -1;
  return (q_loc + 2 * kv_loc) * head_dim;
}

TP_API size_t tp_attn_qkv_workspace_bytes(int64_t M, int64_t h, int64_t n_heads, int64_t n_kv_heads,
                                          int64_t head_dim, int32_t t, int32_t act_dtype, int32_t w_dtype) {
  int64_t q_loc = 0, kv_loc = 0;
  if (M < 1 || M > kMaxDim || h < 1 || h > kMaxDim || head_dim < 1 || t < 1 || t > tpmlp::kMaxPartials ||
      !attn_local_heads(n_heads, n_kv_heads, t, &q_loc, &kv_loc) || n_heads * head_dim > kMaxDim)
    return 0;
  if (elem_bytes(act_dtype) == 0 || elem_bytes(w_dtype) == 0) return 0;
  const int64_t n_loc = (q_loc + 2 * kv_loc) * head_dim;
  if (act_dtype == TP_BF16 && (h % 64 != 0 || n_loc % 16 != 0)) return 0;
  return (size_t)round_up(linear_workspace_need(M, n_loc, h, act_dtype, w_dtype), 256);
}

TP_API tp_status tp_attn_qkv_forward(int64_t M, int64_t h, int64_t n_heads, int64_t n_kv_heads,
                                     int64_t head_dim, int32_t t, int32_t k, int32_t act_dtype,
                                     int32_t w_dtype, const void* x, int64_t ldx, const void* w_qkv,
                                     int64_t ldw, const float* s_qkv, void* qkv, int64_t ldq,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  int64_t q_loc = 0, kv_loc = 0;
  tp_status st = check_attn(M, h, n_heads, n_kv_heads, head_dim, t, k, &q_loc, &kv_loc);
  if (st != TP_OK) return st;
  const int64_t n_loc = (q_loc + 2 * kv_loc) * head_dim;
  return linear_impl(M, n_loc, h, act_dtype, w_dtype, x, ldx, w_qkv, ldw, s_qkv, qkv, ldq, false, workspace,
                     workspace_bytes, true, tpmlp::K_QKV_DECODE, tpmlp::K_QKV_PREFILL, tpmlp::K_QKV_F32, stream);
}

TP_API tp_status tp_attn_out_forward(int64_t M, int64_t h, int64_t n_heads, int64_t head_dim, int32_t t,
                                     int32_t k, int32_t act_dtype, int32_t w_dtype, const void* attn,
                                     int64_t lda, const void* w_o, int64_t ldw, const float* s_o,
                                     float* partial, int64_t ldp, void* stream) {
  int64_t q_loc = 0, kv_loc = 0;
  // the output projection sees only the query heads; any KV count that
  // splits them is accepted (n_kv_heads = n_heads)
  tp_status st = check_attn(M, h, n_heads, n_heads, head_dim, t, k, &q_loc, &kv_loc);
  if (st != TP_OK) return st;
  return linear_impl(M, h, q_loc * head_dim, act_dtype, w_dtype, attn, lda, w_o, ldw, s_o, partial, ldp, true,
                     nullptr, 0, false, tpmlp::K_OPROJ_DECODE, tpmlp::K_OPROJ_PREFILL, tpmlp::K_OPROJ_F32,
                     stream);
}

TP_API const char* tp_status_string(int32_t status) {
  switch (status) {
    case TP_OK: return "TP_OK";
    case TP_ERR_INVALID_ARG: return "TP_ERR_INVALID_ARG: invalid argument";
    case TP_ERR_UNSUPPORTED: return "TP_ERR_UNSUPPORTED: valid but unsupported argument";
    case TP_ERR_WORKSPACE: return "TP_ERR_WORKSPACE: workspace missing or too small";
    case TP_ERR_HIP: return "TP_ERR_HIP: HIP runtime error";
    default: return "unknown status";
  }
}

TP_API const char* tp_last_error(void) { return g_last_error; }

TP_API int32_t tp_kernel_kind_count(void) { return tpmlp::K_NUM_KINDS; }

TP_API const char* tp_kernel_kind_name(int32_t kind) {
  if (kind < 0 || kind >= tpmlp::K_NUM_KINDS) return nullptr;
  return kKindNames[kind];
}

TP_API tp_status tp_profile_enable(int32_t kinds) {
  g_prof_mask = (uint32_t)kinds;
  return TP_OK;
}

TP_API tp_status tp_profile_reserve(int64_t records) {
  if (records < 0) return fail(TP_ERR_INVALID_ARG, "negative record count");
  while ((int64_t)g_prof_pool.size() < records)
    if (!prof_grow()) return fail(TP_ERR_HIP, "hipEventCreate failed while reserving timing records");
  return TP_OK;
}

TP_API tp_status tp_profile_durations(int32_t kind, float* ms, int64_t capacity, int64_t* n) {
  if (!n || capacity < 0 || (capacity > 0 && !ms)) return fail(TP_ERR_INVALID_ARG, "bad output arrays");
  int64_t k = 0;
  for (size_t i = 0; i < g_prof_used; ++i) {
    ProfRec& r = g_prof_pool[i];
    if (r.kind != kind) continue;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return from_hip(e, "hipEventSynchronize");
    float v = 0.f;
    e = hipEventElapsedTime(&v, r.start, r.stop);
    if (e != hipSuccess) return from_hip(e, "hipEventElapsedTime");
    if (k < capacity) ms[k] = v;
    ++k;
  }
  *n = k;
  return TP_OK;
}

TP_API tp_status tp_profile_collect(double* total_ms, int64_t* counts, int32_t n_kinds) {
  if (!total_ms || !counts || n_kinds < 0) return fail(TP_ERR_INVALID_ARG, "bad output arrays");
  for (size_t i = 0; i < g_prof_used; ++i) {
    ProfRec& r = g_prof_pool[i];
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) {
      g_prof_used = 0;
      return from_hip(e, "hipEventSynchronize");
    }
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) {
      g_prof_used = 0;
      return from_hip(e, "hipEventElapsedTime");
    }
    if (r.kind < n_kinds) {
      total_ms[r.kind] += ms;
      counts[r.kind] += 1;
    }
  }
  g_prof_used = 0;
  return TP_OK;
}
