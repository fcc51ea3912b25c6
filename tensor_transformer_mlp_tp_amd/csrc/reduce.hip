// Fixed-order sum of t fp32 partial buffers (the local half of the all-reduce
// that follows the row-parallel down projection: "The Tensor-Parallel Shard
// Group", scalablesystem.dev; Z = sum_k Z_k in section 12.2.1 of the
// arunshar.com chapter).
//
// out[i] = (((p0[i] + p1[i]) + p2[i]) + ...) + p_{t-1}[i], binary32 adds in
// exactly that order.  The kernel is HBM-bound: (t + 1) * 4 bytes per element.
// Each thread owns UNROLL float4 positions spaced one block apart, issues all
// t * UNROLL 16-byte loads before the first add (for compile-time t), and
// writes each float4 once.
#include "common.h"
#include "internal.h"

namespace tpmlp {

namespace {

// Block shape: 1024 threads for the large (bandwidth-bound) reduces, 256 for
// small ones (a decode partial of a few hundred KB), where more blocks
// finish sooner.
constexpr int kReduceThreadsSmall = 256;
constexpr int64_t kReduceSmallN4 = 1 << 20;
constexpr int kReduceThreads = 1024;
constexpr int kReduceUnroll = 1;

// Loads are non-temporal: every input byte is read exactly once.  Stores:
// when the output fits well inside the 256 MB last-level cache, plain stores
// (written back later, interleaved with the read streams) measured about 3 %
// faster than streaming stores on MI355X; for larger outputs that write-back
// thrashes the cache and streaming stores are faster (5 % at 512 MiB).
constexpr int64_t kReducePlainStoreMaxBytes = 192ll << 20;

__device__ __forceinline__ f32x4 ld4(const f32x4* p) { return __builtin_nontemporal_load(p); }

template <bool NTS>
__device__ __forceinline__ void st4(f32x4 v, f32x4* p) {
  if constexpr (NTS) __builtin_nontemporal_store(v, p);
  else *p = v;
}

template <int T, int THREADS, bool NTS>
__global__ __launch_bounds__(THREADS) void partial_reduce_kernel(
    PartialPtrs ptrs, int t_rt, float* __restrict__ out, int64_t n) {
  const int t = T > 0 ? T : t_rt;
  const int64_t n4 = n >> 2;
  const int64_t base = (int64_t)blockIdx.x * (THREADS * kReduceUnroll) + threadIdx.x;

  f32x4 acc[kReduceUnroll];
  bool ok[kReduceUnroll];
#pragma unroll
  for (int u = 0; u < kReduceUnroll; ++u) {
    const int64_t idx = base + (int64_t)u * THREADS;
    ok[u] = idx < n4;
    acc[u] = ok[u] ? ld4(reinterpret_cast<const f32x4*>(ptrs.p[0]) + idx)
                   : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if constexpr (T > 0) {
    f32x4 v[T > 1 ? T - 1 : 1][kReduceUnroll];
#pragma unroll
    for (int j = 1; j < T; ++j)
#pragma unroll
      for (int u = 0; u < kReduceUnroll; ++u) {
        const int64_t idx = base + (int64_t)u * THREADS;
        v[j - 1][u] = ok[u] ? ld4(reinterpret_cast<const f32x4*>(ptrs.p[j]) + idx)
                            : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int j = 1; j < T; ++j)
#pragma unroll
      for (int u = 0; u < kReduceUnroll; ++u) acc[u] = acc[u] + v[j - 1][u];
  } else {
    for (int j = 1; j < t; ++j) {
#pragma unroll
      for (int u = 0; u < kReduceUnroll; ++u) {
        const int64_t idx = base + (int64_t)u * THREADS;
        if (ok[u]) acc[u] = acc[u] + ld4(reinterpret_cast<const f32x4*>(ptrs.p[j]) + idx);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kReduceUnroll; ++u) {
    const int64_t idx = base + (int64_t)u * THREADS;
    if (ok[u]) st4<NTS>(acc[u], reinterpret_cast<f32x4*>(out) + idx);
  }

  // n % 4 trailing elements: the first block's first threads, scalar.
  if (blockIdx.x == 0) {
    const int64_t tail = n - (n4 << 2);
    if (threadIdx.x < tail) {
      const int64_t i = (n4 << 2) + threadIdx.x;
      float s = ptrs.p[0][i];
      for (int j = 1; j < t; ++j) s = s + ptrs.p[j][i];
      out[i] = s;
    }
  }
}

template <int THREADS, bool NTS>
hipError_t launch_reduce_shape(const PartialPtrs& ptrs, int t, float* out, int64_t n, hipStream_t stream) {
  const int64_t n4 = n >> 2;
  const int64_t per_block = (int64_t)THREADS * kReduceUnroll;
  int64_t blocks = (n4 + per_block - 1) / per_block;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks), block(THREADS);
  switch (t) {
    case 1: return launch(K_PARTIAL_REDUCE, partial_reduce_kernel<1, THREADS, NTS>, grid, block, 0, stream, ptrs, t, out, n);
    case 2: return launch(K_PARTIAL_REDUCE, partial_reduce_kernel<2, THREADS, NTS>, grid, block, 0, stream, ptrs, t, out, n);
    case 4: return launch(K_PARTIAL_REDUCE, partial_reduce_kernel<4, THREADS, NTS>, grid, block, 0, stream, ptrs, t, out, n);
    case 8: return launch(K_PARTIAL_REDUCE, partial_reduce_kernel<8, THREADS, NTS>, grid, block, 0, stream, ptrs, t, out, n);
    default: return launch(K_PARTIAL_REDUCE, partial_reduce_kernel<0, THREADS, NTS>, grid, block, 0, stream, ptrs, t, out, n);
  }
}

}  // namespace

hipError_t launch_partial_reduce(const PartialPtrs& ptrs, int t, float* out, int64_t n,
                                 hipStream_t stream) {
  if ((n >> 2) < kReduceSmallN4) return launch_reduce_shape<kReduceThreadsSmall, false>(ptrs, t, out, n, stream);
  if (n * 4 <= kReducePlainStoreMaxBytes) return launch_reduce_shape<kReduceThreads, false>(ptrs, t, out, n, stream);
  return launch_reduce_shape<kReduceThreads, true>(ptrs, t, out, n, stream);
}

}  // namespace tpmlp
