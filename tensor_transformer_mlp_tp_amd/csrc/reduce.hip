// Fixed-order sum of t fp32 partial buffers (the local half of the all-reduce
// that follows the row-parallel down projection: "The Tensor-Parallel Shard
// Group", scalablesystem.dev; Z = sum_k Z_k in section 12.2.1 of the
// arunshar.com chapter).
//
// out[i] = (((p0[i] + p1[i]) + p2[i]) + ...) + p_{t-1}[i], binary32 adds in
// exactly that order.  The kernel is HBM-bound: (t + 1) * 4 bytes per element.
// Each thread owns UNROLL float4 positions spaced one block apart, issues all
// t * UNROLL 16-byte loads before the first add (for compile-time t), and
// writes each float4 once.  Loads and stores are non-temporal: every byte is
// touched exactly once, so there is no reuse to keep in L2 / the MALL.
#include "common.h"
#include "internal.h"

namespace tpmlp {

namespace {

constexpr int kReduceThreads = 256;
constexpr int kReduceUnroll = 2;

template <int T>
__global__ __launch_bounds__(kReduceThreads) void partial_reduce_kernel(
    PartialPtrs ptrs, int t_rt, float* __restrict__ out, int64_t n) {
  const int t = T > 0 ? T : t_rt;
  const int64_t n4 = n >> 2;
  const int64_t base = (int64_t)blockIdx.x * (kReduceThreads * kReduceUnroll) + threadIdx.x;

  f32x4 acc[kReduceUnroll];
  bool ok[kReduceUnroll];
#pragma unroll
  for (int u = 0; u < kReduceUnroll; ++u) {
    const int64_t idx = base + (int64_t)u * kReduceThreads;
    ok[u] = idx < n4;
    acc[u] = ok[u] ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(ptrs.p[0]) + idx)
                   : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if constexpr (T > 0) {
    f32x4 v[T > 1 ? T - 1 : 1][kReduceUnroll];
#pragma unroll
    for (int j = 1; j < T; ++j)
#pragma unroll
      for (int u = 0; u < kReduceUnroll; ++u) {
        const int64_t idx = base + (int64_t)u * kReduceThreads;
        v[j - 1][u] = ok[u] ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(ptrs.p[j]) + idx)
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
        const int64_t idx = base + (int64_t)u * kReduceThreads;
        if (ok[u]) acc[u] = acc[u] + __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(ptrs.p[j]) + idx);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kReduceUnroll; ++u) {
    const int64_t idx = base + (int64_t)u * kReduceThreads;
    if (ok[u]) __builtin_nontemporal_store(acc[u], reinterpret_cast<f32x4*>(out) + idx);
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

}  // namespace

hipError_t launch_partial_reduce(const PartialPtrs& ptrs, int t, float* out, int64_t n,
                                 hipStream_t stream) {
  const int64_t n4 = n >> 2;
  const int64_t per_block = (int64_t)kReduceThreads * kReduceUnroll;
  int64_t blocks = (n4 + per_block - 1) / per_block;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks), block(kReduceThreads);
  switch (t) {
    case 1: return launch(K_PARTIAL_REDUCE, partial_reduce_kernel<1>, grid, block, 0, stream, ptrs, t, out, n);
    case 2: return launch(K_PARTIAL_REDUCE, partial_reduce_kernel<2>, grid, block, 0, stream, ptrs, t, out, n);
    case 4: return launch(K_PARTIAL_REDUCE, partial_reduce_kernel<4>, grid, block, 0, stream, ptrs, t, out, n);
    case 8: return launch(K_PARTIAL_REDUCE, partial_reduce_kernel<8>, grid, block, 0, stream, ptrs, t, out, n);
    default: return launch(K_PARTIAL_REDUCE, partial_reduce_kernel<0>, grid, block, 0, stream, ptrs, t, out, n);
  }
}

}  // namespace tpmlp
