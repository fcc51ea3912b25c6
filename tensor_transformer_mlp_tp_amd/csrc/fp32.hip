// fp32 activations with fp32 weights: the full-precision variant of the same
// rank forward (column-parallel gate/up with SiLU(gate) * up applied locally,
// then the row-parallel down projection to an fp32 partial; "The
// Tensor-Parallel Shard Group", scalablesystem.dev).
//
// The same row kernel serves the attention block's projections in fp32.
//
// This is the precision path for small problems and checks, not a
// throughput path: one wave per output element, lanes split the dot product
// and a butterfly of cross-lane adds finishes it (every lane ends with the
// same bits, so the result is deterministic).  fp32 FMA accumulation.
#include "common.h"
#include "internal.h"

namespace tpmlp {

namespace {

constexpr int kF32Waves = 4;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = v + __shfl_xor(v, off);
  return v;
}

__global__ __launch_bounds__(kF32Waves * 64) void gateup_f32_kernel(
    int M, int h, int I_s, const XRows xrows,
    const float* __restrict__ wg, const float* __restrict__ wu, int64_t ldw,
    float* __restrict__ a_out, int64_t lda) {
  const int lane = threadIdx.x & 63;
  const int64_t id = (int64_t)blockIdx.x * kF32Waves + (threadIdx.x >> 6);
  if (id >= (int64_t)M * I_s) return;  // whole wave leaves together
  const int m = (int)(id / I_s), j = (int)(id % I_s);
  const float* xr = x_row<float>(xrows, m);
  const float* gr = wg + (int64_t)j * ldw;
  const float* ur = wu + (int64_t)j * ldw;
  float g = 0.f, u = 0.f;
  for (int i = lane; i < h; i += 64) {
    const float xv = xr[i];
    g = fmaf(xv, gr[i], g);
    u = fmaf(xv, ur[i], u);
  }
  g = wave_sum(g);
  u = wave_sum(u);
  if (lane == 0) a_out[(int64_t)m * lda + j] = silu(g) * u;
}

__global__ __launch_bounds__(kF32Waves * 64) void down_f32_kernel(
    int M, int h, int I_s, const float* __restrict__ a_in, int64_t lda,
    const float* __restrict__ wd, int64_t ldw, float* __restrict__ p, int64_t ldp) {
  const int lane = threadIdx.x & 63;
  const int64_t id = (int64_t)blockIdx.x * kF32Waves + (threadIdx.x >> 6);
  if (id >= (int64_t)M * h) return;
  const int m = (int)(id / h), n = (int)(id % h);
  const float* ar = a_in + (int64_t)m * lda;
  const float* dr = wd + (int64_t)n * ldw;
  float s = 0.f;
  for (int j = lane; j < I_s; j += 64) s = fmaf(ar[j], dr[j], s);
  s = wave_sum(s);
  if (lane == 0) p[(int64_t)m * ldp + n] = s;
}

}  // namespace

hipError_t launch_rowgemm_f32(const RowGemm& g, hipStream_t stream) {
  const int64_t blocks = ((int64_t)g.M * g.N + kF32Waves - 1) / kF32Waves;
  return launch(g.kind_f32, down_f32_kernel, dim3((unsigned)blocks), dim3(kF32Waves * 64), 0, stream, g.M,
                g.N, g.K, (const float*)g.a, g.lda, (const float*)g.w, g.ldw, (float*)g.out, g.ldo);
}

hipError_t launch_forward_f32(const ShardArgs& a, hipStream_t stream) {
  const dim3 block(kF32Waves * 64);
  const int64_t g1 = ((int64_t)a.M * a.I_s + kF32Waves - 1) / kF32Waves;
  hipError_t e = launch(K_GATEUP_F32, gateup_f32_kernel, dim3((unsigned)g1), block, 0, stream, a.M,
                        a.h, a.I_s, a.x, (const float*)a.wg,
                        (const float*)a.wu, a.ldw_gu, (float*)a.a, a.lda);
  if (e != hipSuccess) return e;
  return launch_rowgemm_f32(down_of(a), stream);
}

}  // namespace tpmlp
