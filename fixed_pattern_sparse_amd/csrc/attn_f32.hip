// Skiparse-2D attention forward in fp32 (fp32 in, fp32 out), the
// full-precision path of the library.  Same method as the bf16 kernel
// (OSP-Next summary, 核心方法 core method and 方法步骤详情 method steps), on
// the vector ALUs: one lane per query, an exact online softmax over the keys
// of the query's subsequence, K/V rows staged through LDS 64 at a time.
#include "internal.h"

namespace skiparse {
namespace {

constexpr int kRows = 64;   // queries per work-group (one wave)
constexpr int kKeys = 32;   // keys per LDS tile

template <int D>
__global__ void __launch_bounds__(64) attn_fwd_f32_kernel(const AttnArgs a) {
  __shared__ float sK[kKeys][D + 1];
  __shared__ float sV[kKeys][D + 1];
  const int lane = threadIdx.x;
  const int bh = blockIdx.x / a.tiles_per_bh;
  const int rem = blockIdx.x - bh * a.tiles_per_bh;
  const int b = bh / a.heads;
  const int head = bh - b * a.heads;
  int si = 0;
  while (si + 1 < a.n_run && a.sub[si + 1].tile0 <= rem) ++si;
  const SubGeom sg = a.sub[si];
  const int n = sg.n;
  const int j = (rem - sg.tile0) * kRows + lane;
  const bool ok = j < n;
  const int64_t base = (int64_t)b * a.batch_stride + (int64_t)head * D;
  const float* __restrict__ qp = (const float*)a.q + base;
  const float* __restrict__ kp = (const float*)a.k + base;
  const float* __restrict__ vp = (const float*)a.v + base;
  float* __restrict__ op = (float*)a.o + base;
  const int64_t rs = a.row_stride;

  const int64_t qoff = (int64_t)token_of((uint32_t)(ok ? j : n - 1), sg, a.g) * rs;
  float q[D], acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) { q[e] = qp[qoff + e]; acc[e] = 0.f; }
  const float scale = a.scale;
  float m = -INFINITY, l = 0.f;

  for (int t0 = 0; t0 < n; t0 += kKeys) {
    const int cnt = n - t0 < kKeys ? n - t0 : kKeys;
    __syncthreads();
    if (lane < cnt) {
      const int64_t off = (int64_t)token_of((uint32_t)(t0 + lane), sg, a.g) * rs;
      for (int e = 0; e < D; ++e) { sK[lane][e] = kp[off + e]; sV[lane][e] = vp[off + e]; }
    }
    __syncthreads();
    for (int y = 0; y < cnt; ++y) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) dot = __builtin_fmaf(q[e], sK[y][e], dot);
      const float sc = dot * scale;
      const float mn = fmaxf(m, sc);
      const float alpha = expf(m - mn);
      const float p = expf(sc - mn);
      l = l * alpha + p;
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = __builtin_fmaf(p, sV[y][e], acc[e] * alpha);
      m = mn;
    }
  }
  if (ok) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < D; ++e) op[qoff + e] = acc[e] * inv;
  }
}

template <int D>
hipError_t launch_d(AttnArgs a, int B, hipStream_t stream) {
  assign_tiles(a, B, kRows);
  if (a.total_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(attn_fwd_f32_kernel<D>, dim3(a.total_tiles), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(AttnArgs a, int B, int d, hipStream_t stream) {
  if (d == 128) return launch_d<128>(a, B, stream);
  return launch_d<64>(a, B, stream);
}

}  // namespace skiparse
