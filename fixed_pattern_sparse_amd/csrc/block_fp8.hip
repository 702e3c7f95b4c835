// The 3-axis rotary embedding of the fp8 attention block, fused with the
// per-tensor e4m3 quantization of its output.
//
// The 8-bit DiT quantizes per tensor with scale = FP8max / (Amax + eps)
// (OSP-Next summary, 方法步骤详情 method steps).  Q and K are quantized
// after the rotary embedding, so their Amax is that of the rotated values:
// two streaming passes over the bf16 projection output, the first rotating
// and reducing max |.|, the second rotating again and encoding, so the
// rotated tensor never goes back to memory.
//
// Rotary embedding: head dimension d cut into (d_t, d_h, d_w); inside the part
// of axis a, pair (x_2i, x_2i+1) (i counted from the part's start) turns by
// pos_a * theta^(-2i / d_a), pos_a the token's t, h or w.  The cos/sin of every
// (axis, position, pair) come from a table the first kernel fills in float64;
// when it fits (kTabCap entries), each work-group of the two streaming kernels
// copies it to LDS first, so the four lookups per 16-byte vector are LDS
// reads rather than dependent global loads.
#include <cmath>

#include "fp8_codec.h"
#include "block.h"

namespace skiparse {
namespace {

constexpr int kThreads = kQuantThreads;
constexpr int kMaxBlocks = 2048;
constexpr int kTabCap = 4096;   // table entries staged in LDS (32 KB)

__global__ void rope_table_kernel(RopeGeom r, double log_theta, float2* __restrict__ tab) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= r.tab_len) return;
  int base, half;
  if (i < r.tab_h) {
    base = 0, half = r.dt / 2;
  } else if (i < r.tab_w) {
    base = r.tab_h, half = r.dh / 2;
  } else {
    base = r.tab_w, half = r.dw / 2;
  }
  const int local = i - base;
  const int pos = local / half, pair = local % half;
  const int da = 2 * half;
  const double ang = (double)pos * exp(-(2.0 * pair / da) * log_theta);
  double s, c;
  sincos(ang, &s, &c);
  tab[i] = make_float2((float)c, (float)s);
}

// cos/sin of the pair that starts at even head-dim index e of a token at
// (t, h, w).
__device__ __forceinline__ float2 rope_cs(const RopeGeom& r, const float2* tab, int e, int t, int h, int w) {
  const int p = e >> 1;
  if (e < r.dt) return tab[t * (r.dt >> 1) + p];
  if (e < r.dt + r.dh) return tab[r.tab_h + h * (r.dh >> 1) + (p - (r.dt >> 1))];
  return tab[r.tab_w + w * (r.dw >> 1) + (p - ((r.dt + r.dh) >> 1))];
}

// Rotate the 8 bf16 values of vector i (token tok, head-dim offset e0) into v[8].
__device__ __forceinline__ void rope8(const RopeGeom& r, const float2* tab, uint4 u, uint32_t i, float v[8]) {
  const uint32_t tok = fdiv(i, r.div_cv);
  const uint32_t e0 = (i - tok * r.div_cv.d) * 8u;
  const uint32_t e = e0 & (uint32_t)(r.d - 1);          // d is a power of two
  const uint32_t r1 = fdiv(tok, r.div_w);
  const int w = (int)(tok - r1 * r.div_w.d);
  const uint32_t r2 = fdiv(r1, r.div_h);
  const int h = (int)(r1 - r2 * r.div_h.d);
  const int t = (int)(r2 - fdiv(r2, r.div_t) * r.div_t.d);
  const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = bf16_bits_to_f32(wd[j] & 0xFFFFu);
    const float b = bf16_bits_to_f32(wd[j] >> 16);
    const float2 cs = rope_cs(r, tab, (int)e + 2 * j, t, h, w);
    v[2 * j] = a * cs.x - b * cs.y;
    v[2 * j + 1] = a * cs.y + b * cs.x;
  }
}

// The table as the streaming loop reads it: staged in LDS (LDS_TAB) or global.
template <bool LDS_TAB>
__device__ __forceinline__ const float2* rope_table(const RopeGeom& r, const float2* __restrict__ tab,
                                                    float2* stage) {
  if constexpr (LDS_TAB) {
    for (int k = threadIdx.x; k < r.tab_len; k += kThreads) stage[k] = tab[k];
    __syncthreads();
    return stage;
  } else {
    return tab;
  }
}

template <bool LDS_TAB>
__global__ void __launch_bounds__(kThreads) rope_amax_kernel(RopeGeom r, const float2* __restrict__ gtab,
                                                             const uint4* __restrict__ x, float* __restrict__ part) {
  __shared__ float2 stage[LDS_TAB ? kTabCap : 1];
  const float2* tab = rope_table<LDS_TAB>(r, gtab, stage);
  uint32_t m = 0;   // bits of max |rope(x)|, NaN-propagating
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < r.nvec; i += gridDim.x * kThreads) {
    float v[8];
    rope8(r, tab, x[i], i, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = max(m, abs_bits(v[j]));
  }
  m = block_max_u32(m);
  if (threadIdx.x == 0) part[blockIdx.x] = __uint_as_float(m);
}

template <bool LDS_TAB>
__global__ void __launch_bounds__(kThreads) rope_encode_kernel(RopeGeom r, const float2* __restrict__ gtab,
                                                               const uint4* __restrict__ x,
                                                               const float* __restrict__ scale,
                                                               uint2* __restrict__ y) {
  __shared__ float2 stage[LDS_TAB ? kTabCap : 1];
  const float2* tab = rope_table<LDS_TAB>(r, gtab, stage);
  const float s = scale[0];
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < r.nvec; i += gridDim.x * kThreads) {
    float v[8];
    rope8(r, tab, x[i], i, v);
    y[i] = make_uint2(cvt4(v[0], v[1], v[2], v[3], s), cvt4(v[4], v[5], v[6], v[7], s));
  }
}

int rope_blocks(uint32_t nvec) {
  int64_t b = ((int64_t)nvec + 2047) / 2048;
  return (int)(b < 1 ? 1 : (b > kMaxBlocks ? kMaxBlocks : b));
}

}  // namespace

size_t rope_partials_bytes(uint32_t nvec) { return (size_t)rope_blocks(nvec) * sizeof(float); }

hipError_t launch_rope_table(const RopeGeom& r, float theta, float2* tab, hipStream_t stream) {
  hipLaunchKernelGGL(rope_table_kernel, dim3((r.tab_len + 255) / 256), dim3(256), 0, stream, r,
                     std::log((double)theta), tab);
  return hipGetLastError();
}

hipError_t launch_rope_quant(const RopeGeom& r, const float2* tab, const void* x, uint8_t* y, float* scale,
                             float* part, hipStream_t stream) {
  const int nb = rope_blocks(r.nvec);
  const bool lds = r.tab_len <= kTabCap;
  if (lds)
    hipLaunchKernelGGL(rope_amax_kernel<true>, dim3(nb), dim3(kThreads), 0, stream, r, tab, (const uint4*)x, part);
  else
    hipLaunchKernelGGL(rope_amax_kernel<false>, dim3(nb), dim3(kThreads), 0, stream, r, tab, (const uint4*)x, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_fp8_scale(part, nb, kE4M3Max, 1e-12f, scale, stream);
  if (e != hipSuccess) return e;
  if (lds)
    hipLaunchKernelGGL(rope_encode_kernel<true>, dim3(nb), dim3(kThreads), 0, stream, r, tab, (const uint4*)x, scale,
                       (uint2*)y);
  else
    hipLaunchKernelGGL(rope_encode_kernel<false>, dim3(nb), dim3(kThreads), 0, stream, r, tab, (const uint4*)x,
                       scale, (uint2*)y);
  return hipGetLastError();
}

}  // namespace skiparse
