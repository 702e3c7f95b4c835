// Device helpers shared by the per-tensor fp8 quantizers: bf16 widening,
// saturating e4m3 conversion and work-group max reduction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skiparse {

constexpr int kQuantThreads = 256;
constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Max over a work-group of kQuantThreads threads; every thread gets it.
__device__ __forceinline__ float block_max(float v) {
  __shared__ float part[kQuantThreads / 64];
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = part[0];
#pragma unroll
  for (int i = 1; i < kQuantThreads / 64; ++i) r = fmaxf(r, part[i]);
  return r;
}

// Four e4m3 codes of a*s, b*s, c*s, d*s (lowest byte first): the fp32
// product is clamped to +-448 and converted by v_cvt_pk_fp8_f32 (round to
// nearest even), which equals round-to-nearest-even with saturation.
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d, float s) {
  auto sat = [](float v) { return fminf(fmaxf(v, -kE4M3Max), kE4M3Max); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a * s), sat(b * s), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(c * s), sat(d * s), w, true);
  return (uint32_t)w;
}

}  // namespace skiparse
