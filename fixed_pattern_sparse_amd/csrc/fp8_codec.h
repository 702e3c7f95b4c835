// Device helpers shared by the per-tensor fp8 quantizers: bf16 widening,
// saturating e4m3 conversion and a NaN-propagating work-group max.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skiparse {

constexpr int kQuantThreads = 256;
constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Magnitude maxima are taken on the bit patterns of |x| as unsigned integers.
// For non-negative floats that order is the numeric one, and every NaN (sign
// cleared) sorts above +inf, so one NaN anywhere makes the maximum NaN, and
// the per-tensor scale with it, instead of being dropped as fmaxf would.
__device__ __forceinline__ uint32_t abs_bits(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

// Max over a work-group of kQuantThreads threads; every thread gets it.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v) {
  __shared__ uint32_t part[kQuantThreads / 64];
  v = wave_max_u32(v);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = part[0];
#pragma unroll
  for (int i = 1; i < kQuantThreads / 64; ++i) r = max(r, part[i]);
  return r;
}

// Four e4m3 codes of a*s, b*s, c*s, d*s (lowest byte first): the fp32
// product is clamped to +-448 and converted by v_cvt_pk_fp8_f32 (round to
// nearest even), which equals round-to-nearest-even with saturation.  A NaN
// product is kept a NaN through the clamp (fminf/fmaxf alone would turn it
// into -448) and leaves the conversion as the code 0xFF.
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d, float s) {
  auto sat = [](float v) {
    const float c = fminf(fmaxf(v, -kE4M3Max), kE4M3Max);
    return v != v ? __uint_as_float(0x7FC00000u) : c;
  };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a * s), sat(b * s), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(c * s), sat(d * s), w, true);
  return (uint32_t)w;
}

}  // namespace skiparse
