// Per-tensor 8-bit quantization with the pages' scale rule
// scale = FP8max / (Amax + eps), Amax = max |x| over the whole tensor, one
// scale per tensor (OSP-Next summary, 方法步骤详情 method steps).  The pages'
// HiF8 format is replaced by OCP e4m3 (largest finite value 448).
//
// Three streaming passes, all HBM-bound:
//   1. per-work-group max |x| into the workspace (16-byte loads); a NaN
//      anywhere makes the maximum NaN;
//   2. one work-group reduces the partial maxima and writes {scale, 1/scale},
//      each an IEEE fp32 division;
//   3. y = e4m3(x * scale): the fp32 product is clamped to +-448 and
//      converted by v_cvt_pk_fp8_f32 (round to nearest even), which equals
//      round-to-nearest-even with saturation.
#include <atomic>
#include <mutex>

#include "fp8_codec.h"
#include "block.h"

namespace skiparse {
namespace {

constexpr int kThreads = kQuantThreads;
constexpr int kMaxBlocks = 2048;

template <bool BF16>
__global__ void __launch_bounds__(kThreads) amax_partial_kernel(const void* __restrict__ x, int64_t numel,
                                                                 float* __restrict__ part) {
  uint32_t m = 0;                    // bits of max |x|, NaN-propagating
  constexpr int VE = BF16 ? 8 : 4;   // elements per 16-byte vector
  const int64_t nvec = numel / VE;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride) {
    const uint4 u = ((const uint4*)x)[i];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    if (BF16) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        m = max(m, abs_bits(bf16_bits_to_f32(w[e] & 0xFFFFu)));
        m = max(m, abs_bits(bf16_bits_to_f32(w[e] >> 16)));
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) m = max(m, abs_bits(__uint_as_float(w[e])));
    }
  }
  if (blockIdx.x == 0) {   // scalar tail
    for (int64_t i = nvec * VE + threadIdx.x; i < numel; i += kThreads) {
      const float v = BF16 ? bf16_bits_to_f32(((const uint16_t*)x)[i]) : ((const float*)x)[i];
      m = max(m, abs_bits(v));
    }
  }
  m = block_max_u32(m);
  if (threadIdx.x == 0) part[blockIdx.x] = __uint_as_float(m);
}

__global__ void __launch_bounds__(kThreads) scale_kernel(const float* __restrict__ part, int nparts, float fp8_max,
                                                         float eps, float* __restrict__ scale) {
  uint32_t mb = 0;
  for (int i = threadIdx.x; i < nparts; i += kThreads) mb = max(mb, abs_bits(part[i]));
  const float m = __uint_as_float(block_max_u32(mb));
  if (threadIdx.x == 0) {
    // a NaN maximum gives a NaN scale, so every code of the tensor is NaN
    const float s = fp8_max / (m + eps);
    scale[0] = s;
    scale[1] = 1.0f / s;
  }
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads) quantize_kernel(const void* __restrict__ x, int64_t numel,
                                                            const float* __restrict__ scale, uint8_t* __restrict__ y) {
  const float s = scale[0];
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  if (BF16) {
    const int64_t nvec = numel / 8;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride) {
      const uint4 u = ((const uint4*)x)[i];
      uint2 o;
      o.x = cvt4(bf16_bits_to_f32(u.x & 0xFFFFu), bf16_bits_to_f32(u.x >> 16), bf16_bits_to_f32(u.y & 0xFFFFu),
                 bf16_bits_to_f32(u.y >> 16), s);
      o.y = cvt4(bf16_bits_to_f32(u.z & 0xFFFFu), bf16_bits_to_f32(u.z >> 16), bf16_bits_to_f32(u.w & 0xFFFFu),
                 bf16_bits_to_f32(u.w >> 16), s);
      ((uint2*)y)[i] = o;
    }
    if (blockIdx.x == 0) {
      for (int64_t i = nvec * 8 + threadIdx.x; i < numel; i += kThreads) {
        const float v = bf16_bits_to_f32(((const uint16_t*)x)[i]);
        y[i] = (uint8_t)(cvt4(v, 0.f, 0.f, 0.f, s) & 0xFF);
      }
    }
  } else {
    const int64_t nvec = numel / 4;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride) {
      const float4 v = ((const float4*)x)[i];
      ((uint32_t*)y)[i] = cvt4(v.x, v.y, v.z, v.w, s);
    }
    if (blockIdx.x == 0) {
      for (int64_t i = nvec * 4 + threadIdx.x; i < numel; i += kThreads)
        y[i] = (uint8_t)(cvt4(((const float*)x)[i], 0.f, 0.f, 0.f, s) & 0xFF);
    }
  }
}

int blocks_for(int64_t numel) {
  int64_t b = (numel + 16383) / 16384;
  if (b < 1) b = 1;
  if (b > kMaxBlocks) b = kMaxBlocks;
  return (int)b;
}

// Scratch of the allocation-free entry point: room for the partial maxima of
// the largest grid (kMaxBlocks work-groups, 8 KiB), so it serves every numel.
// One copy per GPU, held until the process ends; every call on a GPU shares it.
static __device__ __align__(256) float scratch[kMaxBlocks];

constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

size_t quant_workspace_bytes(int64_t numel) { return (size_t)blocks_for(numel) * sizeof(float); }

size_t quant_scratch_bytes() { return sizeof(scratch); }

// Device address of this GPU's copy of the scratch array, looked up once per
// device with that device current.  In host code the array's name is only a
// host-side stand-in, never a device address.
hipError_t quant_scratch(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* a = nullptr;
      e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (a == nullptr) return hipErrorInvalidSymbol;
      p = (float*)a;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_fp8_scale(const float* part, int nparts, float fp8_max, float eps, float* scale,
                            hipStream_t stream) {
  hipLaunchKernelGGL(scale_kernel, dim3(1), dim3(kThreads), 0, stream, part, nparts, fp8_max, eps, scale);
  return hipGetLastError();
}

hipError_t launch_quant_fp8(const void* x, int x_is_bf16, int64_t numel, uint8_t* y, float* scale,
                            float fp8_max, float eps, void* ws, hipStream_t stream) {
  const int nb = blocks_for(numel);
  float* part = (float*)ws;
  if (x_is_bf16)
    hipLaunchKernelGGL(amax_partial_kernel<true>, dim3(nb), dim3(kThreads), 0, stream, x, numel, part);
  else
    hipLaunchKernelGGL(amax_partial_kernel<false>, dim3(nb), dim3(kThreads), 0, stream, x, numel, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scale_kernel, dim3(1), dim3(kThreads), 0, stream, part, nb, fp8_max, eps, scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int qb = nb;
  if (x_is_bf16)
    hipLaunchKernelGGL(quantize_kernel<true>, dim3(qb), dim3(kThreads), 0, stream, x, numel, scale, y);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, dim3(qb), dim3(kThreads), 0, stream, x, numel, scale, y);
  return hipGetLastError();
}

}  // namespace skiparse
