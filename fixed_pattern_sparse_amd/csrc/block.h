// Internal interface of the fp8 attention block: the rotary embedding fused
// with per-tensor quantization, the scale step of the quantizer, and the e4m3
// GEMM.
#pragma once

#include "internal.h"

namespace skiparse {

hipError_t launch_fp8_scale(const float* part, int nparts, float fp8_max, float eps, float* scale,
                            hipStream_t stream);

// Token-major tensor (B, T, H, W, heads, d) seen by the rotary embedding,
// walked in 8-element vectors: vector i belongs to token i / (heads*d/8).
struct RopeGeom {
  int32_t T, H, W, d;          // d a power of two, >= 8
  int32_t dt, dh, dw;          // even, dt + dh + dw == d
  int32_t tab_h, tab_w, tab_len;   // float2 table: t part at 0, h at tab_h, w at tab_w
  uint32_t nvec;               // vectors in the tensor (< 2^31)
  FastDiv div_cv, div_w, div_h, div_t;   // heads*d/8, W, H, T
};

size_t rope_partials_bytes(uint32_t nvec);
hipError_t launch_rope_table(const RopeGeom& r, float theta, float2* tab, hipStream_t stream);
// y = e4m3(rope(x) * scale), scale = 448 / (max |rope(x)| + 1e-12) written as
// {scale, 1/scale}; part holds rope_partials_bytes(r.nvec).
hipError_t launch_rope_quant(const RopeGeom& r, const float2* tab, const void* x, uint8_t* y, float* scale,
                             float* part, hipStream_t stream);

// Y (M x N row-major bf16) = *sx * *sw * X (M x K row-major e4m3) . W (N x K
// row-major e4m3)^T; N and K multiples of 128, 1 <= M, M * K < 2^62.
hipError_t launch_gemm_fp8_bf16(const uint8_t* x, const uint8_t* w, const float* sx, const float* sw, void* y,
                                int64_t M, int N, int K, hipStream_t stream);

}  // namespace skiparse
