// Internal interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include "geom.h"
#include "skiparse.h"

namespace skiparse {

constexpr int kMaxRun = SKIPARSE_MAX_K * SKIPARSE_MAX_K;

// Arguments of one attention launch, passed to the kernel by value.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const float* descale;     // FP8 only: {s_q, 1/s_q, s_k, 1/s_k, s_v, 1/s_v} on the device
  const float* descale_do;  // FP8 backward only: {s_do, 1/s_do} of dO on the device
  float* lse;               // forward: natural-log softmax log-sum-exp, (B, T*H*W, heads), or NULL
  const void* dout;         // backward: upstream gradient dO, same layout as o
  float* dsum;              // backward: rowsum(dO * O), (B, T*H*W, heads), written by the first kernel
  void* dq;                 // backward outputs, same layout as q
  void* dk;
  void* dv;
  int64_t batch_stride;     // elements per batch sample: T*H*W*heads*d
  int32_t row_stride;       // elements per token: heads*d
  int32_t heads;
  int32_t n_run;            // subsequences in this launch
  int32_t tiles_per_bh;     // query tiles per (b, head), filled by the launcher
  int32_t total_tiles;      // B * heads * tiles_per_bh, filled by the launcher
  float scale;              // softmax scale
  float scale_log2;         // softmax scale * log2(e)
  Geom g;
  SubGeom sub[kMaxRun];
};

// Fill tile0 / tiles_per_bh / total_tiles for query tiles of bm rows.
inline void assign_tiles(AttnArgs& a, int B, int bm) {
  int32_t acc = 0;
  for (int i = 0; i < a.n_run; ++i) {
    a.sub[i].tile0 = acc;
    acc += (a.sub[i].n + bm - 1) / bm;
  }
  a.tiles_per_bh = acc;
  a.total_tiles = acc * a.heads * B;
}

// Launchers; each returns hipGetLastError() after its launch.  They assume the
// ABI layer validated every argument.
hipError_t launch_attn_bf16(AttnArgs a, int B, int d, hipStream_t stream);
hipError_t launch_attn_f32(AttnArgs a, int B, int d, hipStream_t stream);
hipError_t launch_attn_fp8(AttnArgs a, int B, int d, hipStream_t stream);
hipError_t launch_attn_bwd(AttnArgs a, int B, int d, hipStream_t stream);
hipError_t launch_attn_bwd_fp8(AttnArgs a, int B, int d, hipStream_t stream);
hipError_t launch_index_map(const Geom& g, const SubGeom* subs, int n_sub, int sub_h, int sub_w,
                            int32_t* out, hipStream_t stream);
size_t quant_workspace_bytes(int64_t numel);
// The allocation-free quantizer's scratch: its capacity in bytes, and this
// GPU's device address of it (looked up once per device).
size_t quant_scratch_bytes();
hipError_t quant_scratch(float** out);
hipError_t launch_quant_fp8(const void* x, int x_is_bf16, int64_t numel, uint8_t* y, float* scale,
                            float fp8_max, float eps, void* ws, hipStream_t stream);

}  // namespace skiparse
