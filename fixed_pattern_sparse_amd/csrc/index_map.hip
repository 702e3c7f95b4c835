// Device copy of the Skiparse-2D index map (OSP-Next summary, 核心方法 core
// method; 方法步骤详情 method steps), written by the same token_of() the
// attention kernels use to gather Q/K/V rows and scatter O rows, so the map
// can be compared bit for bit with an independent implementation.
#include "internal.h"

namespace skiparse {
namespace {

struct MapArgs {
  Geom g;
  int32_t n_sub, sub_h, sub_w;
  int64_t slots;               // sub_len_padded
  SubGeom sub[kMaxRun];
};

__global__ void __launch_bounds__(256) index_map_kernel(const MapArgs a, int32_t* __restrict__ out) {
  const int64_t total = a.slots * a.n_sub;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < total;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int s = (int)(x / a.slots);
    const int64_t slot = x - (int64_t)s * a.slots;
    const int64_t plane = (int64_t)a.sub_h * a.sub_w;
    const int t = (int)(slot / plane);
    const int r = (int)(slot - (int64_t)t * plane);
    const int hl = r / a.sub_w;
    const int wl = r - hl * a.sub_w;
    const SubGeom& sg = a.sub[s];
    int32_t v = -1;
    if (sg.n > 0) {
      const int wr = (int)sg.div_w.d;
      const int hr = (int)(sg.div_hw.d / sg.div_w.d);
      if (hl < hr && wl < wr) {
        const uint32_t j = ((uint32_t)t * (uint32_t)hr + (uint32_t)hl) * (uint32_t)wr + (uint32_t)wl;
        v = (int32_t)token_of(j, sg, a.g);
      }
    }
    out[x] = v;
  }
}

}  // namespace

hipError_t launch_index_map(const Geom& g, const SubGeom* subs, int n_sub, int sub_h, int sub_w,
                            int32_t* out, hipStream_t stream) {
  MapArgs a;
  a.g = g;
  a.n_sub = n_sub;
  a.sub_h = sub_h;
  a.sub_w = sub_w;
  a.slots = (int64_t)g.T * sub_h * sub_w;
  for (int i = 0; i < n_sub; ++i) a.sub[i] = subs[i];
  const int64_t total = a.slots * n_sub;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(index_map_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, out);
  return hipGetLastError();
}

}  // namespace skiparse
