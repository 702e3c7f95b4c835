// Index function of the Skiparse rearrange, shared by the host plan and every
// device kernel of libskiparse.
//
// Rule along one axis with stride k (OSP-Next summary, 核心方法 core method;
// 方法步骤详情 method steps):
//   token-wise:  x = x' * k + p                      (pixel unshuffle)
//   group-wise:  x = (x' / k) * k^2 + p * k + x' % k  (patch unshuffle, block index mod k)
// Skiparse-2D applies it to h (stride kh = k, coordinate p) and w (kw = k, q).
// Skiparse-1D applies it to each frame's flattened l = h*W + w with stride
// K = k*k (技术新颖性 novelty: the 2D pattern is the 1D one per axis): the
// kernels see the grid (T, 1, H*W) with kh = 1 and kw = K.  Either way the
// real tokens of subsequence s = p*kw + q fill the prefix box
// [0,T) x [0,Hr(p)) x [0,Wr(q)) of its local grid, so the kernels enumerate a
// subsequence compactly, j = (t * Hr + h') * Wr + w', j in [0, T*Hr*Wr), and
// never touch padding.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define SK_HD __host__ __device__ __forceinline__
#else
#define SK_HD inline
#endif

namespace skiparse {

// Exact unsigned division n / d for 0 <= n < 2^31 and 1 <= d < 2^31 by a
// multiply-high, add and shift (round-up multiplier, Granlund & Montgomery,
// "Division by invariant integers using multiplication", PLDI 1994):
//   l = ceil(log2 d),  m = floor(2^32 (2^l - d) / d) + 1,
//   n / d = (mulhi(n, m) + n) >> l.
struct FastDiv {
  uint32_t d;
  uint32_t m;
  uint32_t l;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
  FastDiv f;
  f.d = d;
  f.m = (uint32_t)m;
  f.l = l;
  return f;
}

SK_HD uint32_t mulhi32(uint32_t a, uint32_t b) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __umulhi(a, b);
#else
  return (uint32_t)(((uint64_t)a * b) >> 32);
#endif
}

SK_HD uint32_t fdiv(uint32_t n, const FastDiv& f) { return (mulhi32(n, f.m) + n) >> f.l; }

// Geometry of one subsequence as the kernels see it.
struct SubGeom {
  int32_t n;         // real tokens T * hr * wr
  int32_t p, q;      // subsequence coordinates
  int32_t tile0;     // first query tile of this subsequence within a (b, head)
  FastDiv div_hw;    // division by hr * wr (div_hw.d == hr * wr)
  FastDiv div_w;     // division by wr      (div_w.d == wr)
};

// Call-wide geometry: the grid the kernels index (T, H, W; for Skiparse-1D
// (T, 1, H*W)) and the stride along each axis.
struct Geom {
  int32_t T, H, W;
  int32_t kh, kw;    // strides along h and w (1 leaves the axis whole)
  int32_t rule;      // 0 token-wise, 1 group-wise (a stride of 1 behaves as either)
  FastDiv div_kh, div_kw;
};

// Spatial index of local coordinate xl on an axis of stride k and
// subsequence coordinate p.
SK_HD uint32_t axis_of_local(uint32_t xl, uint32_t p, uint32_t k, const FastDiv& div_k, int32_t rule) {
  if (rule == 0) return xl * k + p;
  uint32_t blk = fdiv(xl, div_k);
  return blk * k * k + p * k + (xl - blk * k);
}
SK_HD uint32_t h_of_local(uint32_t xl, uint32_t p, const Geom& g) { return axis_of_local(xl, p, (uint32_t)g.kh, g.div_kh, g.rule); }
SK_HD uint32_t w_of_local(uint32_t xl, uint32_t q, const Geom& g) { return axis_of_local(xl, q, (uint32_t)g.kw, g.div_kw, g.rule); }

// Flat token index (t*H + h)*W + w of compact member j of subsequence s.
SK_HD uint32_t token_of(uint32_t j, const SubGeom& s, const Geom& g) {
  uint32_t t = fdiv(j, s.div_hw);
  uint32_t r = j - t * s.div_hw.d;
  uint32_t hl = fdiv(r, s.div_w);
  uint32_t wl = r - hl * s.div_w.d;
  uint32_t h = h_of_local(hl, (uint32_t)s.p, g);
  uint32_t w = w_of_local(wl, (uint32_t)s.q, g);
  return (t * (uint32_t)g.H + h) * (uint32_t)g.W + w;
}

}  // namespace skiparse
