// Pieces shared by the attention kernels: the work-item decode with an
// XCD-aware order, and the per-work-group row walker that gathers key rows of
// a subsequence (the rearrange of the OSP-Next summary, 核心方法 core method,
// with the any-resolution prefix boxes of 方法步骤详情 method steps).
#pragma once

#include "internal.h"

namespace skiparse {

constexpr int kRowCap = 2048;   // capacity of the (t, h') row table
constexpr int kColCap = 512;    // capacity of the w' column table

// Work-groups are handed to the 8 XCDs round-robin.  Give each XCD one
// contiguous range of logical tiles, so the query tiles that stream the same
// subsequence's K/V run side by side on one XCD and share its L2.
__device__ __forceinline__ int xcd_remap(int i, int n) {
  constexpr int X = 8;
  int xcd = i % X, local = i / X;
  int per = n / X, rem = n % X;
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + local;
}

// (batch, head, subsequence, query tile) of a work-group.
struct WorkItem {
  int b, head, qtile;
  SubGeom sg;
};

__device__ __forceinline__ WorkItem decode_work(const AttnArgs& a) {
  WorkItem w;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = wg / a.tiles_per_bh;
  const int rem = wg - bh * a.tiles_per_bh;
  w.b = bh / a.heads;
  w.head = bh - w.b * a.heads;
  int si = 0;
  while (si + 1 < a.n_run && a.sub[si + 1].tile0 <= rem) ++si;
  w.sg = a.sub[si];
  w.qtile = rem - w.sg.tile0;
  return w;
}

// Fill the LDS tables of a subsequence: rowbase[t*hr + h'] = (t*H + h)*W and
// colmap[w'] = w, so a compact member j = th*wr + w' sits at token
// rowbase[th] + colmap[w'].  Ends with a barrier.
__device__ __forceinline__ void build_row_tables(const AttnArgs& a, const SubGeom& sg, int32_t* rowbase,
                                                 int32_t* colmap, int nthreads) {
  const int wr = (int)sg.div_w.d;
  const int th_end = sg.n / wr;
  const int hr = th_end / a.g.T;
  for (int x = threadIdx.x; x < th_end; x += nthreads) {
    const int t = x / hr;
    const int hh = (int)h_of_local((uint32_t)(x - t * hr), (uint32_t)sg.p, a.g);
    rowbase[x] = (t * a.g.H + hh) * a.g.W;
  }
  for (int x = threadIdx.x; x < wr; x += nthreads) colmap[x] = (int)w_of_local((uint32_t)x, (uint32_t)sg.q, a.g);
  __syncthreads();
}

// Walks one key row through consecutive tiles of TILE rows: compact index
// j = tile*TILE + r = th*wr + w', advanced by TILE = dth*wr + dw per step.
// Rows past the end of the subsequence return the last member's token.
template <int TILE>
struct RowWalker {
  int th, w, dth, dw, wr, th_end, tok_last;

  __device__ __forceinline__ void init(const SubGeom& sg, int r, const int32_t* rowbase, const int32_t* colmap) {
    wr = (int)sg.div_w.d;
    th_end = sg.n / wr;
    th = r / wr;
    w = r - th * wr;
    dth = TILE / wr;
    dw = TILE - dth * wr;
    const int jl = sg.n - 1;
    const int tl = jl / wr;
    tok_last = rowbase[tl] + colmap[jl - tl * wr];
  }
  // token of the current row, then step to the next tile
  __device__ __forceinline__ int next(const int32_t* rowbase, const int32_t* colmap) {
    const int tok = th < th_end ? rowbase[th] + colmap[w] : tok_last;
    w += dw;
    const int cy = w >= wr;
    w -= cy ? wr : 0;
    th += dth + cy;
    return tok;
  }
};

// Whether 32-bit row offsets work: 24-bit tokens and row strides, and a
// batch sample's tensor below 4 GB.
inline bool offsets32_ok(const AttnArgs& a, int64_t row_bytes) {
  const int64_t tokens = (int64_t)a.g.T * a.g.H * a.g.W;
  return tokens < (1 << 24) && row_bytes < (1 << 24) && tokens * row_bytes < (int64_t(1) << 32);
}

// Whether every run subsequence holds at most cap members (its whole token
// list then fits one LDS table) and 32-bit offsets work.
inline bool token_table_ok(const AttnArgs& a, int64_t row_bytes, int cap) {
  bool ok = offsets32_ok(a, row_bytes);
  for (int i = 0; i < a.n_run && ok; ++i) ok = a.sub[i].n <= cap;
  return ok;
}

// Whether every run subsequence fits the row/column tables and 32-bit
// offsets work.
inline bool fast_rows_ok(const AttnArgs& a, int64_t row_bytes) {
  bool fast = offsets32_ok(a, row_bytes);
  for (int i = 0; i < a.n_run && fast; ++i) {
    const SubGeom& s = a.sub[i];
    if (s.n == 0) continue;
    const int64_t th = s.n / (int64_t)s.div_w.d;
    fast = th <= kRowCap && (int64_t)s.div_w.d <= kColCap;
  }
  return fast;
}

}  // namespace skiparse
