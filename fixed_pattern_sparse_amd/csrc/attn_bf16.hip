// Skiparse-2D attention forward, bf16 in / bf16 out, fp32 accumulation, on
// CDNA4 (gfx950) matrix cores.
//
// Method (OSP-Next summary, 核心方法 core method and 方法步骤详情 method
// steps): dense softmax attention inside each of the k*k subsequences of the
// token-wise or group-wise rearrange, written back in the original layout;
// padding from the any-resolution rule is never computed.
//
// Work decomposition: one work-group of 8 waves per (batch, head,
// subsequence, tile of 256 queries); each wave owns 32 queries.  Keys are
// streamed in tiles of 64 rows through double-buffered LDS.  Each iteration
// first issues the global loads of the next K/V tile into registers (rows
// gathered straight from the (B, T, H, W, heads, d) tensors, no permuted
// copy), computes on the current tile, then writes the staged rows to the
// other LDS buffer with 16-byte stores.  Plain loads and LDS stores measured
// well ahead of direct global->LDS loads for this access pattern.
//
// Per 64-key tile and 32-query block:
//   S^T = K Q^T    v_mfma_f32_32x32x16_bf16; the transposed orientation
//                  leaves one query per lane, so row statistics need one
//                  cross-half swap and no shuffles;
//   online softmax in the log2 domain against a lazily raised running max:
//                  p = exp2(s c - m) is formed with m as it stands, and only
//                  when a lane's partial sum of p exceeds 2^20 (or is not
//                  finite, as on the first tile) is the tile's max taken, O
//                  and l rescaled and p formed again.  O and l always share
//                  one offset, so the normalized result is exact, and every
//                  p stays below 2^20, far inside fp32 and bf16 range;
//   O^T += V^T P^T  V^T comes from row-major V in LDS through
//                  ds_read_b64_tr_b16; P^T stays in registers as bf16.
#include <type_traits>

#include "attn_common.h"

namespace skiparse {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

constexpr int kBN = 64;            // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;   // queries per work-group
constexpr float kBig = 1048576.0f; // 2^20: bound on a lane's partial sum before the max is raised
constexpr int kTileBytes = kBN * 128 * 2;

__shared__ __attribute__((aligned(16))) char gKV[4 * kTileBytes];   // K0 K1 V0 V1
__shared__ int32_t gRowBase[kRowCap];   // (t*H + h) * W for local row th = t*hr + h'
__shared__ int32_t gColMap[kColCap];    // w for local column w'
constexpr int kTokCap = 24064;          // token table: the whole subsequence
__shared__ int32_t gTok[kTokCap];       // token of compact member j

template <int D>
struct Layout {
  static constexpr int CH = D / 8;             // 16-byte chunks per row
  static constexpr int ROWB = D * 2;           // bytes per row
  static constexpr int CPT = kBN * CH / kThreads;  // chunks per thread per tile and matrix
  static constexpr int RSTEP = kThreads / CH;  // row distance between a thread's chunks
  // XOR swizzles of the 16-byte chunk index: K rows are read 32 at a time at
  // one chunk (ds_read_b128), V rows 8 at a time over 4 chunks
  // (ds_read_b64_tr_b16); both patterns hit every bank group evenly.
  __device__ static int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static int vswz(int r) { return D == 128 ? ((r & 3) << 2) : ((r & 1) << 2); }
};

// ROWS selects where a key row's token comes from.  3: the token is the
// member index (stride 1 on both axes: k = 1, the whole grid in its own
// order); 2: a table of the whole subsequence's tokens, written once per
// work-group (n <= kTokCap); 1: a walker over the (t, h') row and w' column
// tables (table room needed); these use 32-bit offsets from a scalar base
// (T*H*W < 2^24, heads*d*2 < 2^24, a batch sample's tensor < 4 GB).  0: the
// index function per row.  LSE: the call keeps the log-sum-exp (the training
// forward); its denominator then also sums the unrounded p in fp32, so the
// log-sum-exp is exact up to fp32, while O is normalized by the same
// bf16-rounded sum as without it (the two outputs are identical).
template <int D, int ROWS, bool LSE>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_bf16_kernel(const AttnArgs a) {
  using L = Layout<D>;
  constexpr int KK = D / 16;                 // MFMA steps over d
  constexpr int DB = D / 32;                 // 32-wide d blocks of O
  static_assert(L::CPT >= 1 && L::CPT * kThreads == kBN * L::CH, "tile chunks must split evenly");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;                  // lane half
  const int l32 = lane & 31;

  // ---- work item ---------------------------------------------------------
  const WorkItem wi = decode_work(a);
  const SubGeom& sg = wi.sg;
  const int b = wi.b, head = wi.head, qtile = wi.qtile;
  const int n = sg.n;
  const int nkv = (n + kBN - 1) / kBN;

  const int64_t base = (int64_t)b * a.batch_stride + (int64_t)head * D;
  const __bf16* __restrict__ qp = (const __bf16*)a.q + base;
  const char* __restrict__ kb = (const char*)((const __bf16*)a.k + base);
  const char* __restrict__ vb = (const char*)((const __bf16*)a.v + base);
  __bf16* __restrict__ op = (__bf16*)a.o + base;
  const int64_t rs = a.row_stride;
  const uint32_t rsb = (uint32_t)a.row_stride * 2u;

  // ---- loader: thread owns chunk slot tid % CH of rows tid / CH + i*RSTEP ----
  if constexpr (ROWS == 2) {
    for (int x = tid; x < n; x += kThreads) gTok[x] = (int)token_of((uint32_t)x, sg, a.g);
    __syncthreads();
  } else if constexpr (ROWS == 1) {
    build_row_tables(a, sg, gRowBase, gColMap, kThreads);
  }
  const int lslot = tid % L::CH;
  RowWalker<kBN> walk[L::CPT];
  if constexpr (ROWS == 1) {
#pragma unroll
    for (int i = 0; i < L::CPT; ++i) walk[i].init(sg, tid / L::CH + i * L::RSTEP, gRowBase, gColMap);
  }
  struct Stage { uint4 k[L::CPT], v[L::CPT]; };   // staged chunks of a tile
  auto fetch = [&](int tile) -> Stage {
    Stage sgd;
#pragma unroll
    for (int i = 0; i < L::CPT; ++i) {
      int tok;
      if constexpr (ROWS == 2 || ROWS == 3) {
        int jr = tile * kBN + tid / L::CH + i * L::RSTEP;
        jr = jr < n ? jr : n - 1;
        if constexpr (ROWS == 2) tok = gTok[jr];
        else tok = jr;
        const uint32_t off = __umul24((uint32_t)tok, rsb) + (uint32_t)(lslot * 16);
        sgd.k[i] = *(const uint4*)(kb + off);
        sgd.v[i] = *(const uint4*)(vb + off);
      } else if constexpr (ROWS == 1) {
        tok = walk[i].next(gRowBase, gColMap);
        const uint32_t off = __umul24((uint32_t)tok, rsb) + (uint32_t)(lslot * 16);
        sgd.k[i] = *(const uint4*)(kb + off);
        sgd.v[i] = *(const uint4*)(vb + off);
      } else {
        int j = tile * kBN + tid / L::CH + i * L::RSTEP;
        j = j < n ? j : n - 1;
        tok = (int)token_of((uint32_t)j, sg, a.g);
        const int64_t off = (int64_t)tok * rs * 2 + lslot * 16;
        sgd.k[i] = *(const uint4*)(kb + off);
        sgd.v[i] = *(const uint4*)(vb + off);
      }
    }
    return sgd;
  };
  auto stash = [&](const Stage& sgd, int buf) {
#pragma unroll
    for (int i = 0; i < L::CPT; ++i) {
      const int r = tid / L::CH + i * L::RSTEP;
      *(uint4*)(gKV + buf * kTileBytes + r * L::ROWB + (lslot ^ L::kswz(r)) * 16) = sgd.k[i];
      *(uint4*)(gKV + (2 + buf) * kTileBytes + r * L::ROWB + (lslot ^ L::vswz(r)) * 16) = sgd.v[i];
    }
  };

  const Stage first = fetch(0);

  // ---- Q fragments (B operand of S^T = K Q^T) ------------------------------
  bf16x8 qf[KK];
  const int jq = qtile * kBM + wave * 32 + l32;
  const bool qok = jq < n;
  const int tokq = (int)token_of((uint32_t)(qok ? jq : n - 1), sg, a.g);
  const int64_t qoff = (int64_t)tokq * rs;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    qf[kk] = *(const bf16x8*)(qp + qoff + kk * 16 + hl * 8);
    // pin the fragment in registers: otherwise the compiler re-loads Q from
    // global memory inside the key loop and every QK MFMA waits on it
    __asm__ volatile("" : "+v"(qf[kk]));
  }

  stash(first, 0);
  __syncthreads();

  floatx16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = floatx16{};
  float m_run = -INFINITY, l_run = 0.f;
  float l_exact = 0.f;   // LSE only: sum of the unrounded p
  const float c = a.scale_log2;

  // One tile.  BUF (the LDS buffer holding the tile) and LAST (the final tile:
  // mask the keys past the end, nothing to prefetch) are compile-time, so the
  // LDS addresses fold into immediates and the mask exists only in the last
  // tile's copy.
  auto tile = [&](int j, auto buf_tag, auto last_tag) {
    constexpr int BUF = decltype(buf_tag)::value;
    constexpr bool LAST = decltype(last_tag)::value;
    Stage nxt;
    if constexpr (!LAST) nxt = fetch(j + 1);   // in flight during this tile's compute
    const char* sK = gKV + BUF * kTileBytes;
    const char* sV = gKV + (2 + BUF) * kTileBytes;

    // S^T = K Q^T; the K fragments of step kk+1 are read while step kk's
    // MFMAs run, so LDS latency hides behind the matrix core
    auto kfrag = [&](int kk, int mb) -> bf16x8 {
      const int row = mb * 32 + l32;
      const int ch = (2 * kk + hl) ^ L::kswz(row);
      return *(const bf16x8*)(sK + row * L::ROWB + ch * 16);
    };
    floatx16 s[2] = {floatx16{}, floatx16{}};
    bf16x8 kcur[2] = {kfrag(0, 0), kfrag(0, 1)};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      bf16x8 knext[2];
      if (kk + 1 < KK) {
        knext[0] = kfrag(kk + 1, 0);
        knext[1] = kfrag(kk + 1, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcur[mb], qf[kk], s[mb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (kk + 1 < KK) {
        kcur[0] = knext[0];
        kcur[1] = knext[1];
      }
    }

    // online softmax
    if constexpr (LAST) {   // keys past the end of the subsequence
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = j * kBN + mb * 32 + (i >> 2) * 8 + hl * 4 + (i & 3);
          if (key >= n) s[mb][i] = -INFINITY;
        }
    }
    // P = exp2(S c - m) with the running max as it stands; the tile's own
    // max is taken only when some p could exceed kBig (the partial sum of a
    // lane bounds each of its terms), which also covers the first tile
    bf16x8 pk[2][2];
    float lsum, lsum_exact;
    auto exps = [&]() {
      const float mneg = -m_run;
      float ls[4] = {0.f, 0.f, 0.f, 0.f};
      float le[4] = {0.f, 0.f, 0.f, 0.f};
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][cc * 8 + 2 * e], c, mneg));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][cc * 8 + 2 * e + 1], c, mneg));
            // the row sum takes the bf16-rounded p the PV product uses, two
            // terms per dot2 instruction
            bf16x2 pp = {(__bf16)p0, (__bf16)p1};
            ls[mb * 2 + cc] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, ls[mb * 2 + cc], false);
            if constexpr (LSE) le[mb * 2 + cc] += p0 + p1;
            pk[mb][cc][2 * e] = pp[0];
            pk[mb][cc][2 * e + 1] = pp[1];
          }
      lsum = (ls[0] + ls[1]) + (ls[2] + ls[3]);
      if constexpr (LSE) lsum_exact = (le[0] + le[1]) + (le[2] + le[3]);
    };
    exps();
    if (__builtin_amdgcn_ballot_w64(!(lsum <= kBig))) {
      // rare: raise the running max, rescale, and redo the tile
      float mx = s[0][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      const float mnew = fmaxf(m_run, mx * c);
      const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
      m_run = mnew;
      l_run *= alpha;
      if constexpr (LSE) l_exact *= alpha;
      // an fma with a zero addend, not a multiply: this keeps the compiler
      // from folding the rare rescale into an every-tile multiply
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] = __builtin_fmaf(acc[db][i], alpha, 0.0f);
      exps();
    }
    l_run += lsum;
    if constexpr (LSE) l_exact += lsum_exact;

    // O^T += V^T P^T; V fragments are read one step ahead of their MFMA
    auto vfrag = [&](int step) -> bf16x8 {   // step = (db * 2 + mb) * 2 + cc
      const int db = step >> 2, mb = (step >> 1) & 1, cc = step & 1;
      shortx4 part[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int row = mb * 32 + cc * 16 + x * 8 + hl * 4 + ((lane & 15) >> 2);
        const int col = db * 32 + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;   // elements
        const int ch = (col >> 3) ^ L::vswz(row);
        part[x] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_shortx4*)(sV + row * L::ROWB + ch * 16 + (col & 7) * 2));
      }
      bf16x8 vf;
      __builtin_memcpy(&vf, part, 16);
      return vf;
    };
    constexpr int PVS = DB * 4;
    bf16x8 vcur = vfrag(0);
#pragma unroll
    for (int step = 0; step < PVS; ++step) {
      bf16x8 vnext;
      if (step + 1 < PVS) vnext = vfrag(step + 1);
      __builtin_amdgcn_sched_barrier(0);
      const int db = step >> 2, mb = (step >> 1) & 1, cc = step & 1;
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vcur, pk[mb][cc], acc[db], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (step + 1 < PVS) vcur = vnext;
    }

    if constexpr (!LAST) {
      stash(nxt, BUF ^ 1);   // the other buffer was last read before the previous barrier
      __syncthreads();
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using NotLast = std::integral_constant<bool, false>;
  using Last = std::integral_constant<bool, true>;
  int j = 0;
  for (; j + 2 < nkv; j += 2) {
    tile(j, I0{}, NotLast{});
    tile(j + 1, I1{}, NotLast{});
  }
  if (j + 1 < nkv) {
    tile(j, I0{}, NotLast{});
    tile(j + 1, I1{}, Last{});
  } else {
    tile(j, I0{}, Last{});
  }

  // ---- normalize and scatter back to the original token rows ---------------
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
  const float l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  const float inv = 1.0f / l_tot;
  if constexpr (LSE) {
    // both lane halves hold the same running max; log of the denominator in
    // natural units: ln 2 * (m + log2 l), m being in log2 units of s*scale and
    // l the sum of the unrounded p
    const auto swe = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_exact), __float_as_uint(l_exact), false, false);
    const float le_tot = __uint_as_float(swe[0]) + __uint_as_float(swe[1]);
    if (qok && hl == 0) {
      const int64_t N = (int64_t)a.g.T * a.g.H * a.g.W;
      a.lse[((int64_t)b * N + tokq) * a.heads + head] = 0.69314718055994531f * (m_run + __log2f(le_tot));
    }
  }
  if (qok) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(acc[db][g4 * 4 + e] * inv);
        *(bf16x4*)(op + qoff + db * 32 + g4 * 8 + hl * 4) = v4;
      }
  }
}

template <int D, bool LSE>
hipError_t launch_d(AttnArgs a, int B, hipStream_t stream) {
  assign_tiles(a, B, kBM);
  if (a.total_tiles == 0) return hipSuccess;
  const int64_t row_bytes = (int64_t)a.row_stride * 2;
  if (a.g.kh == 1 && a.g.kw == 1 && offsets32_ok(a, row_bytes))
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, 3, LSE>), dim3(a.total_tiles), dim3(kThreads), 0, stream, a);
  else if (token_table_ok(a, row_bytes, kTokCap))
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, 2, LSE>), dim3(a.total_tiles), dim3(kThreads), 0, stream, a);
  else if (fast_rows_ok(a, row_bytes))
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, 1, LSE>), dim3(a.total_tiles), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, 0, LSE>), dim3(a.total_tiles), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(AttnArgs a, int B, int d, hipStream_t stream) {
  const bool lse = a.lse != nullptr;
  if (d == 128) return lse ? launch_d<128, true>(a, B, stream) : launch_d<128, false>(a, B, stream);
  return lse ? launch_d<64, true>(a, B, stream) : launch_d<64, false>(a, B, stream);
}

}  // namespace skiparse
