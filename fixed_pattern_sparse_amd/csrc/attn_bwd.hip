// Backward pass of Skiparse-2D attention, bf16 in / bf16 out, fp32
// accumulation, on CDNA4 (gfx950) matrix cores.
//
// The sparse model is fine-tuned and trained with this attention in its
// layers (OSP-Next summary, 方法步骤详情 method steps and 复现评估
// reproduction), so each layer needs dQ, dK, dV for an upstream dO.  Inside
// one subsequence, with S = scale Q K^T, P = softmax(S) by rows, O = P V and
// the forward's log-sum-exp L per query (P = exp(S - L)):
//     D  = rowsum(dO * O)            (equals rowsum(P * dP))
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D)
//     dQ = scale dS K,  dK = scale dS^T Q
// Rows are gathered and scattered through the rearrange's index function, as
// in the forward kernel; padded tokens are never read or written.
//
// Kernels:
//   bwd_dsum_kernel      D for every row, one wave per 4 rows (HBM-bound);
//   attn_bwd_dq_kernel   8 waves x 32 queries hold Q and dO fragments; key
//                        tiles of 32 rows stream K and V through LDS;
//                        S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T;
//   attn_bwd_dkv_fused_kernel
//                        8 waves x 32 keys hold K fragments, the work-group's
//                        V rows sit in LDS; query tiles of 32 rows stream Q
//                        and dO (with L and D); S = Q K^T + (-L/c),
//                        P = exp2(c S), dV^T += dO^T P, dP = dO V^T + (-D),
//                        dK^T += Q^T (P * dP).
// 8-bit inputs (F8): Q, K, V and dO arrive as per-tensor e4m3 codes with
// their scales (the pages quantize every tensor of the 8-bit training path
// per tensor, the gradient with its own maximum).  The loaders widen each code
// to bf16, which is exact (every e4m3 value is a bf16 value), so the MFMA
// products of codes are exact as on the 8-bit matrix core; the descales fold
// into scalars: the exp2 constant takes 1/(s_q s_k), D enters as D / f with
// f = 1/(s_do s_v) so dP - D is f (dO^ V^T - D/f), and the outputs take
// scale f / s_k (dQ), scale f / s_q (dK) and 1/s_do (dV).
// Per-query L and D enter the dK/dV kernel through the MFMA accumulator's
// initial value, so they cost no registers of their own.  Each staged tile is
// read both row-major (ds_read_b128, 16 rows at one chunk) and transposed
// (ds_read_b64_tr_b16, 4 rows x 4 chunks), and one XOR swizzle of the 16-byte
// chunk index serves both without bank conflicts.
#include <type_traits>

#include "attn_common.h"

namespace skiparse {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

constexpr int D = 128;              // head dim (the only one built for the backward pass)
constexpr int KK = D / 16;          // MFMA steps over d
constexpr int DB = D / 32;          // 32-wide d blocks
constexpr int kBT = 32;             // rows per streamed tile
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;    // fixed rows (queries or keys) per work-group
constexpr int kRowB = D * 2;        // bytes per row
constexpr int kTileB = kBT * kRowB; // 8 KB
constexpr int kCH = D / 8;          // 16-byte chunks per row
constexpr int kTokCap = 24064;
constexpr float kLog2e = 1.4426950408889634f;
static_assert(kBT * kCH == kThreads, "one chunk per thread and matrix per tile");

__shared__ __attribute__((aligned(16))) char gA[2 * kTileB];   // K (dQ kernel) or Q (dK/dV kernel)
__shared__ __attribute__((aligned(16))) char gB[2 * kTileB];   // V (dQ kernel) or dO (dK/dV kernel)
__shared__ __attribute__((aligned(16))) char gVk[kBM * kRowB];  // dK/dV kernel: V rows of its 256 keys
__shared__ __attribute__((aligned(16))) float gL[2 * kBT];     // dK/dV kernel: -L/c per query row
__shared__ __attribute__((aligned(16))) float gDn[2 * kBT];    // dK/dV kernel: -D per query row
__shared__ int32_t gTokB[kTokCap];

// 16 consecutive rows map to 16 distinct chunks (row-major reads), and each
// aligned group of 4 rows differs in bits 3:2 (transposed reads of 4 chunks).
__device__ __forceinline__ int uswz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Two e4m3 codes (bytes 2*hi, 2*hi + 1 of w) as two bf16 values.  An e4m3
// value has at most 4 significant bits and an exponent within bf16's range,
// so its fp32 form ends in 16 zero bits and the high halves are exact.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_bf16x2(uint32_t w) {
  const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  return __builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u);
}

// Eight consecutive elements starting at element offset e of a row-major
// tensor as loaded (8 bytes of e4m3 codes or 16 of bf16), and widened to
// eight bf16 values.  The streamed tiles keep the loaded form in registers
// and widen it only when they store it to LDS, after the tile's compute, so
// the load's latency stays hidden as it is for bf16.
template <bool F8>
using Raw8 = typename std::conditional<F8, uint2, uint4>::type;

template <bool F8>
__device__ __forceinline__ Raw8<F8> load_raw8(const char* base, int64_t e) {
  if constexpr (F8) return *(const uint2*)(base + e);
  else return *(const uint4*)(base + e * 2);
}

template <bool F8>
__device__ __forceinline__ uint4 widen8(Raw8<F8> c) {
  if constexpr (F8)
    return uint4{e4m3x2_bf16x2<false>(c.x), e4m3x2_bf16x2<true>(c.x), e4m3x2_bf16x2<false>(c.y),
                 e4m3x2_bf16x2<true>(c.y)};
  else return c;
}

template <bool F8>
__device__ __forceinline__ uint4 load8(const char* base, int64_t e) {
  return widen8<F8>(load_raw8<F8>(base, e));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) {
  bf16x8 f;
  __builtin_memcpy(&f, &u, 16);
  return f;
}

// A fragment of a staged tile read row-major: rows l32 (+0), chunk 2*kk + hl.
__device__ __forceinline__ bf16x8 frag_rows(const char* t, int l32, int hl, int kk) {
  return *(const bf16x8*)(t + l32 * kRowB + ((2 * kk + hl) ^ uswz(l32)) * 16);
}

// A fragment of a staged tile read transposed: A[d][row] for d block db and
// rows 16*cc + (8 per part), the row order matching the accumulator layout
// the B operand was packed from.
__device__ __forceinline__ bf16x8 frag_cols(const char* t, int lane, int hl, int db, int cc) {
  shortx4 part[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int row = cc * 16 + x * 8 + hl * 4 + ((lane & 15) >> 2);
    const int col = db * 32 + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;   // elements
    const int ch = (col >> 3) ^ uswz(row);
    part[x] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(t + row * kRowB + ch * 16 + (col & 7) * 2));
  }
  bf16x8 f;
  __builtin_memcpy(&f, part, 16);
  return f;
}

// Pack 16 fp32 accumulator values (rows 8(i/4) + 4hl + i%4) into the two bf16
// B operands of the next contraction over those rows.
__device__ __forceinline__ void pack_b(const float* x, bf16x8 (&out)[2]) {
#pragma unroll
  for (int cc = 0; cc < 2; ++cc)
#pragma unroll
    for (int e = 0; e < 8; ++e) out[cc][e] = (__bf16)x[cc * 8 + e];
}

__device__ __forceinline__ void store_rows_t(__bf16* dst, const floatx16 (&acc)[DB], float mul, int hl) {
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      bf16x4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(acc[db][g4 * 4 + e] * mul);
      *(bf16x4*)(dst + db * 32 + g4 * 8 + hl * 4) = v4;
    }
}

// ---------------------------------------------------------------------------
// D = rowsum(dO * O) for every (b, token, head) row
// ---------------------------------------------------------------------------

// (F8: dO as e4m3 codes, and D / f = s_v * rowsum(dO^ * O) is written.)
template <bool F8>
__global__ void __launch_bounds__(256) bwd_dsum_kernel(const __bf16* __restrict__ o, const void* __restrict__ dout,
                                                       const float* __restrict__ descale, float* __restrict__ dsum,
                                                       int64_t rows) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  const int sub = lane >> 4, ch = lane & 15;   // 4 rows per wave, 16 chunks per row
  for (int64_t r0 = wave * 4; r0 < rows; r0 += nwaves * 4) {
    const int64_t r = r0 + sub;
    float acc = 0.f;
    if (r < rows) {
      const bf16x8 x = *(const bf16x8*)(o + r * D + ch * 8);
      const bf16x8 y = as_bf16x8(load8<F8>((const char*)dout, r * D + ch * 8));
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)x[e], (float)y[e], acc);
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
    if (r < rows && ch == 0) dsum[r] = F8 ? acc * descale[4] : acc;
  }
}

// ---------------------------------------------------------------------------
// Shared work-group prologue: token table and tile loader
// ---------------------------------------------------------------------------

template <int ROWS>
struct Rows {
  const AttnArgs& a;
  const SubGeom& sg;
  int n;
  __device__ Rows(const AttnArgs& a_, const SubGeom& sg_, int n_) : a(a_), sg(sg_), n(n_) {}
  __device__ void build(int tid) {
    if constexpr (ROWS == 2) {
      for (int x = tid; x < n; x += kThreads) gTokB[x] = (int)token_of((uint32_t)x, sg, a.g);
      __syncthreads();
    }
  }
  // token of compact member j (clamped to the last member)
  __device__ int tok(int j) const {
    j = j < n ? j : n - 1;
    if constexpr (ROWS == 2) return gTokB[j];
    return (int)token_of((uint32_t)j, sg, a.g);
  }
};

// ---------------------------------------------------------------------------
// dQ: queries fixed, key tiles streamed
// ---------------------------------------------------------------------------

template <int ROWS, bool F8>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dq_kernel(const AttnArgs a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;
  const int l32 = lane & 31;

  const WorkItem wi = decode_work(a);
  const SubGeom& sg = wi.sg;
  const int n = sg.n;
  const int nkv = (n + kBT - 1) / kBT;
  const int64_t N = (int64_t)a.g.T * a.g.H * a.g.W;
  const int64_t base = (int64_t)wi.b * a.batch_stride + (int64_t)wi.head * D;
  const int64_t rs = a.row_stride;
  constexpr int EB = F8 ? 1 : 2;   // bytes per element
  const char* __restrict__ qb = (const char*)a.q + base * EB;
  const char* __restrict__ dob = (const char*)a.dout + base * EB;
  const char* __restrict__ kb = (const char*)a.k + base * EB;
  const char* __restrict__ vb = (const char*)a.v + base * EB;

  Rows<ROWS> rows(a, sg, n);
  rows.build(tid);
  const int lrow = tid / kCH, lslot = tid % kCH;
  const int sw_st = (lslot ^ uswz(lrow)) * 16;
  auto fetch = [&](int tile, Raw8<F8>& kx, Raw8<F8>& vx) {
    const int64_t e = (int64_t)rows.tok(tile * kBT + lrow) * rs + lslot * 8;
    kx = load_raw8<F8>(kb, e);
    vx = load_raw8<F8>(vb, e);
  };
  Raw8<F8> kx, vx;
  fetch(0, kx, vx);

  // the lane's query: Q and dO fragments (B operands), L and D
  const int jq = wi.qtile * kBM + wave * 32 + l32;
  const bool qok = jq < n;
  const int tq = rows.tok(jq);
  const int64_t qoff = (int64_t)tq * rs;
  bf16x8 qf[KK], dof[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    qf[kk] = as_bf16x8(load8<F8>(qb, qoff + kk * 16 + hl * 8));
    dof[kk] = as_bf16x8(load8<F8>(dob, qoff + kk * 16 + hl * 8));
    __asm__ volatile("" : "+v"(qf[kk]), "+v"(dof[kk]));
  }
  const int64_t ridx = ((int64_t)wi.b * N + tq) * a.heads + wi.head;
  const float lse2 = a.lse[ridx] * kLog2e;
  const float dq_d = a.dsum[ridx];
  const float c = F8 ? a.scale_log2 * a.descale[1] * a.descale[3] : a.scale_log2;

  *(uint4*)(gA + lrow * kRowB + sw_st) = widen8<F8>(kx);
  *(uint4*)(gB + lrow * kRowB + sw_st) = widen8<F8>(vx);
  __syncthreads();

  floatx16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = floatx16{};

  for (int j = 0; j < nkv; ++j) {
    const int buf = j & 1;
    const bool more = j + 1 < nkv;
    if (more) fetch(j + 1, kx, vx);
    const char* sK = gA + buf * kTileB;
    const char* sV = gB + buf * kTileB;
    floatx16 s = floatx16{}, dp = floatx16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows(sK, l32, hl, kk), qf[kk], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows(sV, l32, hl, kk), dof[kk], dp, 0, 0, 0);
    }
    // dS^T = P^T * (dP^T - D); keys past the end of the subsequence get P = 0
    float ds[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = j * kBT + (i >> 2) * 8 + hl * 4 + (i & 3);
      const float p = key < n ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -lse2)) : 0.f;
      ds[i] = p * (dp[i] - dq_d);
    }
    bf16x8 dsb[2];
    pack_b(ds, dsb);
    // dQ^T += K^T dS^T
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_cols(sK, lane, hl, db, cc), dsb[cc], acc[db], 0, 0, 0);
    if (more) {
      *(uint4*)(gA + (buf ^ 1) * kTileB + lrow * kRowB + sw_st) = widen8<F8>(kx);
      *(uint4*)(gB + (buf ^ 1) * kTileB + lrow * kRowB + sw_st) = widen8<F8>(vx);
    }
    __syncthreads();
  }
  const float mul = F8 ? a.scale * a.descale_do[1] * a.descale[5] * a.descale[3] : a.scale;
  if (qok) store_rows_t((__bf16*)a.dq + base + qoff, acc, mul, hl);
}

// ---------------------------------------------------------------------------
// dK and dV together: keys fixed, query tiles streamed.  K fragments stay in
// registers; the work-group's V rows are staged once in LDS and read as the B
// operand of dP, which keeps the two accumulator sets within two waves per
// SIMD.  Rows come from the index function (the V block leaves no room for
// the token table).
// ---------------------------------------------------------------------------

template <bool F8>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dkv_fused_kernel(const AttnArgs a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;
  const int l32 = lane & 31;

  const WorkItem wi = decode_work(a);
  const SubGeom& sg = wi.sg;
  const int n = sg.n;
  const int nq = (n + kBT - 1) / kBT;
  const int64_t N = (int64_t)a.g.T * a.g.H * a.g.W;
  const int64_t base = (int64_t)wi.b * a.batch_stride + (int64_t)wi.head * D;
  const int64_t rs = a.row_stride;
  constexpr int EB = F8 ? 1 : 2;   // bytes per element
  const char* __restrict__ qb = (const char*)a.q + base * EB;
  const char* __restrict__ db_ = (const char*)a.dout + base * EB;
  const char* __restrict__ vb = (const char*)a.v + base * EB;
  const char* __restrict__ kb = (const char*)a.k + base * EB;
  const float c = F8 ? a.scale_log2 * a.descale[1] * a.descale[3] : a.scale_log2;
  const float inv_c = 1.0f / c;
  Rows<0> rows(a, sg, n);

  const int lrow = tid / kCH, lslot = tid % kCH;
  const int sw_st = (lslot ^ uswz(lrow)) * 16;
  auto fetch = [&](int tile, Raw8<F8>& qx, Raw8<F8>& dx, float& ln, float& dn) {
    const int j = tile * kBT + lrow;
    const int t = rows.tok(j);
    const int64_t e = (int64_t)t * rs + lslot * 8;
    qx = load_raw8<F8>(qb, e);
    dx = load_raw8<F8>(db_, e);
    if (lslot == 0) {
      const int64_t ridx = ((int64_t)wi.b * N + t) * a.heads + wi.head;
      ln = j < n ? -(a.lse[ridx] * kLog2e) * inv_c : -INFINITY;
      dn = j < n ? -a.dsum[ridx] : 0.f;
    }
  };
  auto stash = [&](int buf, const Raw8<F8>& qx, const Raw8<F8>& dx, float ln, float dn) {
    *(uint4*)(gA + buf * kTileB + lrow * kRowB + sw_st) = widen8<F8>(qx);
    *(uint4*)(gB + buf * kTileB + lrow * kRowB + sw_st) = widen8<F8>(dx);
    if (lslot == 0) {
      gL[buf * kBT + lrow] = ln;
      gDn[buf * kBT + lrow] = dn;
    }
  };
  Raw8<F8> qx, dx;
  float ln = 0.f, dn = 0.f;
  fetch(0, qx, dx, ln, dn);

  // V rows of the work-group's 256 keys (clamped past the end), swizzled like
  // the tiles: key row r at chunk c ^ uswz(r)
  const int key0 = wi.qtile * kBM;
#pragma unroll
  for (int i = 0; i < kBM * kCH / kThreads; ++i) {
    const int r = lrow + i * kBT;
    const int64_t e = (int64_t)rows.tok(key0 + r) * rs + lslot * 8;
    *(uint4*)(gVk + r * kRowB + (lslot ^ uswz(r)) * 16) = load8<F8>(vb, e);
  }

  const int jk = key0 + wave * 32 + l32;
  const bool kok = jk < n;
  const int64_t koff = (int64_t)rows.tok(jk) * rs;
  bf16x8 kf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    kf[kk] = as_bf16x8(load8<F8>(kb, koff + kk * 16 + hl * 8));
    __asm__ volatile("" : "+v"(kf[kk]));
  }
  const char* sVk = gVk + wave * 32 * kRowB;   // the wave's 32 key rows

  stash(0, qx, dx, ln, dn);
  __syncthreads();

  floatx16 accK[DB], accV[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    accK[db] = floatx16{};
    accV[db] = floatx16{};
  }

  for (int j = 0; j < nq; ++j) {
    const int buf = j & 1;
    const bool more = j + 1 < nq;
    if (more) fetch(j + 1, qx, dx, ln, dn);
    const char* sQ = gA + buf * kTileB;
    const char* sD = gB + buf * kTileB;
    // S = Q K^T - L/c (accumulator starting at -L/c of its query row)
    floatx16 s;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const floatx4 l4 = *(const floatx4*)(gL + buf * kBT + g * 8 + hl * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) s[g * 4 + e] = l4[e];
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows(sQ, l32, hl, kk), kf[kk], s, 0, 0, 0);
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(s[i] * c);
    bf16x8 pb[2];
    pack_b(p, pb);
    // dV^T += dO^T P
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
        accV[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_cols(sD, lane, hl, db, cc), pb[cc], accV[db], 0, 0, 0);
    // dP - D = dO V^T - D; V^T of the lane's key from LDS
    floatx16 dp;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const floatx4 d4 = *(const floatx4*)(gDn + buf * kBT + g * 8 + hl * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) dp[g * 4 + e] = d4[e];
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows(sD, l32, hl, kk), frag_rows(sVk, l32, hl, kk), dp, 0, 0, 0);
    // dS = P * (dP - D), with P taken back from its bf16 copy (the value the
    // dV product used), so the fp32 P need not stay live
    float ds[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) ds[i] = (float)pb[i >> 3][i & 7] * dp[i];
    bf16x8 dsb[2];
    pack_b(ds, dsb);
    // dK^T += Q^T dS
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
        accK[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_cols(sQ, lane, hl, db, cc), dsb[cc], accK[db], 0, 0, 0);
    if (more) stash(buf ^ 1, qx, dx, ln, dn);
    __syncthreads();
  }
  if (kok) {
    const float mk = F8 ? a.scale * a.descale_do[1] * a.descale[5] * a.descale[1] : a.scale;
    const float mv = F8 ? a.descale_do[1] : 1.0f;
    store_rows_t((__bf16*)a.dk + base + koff, accK, mk, hl);
    store_rows_t((__bf16*)a.dv + base + koff, accV, mv, hl);
  }
}

template <bool F8>
hipError_t launch_bwd(AttnArgs a, int B, int d, hipStream_t stream) {
  if (d != D) return hipErrorNotSupported;
  // D for every row of the tensors (rows outside the run subsequences are
  // computed too and never read)
  const int64_t rows = (int64_t)B * a.g.T * a.g.H * a.g.W * a.heads;
  if (rows > 0) {
    int64_t blocks = (rows + 15) / 16;
    blocks = blocks < 8192 ? blocks : 8192;
    hipLaunchKernelGGL(bwd_dsum_kernel<F8>, dim3((unsigned)blocks), dim3(256), 0, stream, (const __bf16*)a.o,
                       a.dout, a.descale, a.dsum, rows);
  }
  assign_tiles(a, B, kBM);
  if (a.total_tiles == 0) return hipGetLastError();
  const bool table = token_table_ok(a, (int64_t)a.row_stride * (F8 ? 1 : 2), kTokCap);
  const dim3 grid(a.total_tiles), block(kThreads);
  if (table)
    hipLaunchKernelGGL((attn_bwd_dq_kernel<2, F8>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((attn_bwd_dq_kernel<0, F8>), grid, block, 0, stream, a);
  hipLaunchKernelGGL(attn_bwd_dkv_fused_kernel<F8>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(AttnArgs a, int B, int d, hipStream_t stream) { return launch_bwd<false>(a, B, d, stream); }

hipError_t launch_attn_bwd_fp8(AttnArgs a, int B, int d, hipStream_t stream) { return launch_bwd<true>(a, B, d, stream); }

}  // namespace skiparse
