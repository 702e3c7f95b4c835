// Pieces shared by the backward kernels: vector types, tile geometry, the
// LDS arrays, the e4m3-to-bf16 widening, the swizzled fragment reads and the
// row source.  The dQ kernel is built in its own translation unit
// (attn_bwd_dq.hip) so that it can take its own scheduling options.
#pragma once

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
typedef int intx8 __attribute__((ext_vector_type(8)));

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
constexpr int kRowB8 = D;          // bytes per row of e4m3 codes
constexpr int kTileB8 = kBT * kRowB8;  // 4 KB
constexpr float kLog2e = 1.4426950408889634f;
static_assert(kBT * kCH == kThreads, "one chunk per thread and matrix per tile");

__shared__ __attribute__((aligned(16))) char gA[2 * kTileB];   // K (dQ kernel) or Q (dK/dV kernel)
__shared__ __attribute__((aligned(16))) char gB[2 * kTileB];   // V (dQ kernel) or dO (dK/dV kernel)
__shared__ __attribute__((aligned(16))) char gVk[kBM * kRowB];  // dK/dV kernel: V rows of its 256 keys
__shared__ __attribute__((aligned(16))) float gL[2 * kBT];     // dK/dV kernel: -L/c per query row
__shared__ __attribute__((aligned(16))) float gDn[2 * kBT];    // dK/dV kernel: -D per query row
__shared__ int32_t gTokB[kTokCap];
// 8-bit path: e4m3 copies of the streamed tiles, read row-major as operands
// of the e4m3 matrix core (the bf16 copies above serve the transposed reads)
__shared__ __attribute__((aligned(16))) char gA8[2 * kTileB8];
__shared__ __attribute__((aligned(16))) char gB8[2 * kTileB8];
__shared__ __attribute__((aligned(16))) char gVk8[kBM * kRowB8];  // dK/dV kernel: V rows of its 256 keys as codes

// 16 consecutive rows map to 16 distinct chunks (row-major reads), and each
// aligned group of 4 rows differs in bits 3:2 (transposed reads of 4 chunks).
__device__ __forceinline__ int uswz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Rows of e4m3 codes (128 bytes, eight 16-byte chunks): chunk c of row r sits
// at slot c ^ ((r >> 1) & 7).  Rows r and r + 1 share a 256-byte bank line, so
// the 16 rows that a 16-lane group of ds_read_b128 reads at one chunk cover
// all 64 banks.
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }

// Operand of v_mfma_*_32x32x64_f8f6f4 from an e4m3 tile read row-major: row
// l32, bytes 64 kk + 32 hl .. + 31.  Both operands of a product take the same
// pairing (byte e of lane half h is element 64 kk + 32 h + e of the row).
__device__ __forceinline__ intx8 frag8_rows(const char* t, int l32, int hl, int kk) {
  const char* r = t + l32 * kRowB8;
  const uint4 lo = *(const uint4*)(r + ((4 * kk + 2 * hl) ^ swz8(l32)) * 16);
  const uint4 hi = *(const uint4*)(r + ((4 * kk + 2 * hl + 1) ^ swz8(l32)) * 16);
  return intx8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// The same operand for a row the lane reads from global memory.
__device__ __forceinline__ intx8 frag8_global(const char* row, int hl, int kk) {
  const uint4 lo = *(const uint4*)(row + 64 * kk + 32 * hl);
  const uint4 hi = *(const uint4*)(row + 64 * kk + 32 * hl + 16);
  return intx8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// A thread's 8 codes (elements 8 lslot .. + 7 of row lrow) into an e4m3 tile.
__device__ __forceinline__ void stash8(char* t, int lrow, int lslot, uint2 c) {
  *(uint2*)(t + lrow * kRowB8 + ((lslot >> 1) ^ swz8(lrow)) * 16 + (lslot & 1) * 8) = c;
}

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

}  // namespace

// dQ for every run subsequence (attn_bwd_dq.hip); table selects the
// whole-subsequence token table as the row source, else the index function.
hipError_t launch_bwd_dq(const AttnArgs& a, bool f8, bool table, hipStream_t stream);

}  // namespace skiparse
