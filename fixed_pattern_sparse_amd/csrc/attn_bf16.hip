// Skiparse-2D attention forward, bf16 in / bf16 out, fp32 accumulation, on
// CDNA4 (gfx950) matrix cores.
//
// Method (OSP-Next summary, 核心方法 core method and 方法步骤详情 method
// steps): dense softmax attention inside each of the k*k subsequences of the
// token-wise or group-wise rearrange, written back in the original layout;
// padding from the any-resolution rule is never computed.
//
// Work decomposition: one work-group per (batch, head, subsequence, tile of BM
// queries).  Each wave owns QB blocks of 32 queries.  Keys are streamed in
// tiles of 64 rows through double-buffered LDS; rows are gathered straight
// from the (B, T, H, W, heads, d) tensors by the index function (no permuted
// copy), with direct global->LDS loads.
//
// Per 64-key tile and 32-query block:
//   S^T = K Q^T   8 x v_mfma_f32_32x32x16_bf16 per 32 keys (d = 128); the
//                 transposed orientation leaves one query per lane, so row
//                 statistics need one cross-half swap and no shuffles;
//   online softmax in the log2 domain with a lazily raised running max: the
//                 accumulator is rescaled only when a tile's max exceeds the
//                 running max by more than 2^8, which keeps p <= 256 and the
//                 result exact (O and l share the same offset);
//   O^T += V^T P^T  V^T comes from row-major V in LDS through
//                 ds_read_b64_tr_b16, P^T stays in registers as bf16.
#include "internal.h"

namespace skiparse {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kBN = 64;          // keys per tile
constexpr float kTau = 8.0f;     // slack of the running max, log2 units

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int xcd_remap(int i, int n) {
  // Work-groups are handed to the 8 XCDs round-robin.  Give each XCD one
  // contiguous range of logical tiles, so the query tiles that stream the same
  // subsequence's K/V run side by side on one XCD and share its L2.
  constexpr int X = 8;
  int xcd = i % X, local = i / X;
  int per = n / X, rem = n % X;
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + local;
}

template <int D>
struct Layout {
  static constexpr int CH = D / 8;           // 16-byte chunks per row
  static constexpr int ROWB = D * 2;         // bytes per row
  static constexpr int TILEB = kBN * ROWB;   // bytes per K or V tile
  // XOR swizzles of the chunk index: K rows are read 32 at a time at one
  // chunk (ds_read_b128), V rows 8 at a time over 4 chunks (ds_read_b64_tr_b16).
  __device__ static int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static int vswz(int r) { return D == 128 ? ((r & 3) << 2) : ((r & 1) << 2); }
};

template <int D, int NW, int QB>
__global__ void __launch_bounds__(NW * 64)
attn_fwd_bf16_kernel(const AttnArgs a) {
  using L = Layout<D>;
  constexpr int BM = NW * QB * 32;
  constexpr int KK = D / 16;                 // MFMA steps over d
  constexpr int DB = D / 32;                 // 32-wide d blocks of O
  constexpr int LOADS = kBN * L::CH / 64;    // 1 KB load instructions per tile and matrix
  constexpr int LPW = LOADS / NW;            // ... per wave
  static_assert(LOADS % NW == 0, "tile loads must split evenly over the waves");

  __shared__ __attribute__((aligned(16))) char smem[4 * L::TILEB];   // K0 K1 V0 V1

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hl = lane >> 5;                  // lane half
  const int l32 = lane & 31;

  // ---- work item ---------------------------------------------------------
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = wg / a.tiles_per_bh;
  const int rem = wg - bh * a.tiles_per_bh;
  const int b = bh / a.heads;
  const int head = bh - b * a.heads;
  int si = 0;
  while (si + 1 < a.n_run && a.sub[si + 1].tile0 <= rem) ++si;
  const SubGeom sg = a.sub[si];
  const int qtile = rem - sg.tile0;
  const int n = sg.n;
  const int nkv = (n + kBN - 1) / kBN;

  const int64_t base = (int64_t)b * a.batch_stride + (int64_t)head * D;
  const __bf16* __restrict__ qp = (const __bf16*)a.q + base;
  const __bf16* __restrict__ kp = (const __bf16*)a.k + base;
  const __bf16* __restrict__ vp = (const __bf16*)a.v + base;
  __bf16* __restrict__ op = (__bf16*)a.o + base;
  const int64_t rs = a.row_stride;

  // ---- K/V tile loader: direct global -> LDS, 16 B per lane -----------------
  // Load instruction u of a tile writes LDS bytes [u*1024, u*1024+1024): row
  // (u*64 + lane) / CH, chunk slot (u*64 + lane) % CH, holding global chunk
  // slot ^ swizzle(row).
  auto issue_tile = [&](int it, int buf) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int u = wave * LPW + i;
      const int lin = u * 64 + lane;
      const int row = lin / L::CH;
      const int slot = lin % L::CH;
      int j = it * kBN + row;
      j = j < n ? j : n - 1;
      const int64_t off = (int64_t)token_of((uint32_t)j, sg, a.g) * rs;
      const int ck = slot ^ L::kswz(row);
      const int cv = slot ^ L::vswz(row);
      __builtin_amdgcn_global_load_lds((const void*)(kp + off + ck * 8),
                                       (lds_void*)(smem + buf * L::TILEB + u * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vp + off + cv * 8),
                                       (lds_void*)(smem + (2 + buf) * L::TILEB + u * 1024), 16, 0, 0);
    }
  };

  issue_tile(0, 0);

  // ---- Q fragments (B operand of S^T = K Q^T) ------------------------------
  bf16x8 qf[QB][KK];
  int64_t qoff[QB];
  bool qok[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int j = qtile * BM + (wave * QB + qb) * 32 + l32;
    qok[qb] = j < n;
    const int jc = j < n ? j : n - 1;
    qoff[qb] = (int64_t)token_of((uint32_t)jc, sg, a.g) * rs;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[qb][kk] = *(const bf16x8*)(qp + qoff[qb] + kk * 16 + hl * 8);
  }

  floatx16 acc[QB][DB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[qb][db] = floatx16{};
  }
  const float c = a.scale_log2;

  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's tile-0 loads landed
  __syncthreads();

  for (int it = 0; it < nkv; ++it) {
    const int buf = it & 1;
    if (it + 1 < nkv) issue_tile(it + 1, buf ^ 1);
    const char* sK = smem + buf * L::TILEB;
    const char* sV = smem + (2 + buf) * L::TILEB;

    // S^T = K Q^T : two 32-key blocks
    floatx16 s[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) { s[qb][0] = floatx16{}; s[qb][1] = floatx16{}; }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = mb * 32 + l32;
        const int ch = (2 * kk + hl) ^ L::kswz(row);
        const bf16x8 kf = *(const bf16x8*)(sK + row * L::ROWB + ch * 16);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][kk], s[qb][mb], 0, 0, 0);
      }
    }

    // keys past the end of the subsequence (last tile only)
    if ((it + 1) * kBN > n) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = it * kBN + mb * 32 + (i >> 2) * 8 + hl * 4 + (i & 3);
          if (key >= n) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[qb][mb][i] = -INFINITY;
          }
        }
    }

    // online softmax; P^T packed to bf16 as the B operand of the PV product
    bf16x8 pk[QB][2][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = s[qb][0][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[qb][0][i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[qb][1][i]);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float mx2 = mx * c;
      if (__builtin_amdgcn_ballot_w64(mx2 > m_run[qb] + kTau)) {
        const float mnew = fmaxf(m_run[qb], mx2);
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - mnew);
        m_run[qb] = mnew;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[qb][db][i] *= alpha;
      }
      const float mneg = -m_run[qb];
      float lsum = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][mb][cc * 8 + e], c, mneg));
            lsum += p;
            pk[qb][mb][cc][e] = (__bf16)p;
          }
      l_run[qb] += lsum;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          shortx4 part[2];
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const int row = mb * 32 + cc * 16 + x * 8 + hl * 4 + ((lane & 15) >> 2);
            const int col = db * 32 + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;   // elements
            const int ch = (col >> 3) ^ L::vswz(row);
            part[x] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) shortx4*)(sV + row * L::ROWB + ch * 16 + (col & 7) * 2));
          }
          bf16x8 vf;
          __builtin_memcpy(&vf, part, 16);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pk[qb][mb][cc], acc[qb][db], 0, 0, 0);
        }
      }
    }

    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): next tile landed in LDS
    __syncthreads();
  }

  // ---- normalize and scatter back to the original token rows ---------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run[qb]), __float_as_uint(l_run[qb]), false, false);
    const float l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const float inv = 1.0f / l;
    if (qok[qb]) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          bf16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(acc[qb][db][g4 * 4 + e] * inv);
          *(bf16x4*)(op + qoff[qb] + db * 32 + g4 * 8 + hl * 4) = v4;
        }
    }
  }
}

template <int D, int NW, int QB>
hipError_t launch_cfg(AttnArgs a, int B, hipStream_t stream) {
  constexpr int BM = NW * QB * 32;
  assign_tiles(a, B, BM);
  if (a.total_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, NW, QB>), dim3(a.total_tiles), dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(AttnArgs a, int B, int d, hipStream_t stream) {
  if (d == 128) return launch_cfg<128, 4, 1>(a, B, stream);
  return launch_cfg<64, 4, 1>(a, B, stream);
}

}  // namespace skiparse
