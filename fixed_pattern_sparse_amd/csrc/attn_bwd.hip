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
// per tensor, the gradient with its own maximum).  S and dP, the products of
// two coded tensors, run on the e4m3 matrix core (v_mfma_*_32x32x64_f8f6f4)
// from e4m3 copies of the staged tiles and code fragments in registers; the
// transposed operands of dV, dK and dQ come from bf16 copies, widened from the
// codes at staging (exact: every e4m3 value is a bf16 value), against P and dS
// in bf16.  The descales fold into scalars: the exp2 constant takes
// 1/(s_q s_k), D enters as D / f with f = 1/(s_do s_v) so dP - D is
// f (dO^ V^T - D/f), and the outputs take scale f / s_k (dQ), scale f / s_q
// (dK) and 1/s_do (dV).
// Per-query L and D enter the dK/dV kernel through the MFMA accumulator's
// initial value, so they cost no registers of their own.  Each staged tile is
// read both row-major (ds_read_b128, 16 rows at one chunk) and transposed
// (ds_read_b64_tr_b16, 4 rows x 4 chunks), and one XOR swizzle of the 16-byte
// chunk index serves both without bank conflicts.
#include "attn_bwd_common.h"

namespace skiparse {
namespace {

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
      // raw L and D of the row: they are scaled only when stored, after the
      // tile's compute, so their latency stays hidden like that of the rows
      const int64_t ridx = ((int64_t)wi.b * N + t) * a.heads + wi.head;
      ln = a.lse[ridx];
      dn = a.dsum[ridx];
    }
  };
  auto stash = [&](int buf, int tile, const Raw8<F8>& qx, const Raw8<F8>& dx, float ln, float dn) {
    *(uint4*)(gA + buf * kTileB + lrow * kRowB + sw_st) = widen8<F8>(qx);
    *(uint4*)(gB + buf * kTileB + lrow * kRowB + sw_st) = widen8<F8>(dx);
    if constexpr (F8) {   // codes for the e4m3 products S and dP
      stash8(gA8 + buf * kTileB8, lrow, lslot, qx);
      stash8(gB8 + buf * kTileB8, lrow, lslot, dx);
    }
    if (lslot == 0) {
      const bool ok = tile * kBT + lrow < n;
      gL[buf * kBT + lrow] = ok ? -(ln * kLog2e) * inv_c : -INFINITY;
      gDn[buf * kBT + lrow] = ok ? -dn : 0.f;
    }
  };
  Raw8<F8> qx, dx;
  float ln = 0.f, dn = 0.f;
  fetch(0, qx, dx, ln, dn);

  // V rows of the work-group's 256 keys (clamped past the end), swizzled like
  // the tiles: key row r at chunk c ^ uswz(r) in bf16, or as codes at slot
  // c ^ swz8(r) on the 8-bit path (V only enters dP, read row-major)
  const int key0 = wi.qtile * kBM;
#pragma unroll
  for (int i = 0; i < kBM * kCH / kThreads; ++i) {
    const int r = lrow + i * kBT;
    const int64_t e = (int64_t)rows.tok(key0 + r) * rs + lslot * 8;
    if constexpr (F8) stash8(gVk8, r, lslot, load_raw8<true>(vb, e));   // as codes
    else *(uint4*)(gVk + r * kRowB + (lslot ^ uswz(r)) * 16) = load8<F8>(vb, e);
  }

  const int jk = key0 + wave * 32 + l32;
  const bool kok = jk < n;
  const int64_t koff = (int64_t)rows.tok(jk) * rs;
  bf16x8 kf[KK];   // bf16 path
  intx8 kf8[2];    // 8-bit path: codes for the e4m3 matrix core
  if constexpr (F8) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      kf8[kk] = frag8_global(kb + koff, hl, kk);
      __asm__ volatile("" : "+v"(kf8[kk]));
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      kf[kk] = as_bf16x8(load8<F8>(kb, koff + kk * 16 + hl * 8));
      __asm__ volatile("" : "+v"(kf[kk]));
    }
  }
  const char* sVk = gVk + wave * 32 * kRowB;     // the wave's 32 key rows
  const char* sVk8 = gVk8 + wave * 32 * kRowB8;  // the same as codes (8-bit path)

  stash(0, 0, qx, dx, ln, dn);
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
    if constexpr (F8) {
      const char* sQ8 = gA8 + buf * kTileB8;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(frag8_rows(sQ8, l32, hl, kk), kf8[kk], s, 0, 0, 0, 0, 0, 0);
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows(sQ, l32, hl, kk), kf[kk], s, 0, 0, 0);
    }
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
    if constexpr (F8) {
      const char* sD8 = gB8 + buf * kTileB8;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        dp = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(frag8_rows(sD8, l32, hl, kk), frag8_rows(sVk8, l32, hl, kk),
                                                             dp, 0, 0, 0, 0, 0, 0);
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows(sD, l32, hl, kk), frag_rows(sVk, l32, hl, kk), dp, 0, 0, 0);
    }
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
    if (more) stash(buf ^ 1, j + 1, qx, dx, ln, dn);
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
  const hipError_t e = launch_bwd_dq(a, F8, table, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_dkv_fused_kernel<F8>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(AttnArgs a, int B, int d, hipStream_t stream) { return launch_bwd<false>(a, B, d, stream); }

hipError_t launch_attn_bwd_fp8(AttnArgs a, int B, int d, hipStream_t stream) { return launch_bwd<true>(a, B, d, stream); }

}  // namespace skiparse
