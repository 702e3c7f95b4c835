// e4m3 GEMM with bf16 output for the block's projections:
//   Y (M x N, row-major) = sx * sw * X (M x K, row-major) . W (N x K, row-major)^T
// with per-tensor dequantization factors sx, sw read from the device.  Both
// operands are K-contiguous, so rows of W feed the MFMA A operand and rows of X
// the B operand directly: each lane then holds 4 consecutive outputs of one
// row of Y, stored as one 8-byte write.
//
// A work-group computes a TN (W rows) x TM (X rows) tile; each wave owns
// WTN x WTM of it as (WTN/32) x (WTM/32) blocks of
// v_mfma_scale_f32_32x32x64_f8f6f4.  K advances 128 bytes per step through
// double-buffered LDS filled from registers loaded one step ahead; 16-byte
// chunks are XOR-swizzled by row / 2 so 16 lanes reading one chunk column of
// 16 rows spread over all 64 banks.  Rows of X past M are clamped on load and masked
// on store.  Tiles are handed out XCD by XCD (work-groups are dispatched to the
// 8 XCDs round-robin), so the tiles that share rows of X run on one XCD and
// share its L2.
//
// Two shapes: 256 x 256 tiles with 8 waves of 128 x 64 (arithmetic intensity
// 256 FLOP per byte of operand traffic) when N is a multiple of 256, else
// 128 x 128 with 4 waves of 64 x 64.
#include "block.h"

namespace skiparse {
namespace {

typedef int intx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kTK = 128;     // bytes of K per step
constexpr int kXcd = 8;

// LDS has 64 banks of 4 bytes: two 128-byte rows share one bank line, and a
// 16-lane group of ds_read_b128 reads 16 rows at one chunk.  Rotating the
// chunk with row / 2 gives those 16 rows 16 distinct (row parity, chunk)
// slots, i.e. all 64 banks once.
__device__ __forceinline__ int chunk_addr(int row, int chunk) {
  return row * kTK + ((chunk ^ ((row >> 1) & 7)) << 4);
}

template <int TN, int TM, int WTN, int WTM>
struct GemmCfg {
  static constexpr int kWavesN = TN / WTN, kWavesM = TM / WTM;
  static constexpr int kWaves = kWavesN * kWavesM;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBN = WTN / 32, kBM = WTM / 32;         // MFMA blocks per wave
  static constexpr int kLW = TN * (kTK / 16) / kThreads;       // 16-byte W chunks per thread and step
  static constexpr int kLX = TM * (kTK / 16) / kThreads;
  static constexpr int kRowsPerPass = kThreads / (kTK / 16);   // rows one pass of the loader covers
  static constexpr int kTileW = TN * kTK, kTileX = TM * kTK;
  static constexpr int kLds = 2 * (kTileW + kTileX);
  static_assert(kLW * kThreads == TN * (kTK / 16) && kLX * kThreads == TM * (kTK / 16), "loader split");
  static_assert(kRowsPerPass % 16 == 0, "rows of one chunk slot share the swizzle");
};

template <int TN, int TM, int WTN, int WTM>
__global__ void __launch_bounds__(64 * (TN / WTN) * (TM / WTM))
gemm_fp8_bf16_kernel(const uint8_t* __restrict__ x, const uint8_t* __restrict__ w, const float* __restrict__ sx,
                     const float* __restrict__ sw, __bf16* __restrict__ y, int M, int N, int K, int tiles_n,
                     int total) {
  using Cfg = GemmCfg<TN, TM, WTN, WTM>;
  constexpr int kBN = Cfg::kBN, kBM = Cfg::kBM, kLW = Cfg::kLW, kLX = Cfg::kLX, kRP = Cfg::kRowsPerPass;
  __shared__ __attribute__((aligned(16))) char lds[Cfg::kLds];   // W0 W1 X0 X1
  char* const ldsW = lds;
  char* const ldsX = lds + 2 * Cfg::kTileW;

  // XCD-major tile order: XCD c runs logical tiles [start(c), start(c) + count(c)).
  const int bid = blockIdx.x;
  const int q = total / kXcd, r = total % kXcd;
  const int c = bid % kXcd;
  const int tile = c * q + (c < r ? c : r) + bid / kXcd;
  const int n0 = (tile % tiles_n) * TN;
  const int m0 = (tile / tiles_n) * TM;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  const int wn = (wave % Cfg::kWavesN) * WTN;   // wave's W rows within the tile
  const int wm = (wave / Cfg::kWavesN) * WTM;   // wave's X rows within the tile

  // loader: pass s < 4 covers rows tid / 8 + kRP * s, 16-byte slot tid % 8;
  // X rows past M are clamped.  Four named registers per operand (not an
  // array, which the compiler would move to LDS).
  static_assert(kLW == 4 && kLX == 4, "the loader holds four chunks per operand");
  const int lrow = tid >> 3, slot = tid & 7;
  const uint8_t* wsrc = w + (int64_t)(n0 + lrow) * K + slot * 16;
  const int64_t wpass = (int64_t)kRP * K;
  auto xrow = [&](int s) -> const uint8_t* {
    const int xr = m0 + lrow + kRP * s;
    return x + (int64_t)(xr < M ? xr : M - 1) * K + slot * 16;
  };
  const uint8_t* const xs0 = xrow(0);
  const uint8_t* const xs1 = xrow(1);
  const uint8_t* const xs2 = xrow(2);
  const uint8_t* const xs3 = xrow(3);
  const int st_off = chunk_addr(lrow, slot);  // rows lrow + kRP s share the swizzle (kRP % 16 == 0)

  floatx16 acc[kBN][kBM];
#pragma unroll
  for (int a = 0; a < kBN; ++a)
#pragma unroll
    for (int b = 0; b < kBM; ++b) acc[a][b] = floatx16{};

  uint4 w0 = *(const uint4*)(wsrc), w1 = *(const uint4*)(wsrc + wpass), w2 = *(const uint4*)(wsrc + 2 * wpass),
        w3 = *(const uint4*)(wsrc + 3 * wpass);
  uint4 x0 = *(const uint4*)(xs0), x1 = *(const uint4*)(xs1), x2 = *(const uint4*)(xs2), x3 = *(const uint4*)(xs3);
  constexpr int kPass = kRP * kTK;   // LDS bytes between passes
  {
    char* dW = ldsW + st_off;
    char* dX = ldsX + st_off;
    *(uint4*)(dW) = w0, *(uint4*)(dW + kPass) = w1, *(uint4*)(dW + 2 * kPass) = w2, *(uint4*)(dW + 3 * kPass) = w3;
    *(uint4*)(dX) = x0, *(uint4*)(dX + kPass) = x1, *(uint4*)(dX + 2 * kPass) = x2, *(uint4*)(dX + 3 * kPass) = x3;
  }
  __syncthreads();

  const int steps = K / kTK;
  for (int st = 0; st < steps; ++st) {
    const int buf = st & 1;
    const bool more = st + 1 < steps;
    if (more) {
      const int k0 = (st + 1) * kTK;
      w0 = *(const uint4*)(wsrc + k0);
      w1 = *(const uint4*)(wsrc + wpass + k0);
      w2 = *(const uint4*)(wsrc + 2 * wpass + k0);
      w3 = *(const uint4*)(wsrc + 3 * wpass + k0);
      x0 = *(const uint4*)(xs0 + k0);
      x1 = *(const uint4*)(xs1 + k0);
      x2 = *(const uint4*)(xs2 + k0);
      x3 = *(const uint4*)(xs3 + k0);
    }
    const char* sW = ldsW + buf * Cfg::kTileW;
    const char* sX = ldsX + buf * Cfg::kTileX;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ch = 4 * kk + 2 * hl;
      intx8 bf[kBM];
#pragma unroll
      for (int b = 0; b < kBM; ++b) {
        const int rxr = wm + b * 32 + l32;
        const uint4 b0 = *(const uint4*)(sX + chunk_addr(rxr, ch));
        const uint4 b1 = *(const uint4*)(sX + chunk_addr(rxr, ch + 1));
        bf[b] = intx8{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
      }
#pragma unroll
      for (int a = 0; a < kBN; ++a) {
        const int rwr = wn + a * 32 + l32;
        const uint4 a0 = *(const uint4*)(sW + chunk_addr(rwr, ch));
        const uint4 a1 = *(const uint4*)(sW + chunk_addr(rwr, ch + 1));
        const intx8 af = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
#pragma unroll
        for (int b = 0; b < kBM; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf[b], acc[a][b], 0, 0, 0, 0, 0, 0);
      }
    }
    if (more) {
      char* dW = ldsW + (buf ^ 1) * Cfg::kTileW + st_off;
      char* dX = ldsX + (buf ^ 1) * Cfg::kTileX + st_off;
      *(uint4*)(dW) = w0, *(uint4*)(dW + kPass) = w1, *(uint4*)(dW + 2 * kPass) = w2, *(uint4*)(dW + 3 * kPass) = w3;
      *(uint4*)(dX) = x0, *(uint4*)(dX + kPass) = x1, *(uint4*)(dX + 2 * kPass) = x2, *(uint4*)(dX + 3 * kPass) = x3;
    }
    __syncthreads();
  }

  // acc[a][b] lane (hl, l32) reg i: n = n0 + wn + 32a + 8(i/4) + 4hl + i%4,
  // m = m0 + wm + 32b + l32
  const float s = sx[0] * sw[0];
#pragma unroll
  for (int b = 0; b < kBM; ++b) {
    const int m = m0 + wm + b * 32 + l32;
    if (m >= M) continue;
    __bf16* yrow = y + (int64_t)m * N + n0 + wn + 4 * hl;
#pragma unroll
    for (int a = 0; a < kBN; ++a)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[a][b][4 * g + e] * s);
        *(bf16x4*)(yrow + 32 * a + 8 * g) = v;
      }
  }
}

template <int TN, int TM, int WTN, int WTM>
hipError_t launch_cfg(const uint8_t* x, const uint8_t* w, const float* sx, const float* sw, void* y, int64_t M,
                      int N, int K, hipStream_t stream) {
  const int tiles_n = N / TN;
  const int64_t total = (M + TM - 1) / TM * tiles_n;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_fp8_bf16_kernel<TN, TM, WTN, WTM>), dim3((unsigned)total),
                     dim3(GemmCfg<TN, TM, WTN, WTM>::kThreads), 0, stream, x, w, sx, sw, (__bf16*)y, (int)M, N, K,
                     tiles_n, (int)total);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp8_bf16(const uint8_t* x, const uint8_t* w, const float* sx, const float* sw, void* y,
                                int64_t M, int N, int K, hipStream_t stream) {
  if (N % 256 == 0) return launch_cfg<256, 256, 128, 64>(x, w, sx, sw, y, M, N, K, stream);
  return launch_cfg<128, 128, 64, 64>(x, w, sx, sw, y, M, N, K, stream);
}

}  // namespace skiparse
