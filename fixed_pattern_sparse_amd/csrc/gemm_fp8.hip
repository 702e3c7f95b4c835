// e4m3 GEMM with bf16 output for the block's projections:
//   Y (M x N, row-major) = sx * sw * X (M x K, row-major) . W (N x K, row-major)^T
// with per-tensor dequantization factors sx, sw read from the device.  Both
// operands are K-contiguous, so rows of W feed the MFMA A operand and rows of X
// the B operand directly: each lane then holds 4 consecutive outputs of one
// row of Y, stored as one 8-byte write.
//
// Work-group: 256 threads (4 waves as 2 x 2), tile 128 (n) x 128 (m); a wave
// owns 64 x 64 as 2 x 2 blocks of v_mfma_scale_f32_32x32x64_f8f6f4.  K advances
// 128 bytes per step through double-buffered LDS (16 KB per operand and
// buffer), filled from registers loaded one step ahead; 16-byte chunks are
// XOR-swizzled by row so 32 lanes reading one chunk column of 32 rows spread
// over all banks.  N and K are multiples of 128; rows of X past M are clamped
// on load and masked on store.  Tiles are handed out XCD by XCD (work-groups
// are dispatched to the 8 XCDs round-robin), so the tiles that share rows of X
// run on one XCD and share its L2.
#include "block.h"

namespace skiparse {
namespace {

typedef int intx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTN = 128;     // W rows (output columns) per tile
constexpr int kTM = 128;     // X rows (output rows) per tile
constexpr int kTK = 128;     // bytes of K per step
constexpr int kTileB = kTN * kTK;   // 16 KB per operand tile (kTN == kTM)
constexpr int kXcd = 8;

__device__ __forceinline__ int chunk_addr(int row, int chunk) { return row * kTK + ((chunk ^ (row & 7)) << 4); }

__global__ void __launch_bounds__(kThreads) gemm_fp8_bf16_kernel(const uint8_t* __restrict__ x,
                                                                 const uint8_t* __restrict__ w,
                                                                 const float* __restrict__ sx,
                                                                 const float* __restrict__ sw,
                                                                 __bf16* __restrict__ y, int M, int N, int K,
                                                                 int tiles_n, int total) {
  __shared__ __attribute__((aligned(16))) char lds[4 * kTileB];   // W0 W1 X0 X1

  // XCD-major tile order: XCD c runs logical tiles [start(c), start(c) + count(c)).
  const int bid = blockIdx.x;
  const int q = total / kXcd, r = total % kXcd;
  const int c = bid % kXcd;
  const int tile = c * q + (c < r ? c : r) + bid / kXcd;
  const int n0 = (tile % tiles_n) * kTN;
  const int m0 = (tile / tiles_n) * kTM;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  const int wn = (wave & 1) * 64;   // wave's W rows within the tile
  const int wm = (wave >> 1) * 64;  // wave's X rows within the tile

  // loader: chunk i = tid + 256 * s (s < 4) is row i / 8 = tid / 8 + 32 s,
  // 16-byte slot i % 8 = tid % 8; X rows past M are clamped.
  const int lrow = tid >> 3, slot = tid & 7;
  const uint8_t* wsrc = w + (int64_t)(n0 + lrow) * K + slot * 16;
  int64_t xoff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int xr = m0 + lrow + 32 * s;
    xoff[s] = (int64_t)(xr < M ? xr : M - 1) * K + slot * 16;
  }
  const int64_t wstep = (int64_t)32 * K;      // 32 rows of W
  const int st_off = chunk_addr(lrow, slot);  // rows lrow + 32 s share the swizzle (32 s & 7 == 0)

  floatx16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = floatx16{};

  const int steps = K / kTK;
  uint4 w0r = *(const uint4*)(wsrc), w1r = *(const uint4*)(wsrc + wstep), w2r = *(const uint4*)(wsrc + 2 * wstep),
        w3r = *(const uint4*)(wsrc + 3 * wstep);
  uint4 x0r = *(const uint4*)(x + xoff[0]), x1r = *(const uint4*)(x + xoff[1]), x2r = *(const uint4*)(x + xoff[2]),
        x3r = *(const uint4*)(x + xoff[3]);
  {
    char* dW = lds + st_off;
    char* dX = lds + 2 * kTileB + st_off;
    *(uint4*)(dW) = w0r, *(uint4*)(dW + 32 * kTK) = w1r, *(uint4*)(dW + 64 * kTK) = w2r, *(uint4*)(dW + 96 * kTK) = w3r;
    *(uint4*)(dX) = x0r, *(uint4*)(dX + 32 * kTK) = x1r, *(uint4*)(dX + 64 * kTK) = x2r, *(uint4*)(dX + 96 * kTK) = x3r;
  }
  __syncthreads();
  for (int st = 0; st < steps; ++st) {
    const int buf = st & 1;
    const bool more = st + 1 < steps;
    if (more) {
      const int k0 = (st + 1) * kTK;
      w0r = *(const uint4*)(wsrc + k0);
      w1r = *(const uint4*)(wsrc + wstep + k0);
      w2r = *(const uint4*)(wsrc + 2 * wstep + k0);
      w3r = *(const uint4*)(wsrc + 3 * wstep + k0);
      x0r = *(const uint4*)(x + xoff[0] + k0);
      x1r = *(const uint4*)(x + xoff[1] + k0);
      x2r = *(const uint4*)(x + xoff[2] + k0);
      x3r = *(const uint4*)(x + xoff[3] + k0);
    }
    const char* sW = lds + buf * kTileB;
    const char* sX = lds + (2 + buf) * kTileB;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      intx8 af[2], bf[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int rw = wn + b * 32 + l32;
        const int rx = wm + b * 32 + l32;
        const int ch = 4 * kk + 2 * hl;
        const uint4 a0 = *(const uint4*)(sW + chunk_addr(rw, ch));
        const uint4 a1 = *(const uint4*)(sW + chunk_addr(rw, ch + 1));
        const uint4 b0 = *(const uint4*)(sX + chunk_addr(rx, ch));
        const uint4 b1 = *(const uint4*)(sX + chunk_addr(rx, ch + 1));
        af[b] = intx8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        bf[b] = intx8{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[a], bf[b], acc[a][b], 0, 0, 0, 0, 0, 0);
    }
    if (more) {
      char* dW = lds + (buf ^ 1) * kTileB + st_off;
      char* dX = lds + (2 + (buf ^ 1)) * kTileB + st_off;
      *(uint4*)(dW) = w0r, *(uint4*)(dW + 32 * kTK) = w1r, *(uint4*)(dW + 64 * kTK) = w2r, *(uint4*)(dW + 96 * kTK) = w3r;
      *(uint4*)(dX) = x0r, *(uint4*)(dX + 32 * kTK) = x1r, *(uint4*)(dX + 64 * kTK) = x2r, *(uint4*)(dX + 96 * kTK) = x3r;
    }
    __syncthreads();
  }

  // acc[a][b] lane (hl, l32) reg i: n = n0 + wn + 32a + 8(i/4) + 4hl + i%4,
  // m = m0 + wm + 32b + l32
  const float s = sx[0] * sw[0];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int m = m0 + wm + b * 32 + l32;
    if (m >= M) continue;
    __bf16* yrow = y + (int64_t)m * N + n0 + wn + 4 * hl;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[a][b][4 * g + e] * s);
        *(bf16x4*)(yrow + 32 * a + 8 * g) = v;
      }
  }
}

}  // namespace

hipError_t launch_gemm_fp8_bf16(const uint8_t* x, const uint8_t* w, const float* sx, const float* sw, void* y,
                                int64_t M, int N, int K, hipStream_t stream) {
  const int tiles_n = N / kTN;
  const int64_t tiles_m = (M + kTM - 1) / kTM;
  const int64_t total = tiles_m * tiles_n;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_fp8_bf16_kernel, dim3((unsigned)total), dim3(kThreads), 0, stream, x, w, sx, sw,
                     (__bf16*)y, (int)M, N, K, tiles_n, (int)total);
  return hipGetLastError();
}

}  // namespace skiparse
