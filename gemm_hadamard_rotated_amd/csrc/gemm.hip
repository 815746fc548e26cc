// Prefill GEMM on bf16 MFMA: Y[m][n] = sum_g scale[n][g] * sum_{k in g} X[m][k] * (+-1)(n, k).
//
// X is the rotated activation rounded to bf16; a +-1 weight is exact in bf16,
// so every product is exact and the fp32 MFMA accumulation is the only
// rounding inside a 128-wide K group.  For each group the kernel runs a fresh
// chain of eight v_mfma_f32_32x32x16_bf16 (K = 16 each) into a group
// accumulator P, then adds scale * P to the output accumulator in fp32 --
// the scale of a column is the same for all of its 32x32 block, and every lane
// of the MFMA output holds a single column, so that is one FMA per element.
//
// Tiling: a 512-thread workgroup computes a 128 (M) x 256 (N) tile; wave w
// owns the 64x64 sub-tile (w / 4, w % 4) as 2x2 blocks of 32x32.  Per 128-K
// group the X tile (128 x 128 bf16 = 32 KB) is staged in LDS (double
// buffered, rows padded to 272 B so the 16-byte fragment reads of 8
// consecutive rows hit distinct banks); the 1-bit weights go straight to
// registers (16 bytes per column per group) and are expanded to bf16 +-1 in
// the B operand: two bits become one dword {+-1, +-1} with a multiply that
// spreads them to bits 15 and 31 and an xor onto 0xBF80BF80 (-1, -1).
//
// MFMA operand layout (v_mfma_f32_32x32x16_bf16, wave64): lane l holds
// A[l % 32][8 (l / 32) .. +7] and B[8 (l / 32) .. +7][l % 32]; the 16 output
// registers of lane l hold D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32].
#include "pq1_internal.h"

namespace pq1 {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 256;
constexpr int WM = 64, WN = 64;
constexpr int kThreads = 512;
constexpr int kRowBytes = 272;                // 128 bf16 + 16 B pad
constexpr int kTileBytes = BM * kRowBytes;    // one X buffer

// 8 weight bits -> 8 bf16 values +-1 (bit set = +1).
__device__ __forceinline__ bf16x8 expand8(uint32_t byte) {
  uint32_t d[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t b2 = (byte >> (2 * q)) & 3u;
    d[q] = ((b2 * 0x40008000u) & 0x80008000u) ^ 0xBF80BF80u;
  }
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = {d[0], d[1], d[2], d[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__global__ __launch_bounds__(kThreads) void gemm_kernel(const uint16_t* __restrict__ X,
                                                        const uint32_t* __restrict__ W,
                                                        const float* __restrict__ S,
                                                        float* __restrict__ Y, int M, int N,
                                                        int K) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kTileBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int G = K / 128;
  const int KW = K / 32;
  const int h = lane >> 5;     // which 8-wide K half of a 16-step
  const int c32 = lane & 31;

  // ---- per-thread global->LDS copy assignment for X: 4 chunks of 16 B
  int a_row[4], a_cc[4];
  bool a_in[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = tid + kThreads * q;
    a_row[q] = c >> 4;
    a_cc[q] = c & 15;
    a_in[q] = (m0 + a_row[q]) < M;
  }
  auto load_a = [&](int g, uint4 (&r)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      r[q] = a_in[q] ? *reinterpret_cast<const uint4*>(
                           X + static_cast<int64_t>(m0 + a_row[q]) * K + g * 128 + a_cc[q] * 8)
                     : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_a = [&](int buf, const uint4 (&r)[4]) {
    char* base = smem + buf * kTileBytes;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint4*>(base + a_row[q] * kRowBytes + a_cc[q] * 16) = r[q];
  };

  // ---- weights: this lane's two columns
  int col[2];
  bool c_in[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    col[j] = n0 + wn * WN + 32 * j + c32;
    c_in[j] = col[j] < N;
  }
  auto load_w = [&](int g, uint4 (&w)[2], float (&s)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      w[j] = c_in[j] ? *reinterpret_cast<const uint4*>(W + static_cast<int64_t>(col[j]) * KW + g * 4)
                     : make_uint4(0, 0, 0, 0);
      s[j] = c_in[j] ? S[static_cast<int64_t>(col[j]) * G + g] : 0.0f;
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  uint4 areg[4];
  uint4 wcur[2], wnext[2];
  float scur[2], snext[2];
  load_a(0, areg);
  load_w(0, wcur, scur);
  store_a(0, areg);
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    const bool more = (g + 1) < G;
    if (more) {
      load_a(g + 1, areg);
      load_w(g + 1, wnext, snext);
    }
    const char* abuf = smem + (g & 1) * kTileBytes;
    f32x16 P[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) P[i][j][v] = 0.0f;

#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(abuf + (wm * WM + 32 * i + c32) * kRowBytes +
                                                 s * 32 + h * 16);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t word = (s >> 1) == 0   ? wcur[j].x
                              : (s >> 1) == 1 ? wcur[j].y
                              : (s >> 1) == 2 ? wcur[j].z
                                              : wcur[j].w;
        b[j] = expand8((word >> (16 * (s & 1) + 8 * h)) & 0xFFu);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          P[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], P[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = fmaf(scur[j], P[i][j][v], acc[i][j][v]);

    if (more) {
      store_a((g + 1) & 1, areg);
      wcur[0] = wnext[0];
      wcur[1] = wnext[1];
      scur[0] = snext[0];
      scur[1] = snext[1];
    }
    __syncthreads();
  }

  // ---- store
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (!c_in[j]) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * WM + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        if (row < M) Y[static_cast<int64_t>(row) * N + col[j]] = acc[i][j][v];
      }
    }
}

}  // namespace

hipError_t launch_gemm(const uint16_t* x_bf16, const uint32_t* w_bits, const float* scales,
                       float* y, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((N + BN - 1) / BN), static_cast<unsigned>((M + BM - 1) / BM));
  hipLaunchKernelGGL(gemm_kernel, grid, dim3(kThreads), 0, stream, x_bf16, w_bits,
                     scales, y, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K));
  return hipGetLastError();
}

}  // namespace pq1
