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
// the B operand.
//
// K order inside the MFMA.  A dot product does not depend on the order of
// its K terms, so each 32-wide K block (one weight word) is fed to the MFMA
// in a permuted order, the same for A and B: the bf16 pair in B dword q of
// a lane holds the weights of bits j and j + 16 of one word.  Then one shift
// brings both bits to positions 15 and 31 (the bf16 sign bits) and one
// three-input bit operation turns the word into {+-1, +-1}
// ((X & 0x80008000) ^ 0xBF80BF80).  X is permuted the same way once, while
// it is copied into LDS (one v_perm_b32 per output dword).
//   Within a word block, MFMA K index kappa = 8 h + 2 q + t of step s (h =
//   lane / 32, q = dword, t = half) carries the real K offset
//   8 (s & 1) + 4 h + q + 16 t.  LDS chunk c = 2 (s & 1) + h of the block's
//   64 bytes holds real offsets {4 c + q + 16 t}.
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

// B fragment of one step: dword q = {w bit j, w bit j + 16} as bf16 +-1, where
// the per-lane pre-shifted word ws already accounts for the lane's half and
// `sh` = 11 - 8 (s & 1) - q.
__device__ __forceinline__ uint32_t sign_pair(uint32_t ws, int sh) {
  return ((ws << sh) & 0x80008000u) ^ 0xBF80BF80u;
}

// Permute one 64-byte row segment (32 bf16 of real K order, as 4 uint4) into
// the MFMA K order described above.
__device__ __forceinline__ void permute_segment(const uint4 (&in)[4], uint4 (&out)[4]) {
  const uint32_t v[16] = {in[0].x, in[0].y, in[0].z, in[0].w, in[1].x, in[1].y, in[1].z, in[1].w,
                          in[2].x, in[2].y, in[2].z, in[2].w, in[3].x, in[3].y, in[3].z, in[3].w};
  uint32_t o[16];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = 4 * c + q;           // real offset of the low half
      const int i1 = k >> 1, i2 = i1 + 8;  // input dwords of k and k + 16
      // low half: bf16 k of dword i1, high half: bf16 k + 16 of dword i2
      const uint32_t sel = (k & 1) ? 0x07060302u : 0x05040100u;
      o[4 * c + q] = __builtin_amdgcn_perm(v[i2], v[i1], sel);
    }
#pragma unroll
  for (int c = 0; c < 4; ++c) out[c] = make_uint4(o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]);
}

// Staged 64 bytes of X per thread and one group's weights / scales per lane;
// plain structs of scalars so that the values stay in registers.
struct AStage {
  uint4 q0, q1, q2, q3;
};
struct WStage {
  uint4 w0, w1;
  float s0, s1;
};

template <bool XPERM>
__device__ __forceinline__ AStage load_a(const uint16_t* const (&src)[4], int g) {
  AStage r;
  if constexpr (XPERM) {
    r.q0 = *reinterpret_cast<const uint4*>(src[0] + g * 128);
    r.q1 = *reinterpret_cast<const uint4*>(src[1] + g * 128);
    r.q2 = *reinterpret_cast<const uint4*>(src[2] + g * 128);
    r.q3 = *reinterpret_cast<const uint4*>(src[3] + g * 128);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(src[0] + g * 128);
    r.q0 = p[0];
    r.q1 = p[1];
    r.q2 = p[2];
    r.q3 = p[3];
  }
  return r;
}

template <bool XPERM>
__device__ __forceinline__ void store_a(char* __restrict__ buf, int a_row, int a_col,
                                        const AStage& r) {
  if constexpr (XPERM) {
    *reinterpret_cast<uint4*>(buf + (a_row + 0) * kRowBytes + a_col * 16) = r.q0;
    *reinterpret_cast<uint4*>(buf + (a_row + 32) * kRowBytes + a_col * 16) = r.q1;
    *reinterpret_cast<uint4*>(buf + (a_row + 64) * kRowBytes + a_col * 16) = r.q2;
    *reinterpret_cast<uint4*>(buf + (a_row + 96) * kRowBytes + a_col * 16) = r.q3;
  } else {
    const uint4 in[4] = {r.q0, r.q1, r.q2, r.q3};
    uint4 o[4];
    permute_segment(in, o);
    uint4* dst = reinterpret_cast<uint4*>(buf + a_row * kRowBytes + a_col * 64);
    dst[0] = o[0];
    dst[1] = o[1];
    dst[2] = o[2];
    dst[3] = o[3];
  }
}

__device__ __forceinline__ WStage load_w(const uint4* const (&w)[2], const float* const (&sc)[2],
                                         int g) {
  WStage r;
  r.w0 = w[0][g];
  r.w1 = w[1][g];
  r.s0 = sc[0][g];
  r.s1 = sc[1][g];
  return r;
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// One 128-K group: eight MFMA steps into fresh group accumulators P, then
// acc += scale * P.  `abuf` is this wave's X tile in LDS.
__device__ __forceinline__ void compute_group(const char* __restrict__ abuf, int wm, int c32,
                                              int h, int hshift, const WStage& wst,
                                              f32x16 (&acc)[2][2]) {
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
      const uint32_t ws = word_of(j == 0 ? wst.w0 : wst.w1, s >> 1) << hshift;
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 d = {sign_pair(ws, 11 - 8 * (s & 1)), sign_pair(ws, 10 - 8 * (s & 1)),
                       sign_pair(ws, 9 - 8 * (s & 1)), sign_pair(ws, 8 - 8 * (s & 1))};
      b[j] = __builtin_bit_cast(bf16x8, d);
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
    for (int v = 0; v < 16; ++v) {
      acc[i][0][v] = fmaf(wst.s0, P[i][0][v], acc[i][0][v]);
      acc[i][1][v] = fmaf(wst.s1, P[i][1][v], acc[i][1][v]);
    }
}

template <bool XPERM>  // X is in the GEMM K order already (no permutation in the kernel)
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
  const int hshift = h ? 0 : 4;  // lanes of the first K half use bits 4 lower

  // ---- per-thread global->LDS copy of X.  Rows past M (and, below, columns
  // past N) read a valid row instead: they only feed outputs never stored.
  //  XPERM: 4 chunks of 16 B from rows a_row + 32 q, 16 threads per row
  //         (coalesced), copied as they are.
  //  else:  one 64-byte segment (a word block of 32 bf16) per thread, 4
  //         threads per row, permuted into the GEMM K order on the way.
  const int a_row = XPERM ? (tid >> 4) : (tid >> 2);
  const int a_col = XPERM ? (tid & 15) : (tid & 3);
  const uint16_t* a_src[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    a_src[q] = X + static_cast<int64_t>(min(m0 + a_row + (XPERM ? 32 * q : 0), M - 1)) * K +
               a_col * (XPERM ? 8 : 32);

  // ---- weights: this lane's two columns
  int col[2];
  bool c_in[2];
  const uint4* w_src[2];
  const float* s_src[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    col[j] = n0 + wn * WN + 32 * j + c32;
    c_in[j] = col[j] < N;
    const int64_t cc = min(col[j], N - 1);
    w_src[j] = reinterpret_cast<const uint4*>(W + cc * KW);
    s_src[j] = S + cc * G;
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  {
    const AStage a = load_a<XPERM>(a_src, 0);
    store_a<XPERM>(smem, a_row, a_col, a);
  }
  WStage wA = load_w(w_src, s_src, 0);
  __syncthreads();

  // Two groups per trip: the next group's X and weights are loaded before
  // the current group's MFMAs and consumed after them, with no register copy.
  // The loads are unconditional (the group index is clamped; a clamped load
  // fetches data that is never used) so that no branch forces an early wait.
  for (int g = 0; g < G; g += 2) {
    const int g1 = min(g + 1, G - 1);
    const AStage a1 = load_a<XPERM>(a_src, g1);
    const WStage wB = load_w(w_src, s_src, g1);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the MFMAs
    compute_group(smem, wm, c32, h, hshift, wA, acc);
    store_a<XPERM>(smem + kTileBytes, a_row, a_col, a1);
    __syncthreads();
    if (g + 1 >= G) break;
    const int g2 = min(g + 2, G - 1);
    const AStage a2 = load_a<XPERM>(a_src, g2);
    wA = load_w(w_src, s_src, g2);
    __builtin_amdgcn_sched_barrier(0);
    compute_group(smem + kTileBytes, wm, c32, h, hshift, wB, acc);
    store_a<XPERM>(smem, a_row, a_col, a2);
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

hipError_t launch_gemm(const uint16_t* x_bf16, bool x_gemm_order, const uint32_t* w_bits,
                       const float* scales, float* y, int64_t M, int64_t N, int64_t K,
                       hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((N + BN - 1) / BN), static_cast<unsigned>((M + BM - 1) / BM));
  if (x_gemm_order)
    hipLaunchKernelGGL(gemm_kernel<true>, grid, dim3(kThreads), 0, stream, x_bf16, w_bits, scales,
                       y, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K));
  else
    hipLaunchKernelGGL(gemm_kernel<false>, grid, dim3(kThreads), 0, stream, x_bf16, w_bits, scales,
                       y, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K));
  return hipGetLastError();
}

}  // namespace pq1
