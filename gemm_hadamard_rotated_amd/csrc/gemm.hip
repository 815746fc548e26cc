// ---------------------------------------------------------------------------
// Prefill GEMM on bf16 MFMA: Y[m][n] = sum_g scale[n][g] * sum_{k in g} X[m][k] * (+-1)(n, k).
//
// X is the rotated activation rounded to bf16; a +-1 weight is exact in bf16,
// so every product is exact and the fp32 MFMA accumulation is the only
// rounding inside a 128-wide K group.  For each group a fresh chain of eight
// v_mfma_f32_32x32x16_bf16 (K = 16 each) accumulates a group sum P, and
// scale * P is then added to the output accumulator in fp32 -- the scale of a
// column is the same for all of its 32x32 block and every lane of the MFMA
// output holds a single column, so that is one FMA per element.
//
// K order inside the MFMA.  A dot product does not depend on the order of
// its K terms, so each 32-wide K block (one weight word) is fed to the MFMA
// in a permuted order, the same for A and B: the bf16 pair in B dword q of
// a lane holds the weights of bits j and j + 16 of one word.  Then one shift
// brings both bits to positions 15 and 31 (the bf16 sign bits) and one
// three-input bit operation turns the word into {+-1, +-1}
// ((X & 0x80008000) ^ 0xBF80BF80).  The rotation can write X in this order
// (PQ1_BF16_GEMM).  Row-major X (natural K order) takes the same tile kernel
// with a B fragment that costs one byte permute more per MFMA step (see
// b_fragment_nat).
//   Within a word block, MFMA K index kappa = 8 h + 2 q + t of step s (h =
//   lane / 32, q = dword, t = half) carries the real K offset
//   8 (s & 1) + 4 h + q + 16 t.  LDS chunk c = 2 (s & 1) + h of the block's
//   64 bytes holds real offsets {4 c + q + 16 t}.
//
// MFMA operand layout (v_mfma_f32_32x32x16_bf16, wave64): lane l holds
// A[l % 32][8 (l / 32) .. +7] and B[8 (l / 32) .. +7][l % 32]; the 16 output
// registers of lane l hold D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32].
//
// Three kernels:
//  * gemm_xg_kernel (X already in the GEMM K order): workgroup tile 128 (M) x
//    128 (N), four waves, each wave a 128 x 32 strip (4 M-blocks x 1
//    N-block).  Every column's bit expansion is done once and feeds four
//    MFMAs; each wave reads all 128 rows of the X tile from LDS (one 16-byte
//    fragment per MFMA).  Two workgroups fit on a CU (64 KB of LDS, 248
//    VGPRs per lane).  X rows are stored unpadded (256 bytes) with the
//    16-byte chunks XOR-swizzled by (row & 15), so the fragment reads of 16
//    consecutive rows hit distinct banks.  X is copied one group ahead
//    straight from memory into LDS (buffer-to-LDS loads, no registers), the
//    weights two groups ahead into registers; all global reads are buffer
//    loads with 32-bit offsets from the workgroup's rows and columns.  The
//    previous group's P of a block is folded into the output accumulator
//    right before the block's first MFMA of the next group, overlapping the
//    other blocks' MFMAs.
//    Tail split: when the tiles leave a last round that fills at most a
//    quarter of the resident workgroup slots (1088 tiles on 512 slots for the
//    1024 x 17408 prefill: 64 left over), each of those last tiles is run as
//    four 32 x 128 pieces instead (32 rows of X staged, one 32 x 32 block
//    per wave).  The pieces do a quarter of a tile's MFMAs and staging each
//    and spread over all CUs, so the last round ends sooner.  Every output
//    still comes from the same MFMA chain and fold order, so results do not
//    depend on the split.
//  * gemm_xg_nat_kernel (row-major X, natural K order): the same tile,
//    staging and tail split; only the B fragment differs.
//  * gemm_skinny_kernel (M <= 64 while its weights fit the LDS limit, either
//    layout; in gemm_skinny.hip): 1, 2, 4 or 5 blocks of 16 columns per
//    workgroup, as many as balance the workgroups over the CUs, K split over
//    its waves, each wave's weights copied into LDS in one burst,
//    v_mfma_f32_16x16x32_bf16.
// ---------------------------------------------------------------------------
#include "gemm_common.h"
#include "pq1_internal.h"

namespace pq1 {

namespace {

using namespace gemm_detail;

// ===========================================================================
// 128 x 128 tile, four 128 x 32 waves; X in the GEMM K order (NAT false) or
// row-major in the natural K order (NAT true).  In both layouts LDS chunk c
// of a row holds the 8 X values that MFMA step c / 2, lane half c % 2 reads;
// only the B fragment differs.
// ===========================================================================
constexpr int XG_BM = 128, XG_BN = 128, XG_WAVES = 4, XG_THREADS = 64 * XG_WAVES;
constexpr int XG_ROW = 256;                  // bytes per LDS row (128 bf16), swizzled
constexpr int XG_TILE = XG_BM * XG_ROW;      // one X buffer (32 KB)

// A workgroup stages 32 MB rows of X (MB = M-blocks per wave: 4 for a whole
// tile, 1 for a 32-row piece) straight from memory into LDS: each wave issues
// 2 MB buffer-to-LDS loads per group, each filling 1 KB of LDS (4 rows, 16
// bytes per lane in lane order) without passing through registers.  Copy q
// of a wave fills rows wave * 8 MB + q * 4 .. +3; lane l writes row
// + l / 16, chunk slot l % 16, which holds global chunk (l % 16) ^ (row & 15)
// (`off` holds those per-lane source offsets).  `goff` is the group's byte
// offset within a row.
template <int MB>
__device__ __forceinline__ void xg_copy(char* buf, __amdgpu_buffer_rsrc_t xr, int goff,
                                        const uint32_t* off, int wave) {
#pragma unroll
  for (int q = 0; q < 2 * MB; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        xr, (lds_void*)(buf + (wave * (8 * MB) + q * 4) * XG_ROW), 16, off[q],
        goff, 0, 0);
}

// One group: 8 steps x (MB A fragments, 1 B fragment, MB MFMAs) into P.
// Block i's previous P is folded into acc (scale ps) right before its first
// MFMA.  abuf points at the wave's first A row in the tile buffer.
template <int MB, bool NAT>
__device__ __forceinline__ void xg_group(const char* __restrict__ abuf, int lr, int h, int hshift,
                                         uint32_t sel0, uint32_t sel1, const uint4& w,
                                         f32x16 (&P)[MB], float ps, f32x16 (&acc)[MB]) {
  const f32x16 zero = {};
  const int sw = lr & 15;  // the wave's first row is a multiple of 32
  const char* rowp = abuf + lr * XG_ROW;
  bf16x8 an[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
    an[i] = *reinterpret_cast<const bf16x8*>(rowp + 32 * i * XG_ROW + (h ^ sw) * 16);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    bf16x8 a[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) a[i] = an[i];
    if (s < 7) {  // next step's fragments, one step ahead
      const int slot = (2 * (s + 1) + h) ^ sw;
#pragma unroll
      for (int i = 0; i < MB; ++i)
        an[i] = *reinterpret_cast<const bf16x8*>(rowp + 32 * i * XG_ROW + slot * 16);
    }
    const bf16x8 b = NAT ? b_fragment_nat(w, s, (s & 1) ? sel1 : sel0) : b_fragment(w, s, hshift);
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if (s == 0) {
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = fmaf(ps, P[i][v], acc[i][v]);
      }
      P[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b, s == 0 ? zero : P[i], 0, 0, 0);
    }
  }
}

// One workgroup's work: rows m0 .. m0 + 32 MB - 1 of X staged through LDS by
// all four waves; this wave computes those rows (M-blocks i < MB) of column
// n0 + 32 wave + lane % 32 (one column per lane).  Offsets inside the
// workgroup's X rows and weight columns fit 32 bits (M K < 2^31 elements,
// K < 2^28).
template <int MB, bool NAT>
__device__ __forceinline__ void xg_tile(const uint16_t* __restrict__ X,
                                        const uint32_t* __restrict__ W,
                                        const float* __restrict__ S, float* __restrict__ Y,
                                        int M, int N, int K, int m0, int n0, char* buf0,
                                        char* buf1) {
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int G = K / 128, KW = K / 32;
  const int h = lane >> 5, lr = lane & 31;
  const int hshift = h ? 0 : 4;  // lanes of the first K half use bits 4 lower
  // natural order: byte h (s even) or 2 + h (s odd) of the word into bytes 0 and 2
  const uint32_t sel0 = (0x0C000C00u | static_cast<uint32_t>(h)) | (static_cast<uint32_t>(h) << 16);
  const uint32_t sel1 = sel0 + 0x00020002u;
  const int col = n0 + 32 * wave + lr;

  // X copies: byte offsets from the tile's first row (rows past M read the
  // last row: they only feed outputs that are never stored)
  const __amdgpu_buffer_rsrc_t xr =
      buffer_of(X + static_cast<int64_t>(m0) * K, static_cast<uint32_t>(static_cast<int64_t>(M - m0) * K * 2));
  uint32_t off[2 * MB];
#pragma unroll
  for (int q = 0; q < 2 * MB; ++q) {
    const int r = wave * (8 * MB) + q * 4 + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);
    off[q] = (static_cast<uint32_t>(min(m0 + r, M - 1) - m0) * static_cast<uint32_t>(K) +
              static_cast<uint32_t>(c * 8)) * 2u;
  }
  // this lane's column (columns past N read the last column, never stored),
  // as offsets from the workgroup's first column
  const int ncols = min(N - n0, XG_BN);
  const uint32_t cl = static_cast<uint32_t>(min(col, N - 1) - n0);
  const __amdgpu_buffer_rsrc_t wr = buffer_of(W + static_cast<int64_t>(n0) * KW,
                                              static_cast<uint32_t>(ncols) * KW * 4u);
  const __amdgpu_buffer_rsrc_t sr = buffer_of(S + static_cast<int64_t>(n0) * G,
                                              static_cast<uint32_t>(ncols) * G * 4u);
  const uint32_t woff = cl * static_cast<uint32_t>(KW) * 4u, soff = cl * static_cast<uint32_t>(G) * 4u;
  auto w_at = [&](int g) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wr, woff, g * 16, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
  };
  auto s_at = [&](int g) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, soff, g * 4, 0));
  };

  f32x16 acc[MB], P[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      acc[i][v] = 0.0f;
      P[i][v] = 0.0f;  // folded with scale 0 before the first group
    }
  xg_copy<MB>(buf0, xr, 0, off, wave);
  const int g1 = min(1, G - 1);
  uint4 wa = w_at(0), wb = w_at(g1), wc;
  float sa = s_at(0), sb = s_at(g1), sc;
  __builtin_amdgcn_s_waitcnt(kWaitVmem0);  // this wave's copies have landed
  __syncthreads();
  float ps = 0.0f;
  // group g: X in buffer RB (X of g + 1 copied now into WB), weights of g + 2
  // loaded now into the slot freed by g - 1.  Two distinct LDS arrays (not
  // halves of one) let the compiler see that the group's LDS reads cannot
  // touch the copies in flight, so it does not wait for them; the loop is
  // unrolled six times so that both the buffers and the three weight slots
  // rotate without register copies (a copy of a just-loaded register made the
  // compiler wait for that load).  Before the barrier each wave waits for its
  // own copies, so after it the whole next tile is in LDS: the copies are
  // issued before the group's two weight and scale loads, so vmcnt(2) covers
  // them and leaves those two loads in flight across the barrier (they are
  // used two groups later; waiting for them here made every group wait a
  // full memory round trip).  tests/test_isa_order_cpu.py checks that order
  // on the compiled code.
#define PQ1_XG_STEP(RB, WB, WCUR, SCUR, WNEW, SNEW)                           \
  {                                                                           \
    const int gx = min(g + 1, G - 1), g2 = min(g + 2, G - 1);                 \
    xg_copy<MB>(WB, xr, gx * 256, off, wave);                                 \
    WNEW = w_at(g2);                                                          \
    SNEW = s_at(g2);                                                          \
    __builtin_amdgcn_sched_barrier(0); /* keep the loads ahead of the MFMAs */ \
    xg_group<MB, NAT>(RB, lr, h, hshift, sel0, sel1, WCUR, P, ps, acc);        \
    ps = SCUR;                                                                \
    __builtin_amdgcn_s_waitcnt(wait_vmem(2));                                 \
    __syncthreads();                                                          \
    if (++g >= G) break;                                                      \
  }
  for (int g = 0;;) {
    PQ1_XG_STEP(buf0, buf1, wa, sa, wc, sc)
    PQ1_XG_STEP(buf1, buf0, wb, sb, wa, sa)
    PQ1_XG_STEP(buf0, buf1, wc, sc, wb, sb)
    PQ1_XG_STEP(buf1, buf0, wa, sa, wc, sc)
    PQ1_XG_STEP(buf0, buf1, wb, sb, wa, sa)
    PQ1_XG_STEP(buf1, buf0, wc, sc, wb, sb)
  }
#undef PQ1_XG_STEP
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = fmaf(ps, P[i][v], acc[i][v]);
  if (col < N) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        if (row < M) Y[static_cast<int64_t>(row) * N + col] = acc[i][v];
      }
  }
}

// Workgroup b < n_full: tile b (row tile b / n_tiles_n, column tile
// b % n_tiles_n, so consecutive workgroups share X rows).  Workgroup
// n_full + 4 q + p: piece p (rows 32 p .. 32 p + 31) of tile n_full + q.
template <bool NAT>
__device__ __forceinline__ void xg_workgroup(const uint16_t* __restrict__ X,
                                             const uint32_t* __restrict__ W,
                                             const float* __restrict__ S, float* __restrict__ Y,
                                             int M, int N, int K, int n_tiles_n, int n_full,
                                             char* buf0, char* buf1) {
  const int b = blockIdx.x;
  if (b < n_full) {
    const int m0 = (b / n_tiles_n) * XG_BM, n0 = (b % n_tiles_n) * XG_BN;
    xg_tile<4, NAT>(X, W, S, Y, M, N, K, m0, n0, buf0, buf1);
  } else {
    const int q = b - n_full, tile = n_full + (q >> 2), p = q & 3;
    const int m0 = (tile / n_tiles_n) * XG_BM + 32 * p, n0 = (tile % n_tiles_n) * XG_BN;
    if (m0 >= M) return;  // a piece wholly past the last row (uniform per workgroup)
    xg_tile<1, NAT>(X, W, S, Y, M, N, K, m0, n0, buf0, buf1);
  }
}

#define PQ1_XG_KERNEL(NAME, NAT)                                                              \
  __global__ __launch_bounds__(XG_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))        \
  void NAME(const uint16_t* __restrict__ X, const uint32_t* __restrict__ W,                   \
            const float* __restrict__ S, float* __restrict__ Y, int M, int N, int K,           \
            int n_tiles_n, int n_full) {                                                      \
    __shared__ __attribute__((aligned(1024))) char buf0[XG_TILE];                              \
    __shared__ __attribute__((aligned(1024))) char buf1[XG_TILE];                              \
    xg_workgroup<NAT>(X, W, S, Y, M, N, K, n_tiles_n, n_full, buf0, buf1);                    \
  }
PQ1_XG_KERNEL(gemm_xg_kernel, false)      // X in the GEMM K order
PQ1_XG_KERNEL(gemm_xg_nat_kernel, true)   // X row-major, natural K order
#undef PQ1_XG_KERNEL

}  // namespace

hipError_t launch_gemm(const uint16_t* x_bf16, bool x_gemm_order, const uint32_t* w_bits,
                       const float* scales, float* y, int64_t M, int64_t N, int64_t K, int cus,
                       hipStream_t stream) {
  if (gemm_skinny_fits(M, K))
    return launch_gemm_skinny(x_bf16, x_gemm_order, w_bits, scales, y, M, N, K, cus, stream);
  const int64_t n_tiles_n = (N + XG_BN - 1) / XG_BN;
  const int64_t tiles = ((M + XG_BM - 1) / XG_BM) * n_tiles_n;
  const int64_t slots = 2 * static_cast<int64_t>(cus > 0 ? cus : 1);  // two workgroups per CU
  const int64_t rem = tiles % slots;
  const int64_t tail = (rem > 0 && 4 * rem <= slots) ? rem : 0;
  const int64_t n_full = tiles - tail;
  const dim3 grid(static_cast<unsigned>(n_full + 4 * tail));
  if (x_gemm_order)
    hipLaunchKernelGGL(gemm_xg_kernel, grid, dim3(XG_THREADS), 0, stream, x_bf16, w_bits,
                       scales, y, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K),
                       static_cast<int>(n_tiles_n), static_cast<int>(n_full));
  else
    hipLaunchKernelGGL(gemm_xg_nat_kernel, grid, dim3(XG_THREADS), 0, stream, x_bf16, w_bits,
                       scales, y, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K),
                       static_cast<int>(n_tiles_n), static_cast<int>(n_full));
  return hipGetLastError();
}

}  // namespace pq1
