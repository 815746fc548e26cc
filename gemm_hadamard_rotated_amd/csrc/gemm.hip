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
//  * gemm_skinny_kernel (M <= 24 and K <= 20480, either layout): 16 columns
//    per workgroup, K split over its waves, v_mfma_f32_16x16x32_bf16 (see
//    there).
// ---------------------------------------------------------------------------
#include <stdio.h>
#include <stdlib.h>

#include "pq1_internal.h"

namespace pq1 {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// B fragment dword: {w bit j, w bit j + 16} as bf16 +-1, where the per-lane
// pre-shifted word ws already accounts for the lane's half and `sh` =
// 11 - 8 (s & 1) - q.
__device__ __forceinline__ uint32_t sign_pair(uint32_t ws, int sh) {
  return ((ws << sh) & 0x80008000u) ^ 0xBF80BF80u;
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// B fragment of MFMA step s (0..7) of a group from the column's 4 words.
__device__ __forceinline__ bf16x8 b_fragment(const uint4& w, int s, int hshift) {
  const uint32_t ws = word_of(w, s >> 1) << hshift;
  const int sh = 11 - 8 * (s & 1);
  const u32x4 d = {sign_pair(ws, sh), sign_pair(ws, sh - 1), sign_pair(ws, sh - 2),
                   sign_pair(ws, sh - 3)};
  return __builtin_bit_cast(bf16x8, d);
}

// B fragment of MFMA step s (0..7) of a group in the natural K order: the
// lane's 8 weights are the 8 bits of byte 2 (s & 1) + h of word s / 2.  One
// byte permute puts that byte into both 16-bit halves (`sel` = the lane's
// selector for s even, odd), then per dword a packed 16-bit shift moves bit
// 2q to bit 15 of the low half and bit 2q + 1 to bit 15 of the high half (a
// different shift per half), and the same three-input bit operation as
// above makes {+-1, +-1}.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8 b_fragment_nat(const uint4& w, int s, uint32_t sel) {
  const uint32_t word = word_of(w, s >> 1);
  const u16x2 x = __builtin_bit_cast(u16x2, __builtin_amdgcn_perm(word, word, sel));
  uint32_t d[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u16x2 sh = {static_cast<unsigned short>(15 - 2 * q),
                      static_cast<unsigned short>(14 - 2 * q)};
    d[q] = (__builtin_bit_cast(uint32_t, x << sh) & 0x80008000u) ^ 0xBF80BF80u;
  }
  const u32x4 v = {d[0], d[1], d[2], d[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// ===========================================================================
// 128 x 128 tile, four 128 x 32 waves; X in the GEMM K order (NAT false) or
// row-major in the natural K order (NAT true).  In both layouts LDS chunk c
// of a row holds the 8 X values that MFMA step c / 2, lane half c % 2 reads;
// only the B fragment differs.
// ===========================================================================
constexpr int XG_BM = 128, XG_BN = 128, XG_WAVES = 4, XG_THREADS = 64 * XG_WAVES;
constexpr int XG_ROW = 256;                  // bytes per LDS row (128 bf16), swizzled
constexpr int XG_TILE = XG_BM * XG_ROW;      // one X buffer (32 KB)

// Buffer resource word 3 for raw 32-bit accesses (no swizzle, no index
// stride).  Buffer loads take a uniform base and range from the resource, a
// 32-bit per-lane offset and a uniform offset, so the per-group advance costs
// no vector registers and an out-of-range offset would read zero, not fault.
constexpr int kRawBufferWord3 = 0x00020000;
// s_waitcnt immediate: vector-memory count 0, the other counters unchecked.
constexpr int kWaitVmem0 = 0x0F70;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kRawBufferWord3);
}

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
  // own copies, so after it the whole next tile is in LDS.
#define PQ1_XG_STEP(RB, WB, WCUR, SCUR, WNEW, SNEW)                           \
  {                                                                           \
    const int gx = min(g + 1, G - 1), g2 = min(g + 2, G - 1);                 \
    xg_copy<MB>(WB, xr, gx * 256, off, wave);                                 \
    WNEW = w_at(g2);                                                          \
    SNEW = s_at(g2);                                                          \
    __builtin_amdgcn_sched_barrier(0); /* keep the loads ahead of the MFMAs */ \
    xg_group<MB, NAT>(RB, lr, h, hshift, sel0, sel1, WCUR, P, ps, acc);        \
    ps = SCUR;                                                                \
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);                                   \
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

// ===========================================================================
// Skinny M (M <= kSkinnyMaxM, K <= kSkinnyMaxK): one workgroup per 16
// columns, K split over its waves
// ===========================================================================
// With few rows of X the 128-row tiles leave the GPU to 136 long workgroup
// sequences (about 40 us for any M <= 128 at N = 17408), and the product is
// not a dense contraction: the time goes to streaming the 1-bit weights and
// expanding them, not to the matrix cores.  Here a workgroup owns 16 columns
// (1088 workgroups at N = 17408), so every weight is read and expanded once:
//  * its 16 weight rows and their scales are contiguous in memory; all of
//    them are copied into LDS at the start with buffer-to-LDS loads (16
//    bytes per lane, 1 KB per instruction, coalesced, one memory latency for
//    the whole workgroup -- reading 16-byte pieces of 16 rows per load
//    instead was 4-5 times slower);
//  * its KS waves take consecutive ranges of K groups; a wave computes up to
//    16 MB rows of X with v_mfma_f32_16x16x32_bf16 (MB = 1 for M <= 16, 2
//    above; more rows run as further row blocks side by side, workgroups
//    rb * C + c, so the blocks of a column land on one XCD), reading the
//    A fragments straight from X (small and cache-resident) PF groups ahead
//    into a ring of PF + 1 register slots (the loop is unrolled PF + 1 times,
//    so the slots rotate without copies);
//  * the KS partial blocks are added in wave order through LDS, so results
//    do not depend on timing.
//
// MFMA layout (v_mfma_f32_16x16x32_bf16, wave64): lane l holds
// A[l % 16][8 (l / 16) .. +7] and B[8 (l / 16) .. +7][l % 16]; the four output
// registers of lane l hold D[4 (l / 16) + v][l % 16].  Lane l thus reads the
// 16 bytes at element offset 32 s + 8 (l / 16) of each 32-wide K block s, in
// either X layout, and builds the matching weights of its column:
//  * GEMM order (stored position 8 h + 2 q + t holds element 4 h + q + 16 t,
//    h = l / 16): dword q is {bit 4 h + q, bit 4 h + q + 16} of word s, one
//    shift (by 15 - 4 h - q, a per-lane pre-shift plus a constant) and the
//    three-input bit operation, as in b_fragment;
//  * natural order: dword q is {bit 8 h + 2 q, bit 8 h + 2 q + 1}: byte h of
//    the word into both 16-bit halves by one byte permute, then per dword a
//    packed 16-bit shift and the same bit operation, as in b_fragment_nat.
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kSkinnyMaxK = 20480;  // 16 rows of weights + scales: 50 KB of LDS
constexpr int kSkinnyMaxM = 24;     // from 25 rows on the 128 x 128 tiles are faster

template <int MB>
struct SkX {
  bf16x8 a[MB][4];  // the group's four 32-wide K steps, per 16-row block
};

template <int MB>
__device__ __forceinline__ void sk_load(SkX<MB>& o, __amdgpu_buffer_rsrc_t xr,
                                        const uint32_t (&roff)[MB], int g) {
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      o.a[i][s] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(xr, roff[i], (g * 128 + 32 * s) * 2, 0));
}

// B fragment of step s from the column's words; `hs` = 12 - 4 h (GEMM
// order) and `sel` = byte h into both halves (natural order).
template <bool NAT>
__device__ __forceinline__ bf16x8 sk_b_fragment(const uint4& w, int s, uint32_t hs,
                                                uint32_t sel) {
  const uint32_t word = word_of(w, s);
  u32x4 d;
  if constexpr (NAT) {
    const u16x2 x = __builtin_bit_cast(u16x2, __builtin_amdgcn_perm(word, word, sel));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u16x2 sh = {static_cast<unsigned short>(15 - 2 * q),
                        static_cast<unsigned short>(14 - 2 * q)};
      d[q] = (__builtin_bit_cast(uint32_t, x << sh) & 0x80008000u) ^ 0xBF80BF80u;
    }
  } else {
    const uint32_t ws = word << hs;
#pragma unroll
    for (int q = 0; q < 4; ++q) d[q] = sign_pair(ws, 3 - q);
  }
  return __builtin_bit_cast(bf16x8, d);
}

// LDS bytes of a skinny workgroup: its 16 weight rows, then their scales,
// each rounded up to whole 1 KB copies.
__host__ __device__ constexpr uint32_t sk_round1k(uint32_t b) { return (b + 1023u) & ~1023u; }
__host__ __device__ constexpr uint32_t sk_w_bytes(int K) { return sk_round1k(16u * (K / 32) * 4u); }
__host__ __device__ constexpr uint32_t sk_s_bytes(int K) { return sk_round1k(16u * (K / 128) * 4u); }

template <int MB, int KS, int PF, bool NAT>
__global__ __launch_bounds__(64 * KS) void gemm_skinny_kernel(const uint16_t* __restrict__ X,
                                                               const uint32_t* __restrict__ W,
                                                               const float* __restrict__ S,
                                                               float* __restrict__ Y, int M,
                                                               int N, int K, int C) {
  static_assert(PF == 2 || PF == 3, "groups loaded ahead: 2 or 3");
  extern __shared__ __attribute__((aligned(1024))) char sk_lds[];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int h = lane >> 4, lr = lane & 15;
  const uint32_t hs = static_cast<uint32_t>(12 - 4 * h);
  const uint32_t sel = (0x0C000C00u | static_cast<uint32_t>(h)) | (static_cast<uint32_t>(h) << 16);
  const int c = blockIdx.x % C, rb = blockIdx.x / C;
  const int n0 = c * 16, r0 = rb * 16 * MB;
  const int col = n0 + lr;
  const int G = K / 128, KW = K / 32;
  const int gb = (G * wave) / KS, ge = (G * (wave + 1)) / KS;  // this wave's groups
  const uint32_t wbytes = sk_w_bytes(K), sbytes = sk_s_bytes(K);

  // X rows of this workgroup as offsets from row r0 (rows past M read the
  // last row: they only feed outputs that are never stored); the lane's K
  // position 8 h goes into the per-lane offset
  const __amdgpu_buffer_rsrc_t xr = buffer_of(
      X + static_cast<int64_t>(r0) * K, static_cast<uint32_t>(static_cast<int64_t>(M - r0) * K * 2));
  uint32_t roff[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
    roff[i] = static_cast<uint32_t>(min(r0 + 16 * i + lr, M - 1) - r0) * static_cast<uint32_t>(K) * 2u +
              16u * static_cast<uint32_t>(h);

  // the first X groups, then the workgroup's weight rows and scales into LDS
  // (rows past N: the buffers end at the last column, so those copies read
  // zeros; they feed outputs that are never stored)
  SkX<MB> o0, o1, o2, o3;
  if (gb < ge) {
    sk_load<MB>(o0, xr, roff, gb);
    sk_load<MB>(o1, xr, roff, min(gb + 1, ge - 1));
    if constexpr (PF == 3) sk_load<MB>(o2, xr, roff, min(gb + 2, ge - 1));
  }
  {
    const int ncols = min(N - n0, 16);
    const __amdgpu_buffer_rsrc_t wr = buffer_of(W + static_cast<int64_t>(n0) * KW,
                                                static_cast<uint32_t>(ncols) * KW * 4u);
    const __amdgpu_buffer_rsrc_t sr = buffer_of(S + static_cast<int64_t>(n0) * G,
                                                static_cast<uint32_t>(ncols) * G * 4u);
    const uint32_t lo = 16u * static_cast<uint32_t>(lane);
    for (uint32_t i = static_cast<uint32_t>(wave); i < wbytes / 1024u; i += KS)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void*)(sk_lds + 1024u * i), 16,
                                               1024u * i + lo, 0, 0, 0);
    for (uint32_t i = static_cast<uint32_t>(wave); i < sbytes / 1024u; i += KS)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_void*)(sk_lds + wbytes + 1024u * i), 16,
                                               1024u * i + lo, 0, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmem0);  // this wave's copies (and X groups) have landed
  __syncthreads();                          // ... and every other wave's
  const uint4* wl = reinterpret_cast<const uint4*>(sk_lds + static_cast<uint32_t>(lr) * KW * 4u);
  const float* sl = reinterpret_cast<const float*>(sk_lds + wbytes) + lr * G;

  const f32x4 zero = {};
  f32x4 acc[MB], P[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    acc[i] = zero;
    P[i] = zero;  // folded with scale 0 before the first group
  }
  float ps = 0.0f;
  if (gb < ge) {
    // Straight-line rounds of PF + 1 groups: a group past the wave's range
    // (the last round's tail) re-reads the last group and is folded in with
    // scale 0, so the loop body has no exits and the compiler can count the
    // loads in flight exactly.
    // group g + J: X in CUR; X of g + J + PF is loaded now into NEW (the slot
    // group g + J - 1 used); the column's words and scale come from LDS
#define PQ1_SK_STEP(J, CUR, NEW)                                                        \
    {                                                                                   \
      sk_load<MB>(NEW, xr, roff, min(g + (J) + PF, ge - 1));                            \
      __builtin_amdgcn_sched_barrier(0); /* keep the loads ahead of the MFMAs */       \
      const int gj = min(g + (J), ge - 1);                                              \
      const uint4 w = wl[gj];                                                           \
      _Pragma("unroll") for (int s = 0; s < 4; ++s) {                                   \
        const bf16x8 b = sk_b_fragment<NAT>(w, s, hs, sel);                             \
        _Pragma("unroll") for (int i = 0; i < MB; ++i) {                                \
          if (s == 0) acc[i] += ps * P[i];                                              \
          P[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(CUR.a[i][s], b, s == 0 ? zero : P[i], 0, 0, 0); \
        }                                                                               \
      }                                                                                 \
      ps = g + (J) < ge ? sl[gj] : 0.0f;                                                \
    }
    if constexpr (PF == 3) {
      for (int g = gb; g < ge; g += 4) {
        PQ1_SK_STEP(0, o0, o3)
        PQ1_SK_STEP(1, o1, o0)
        PQ1_SK_STEP(2, o2, o1)
        PQ1_SK_STEP(3, o3, o2)
      }
    } else {
      for (int g = gb; g < ge; g += 3) {
        PQ1_SK_STEP(0, o0, o2)
        PQ1_SK_STEP(1, o1, o0)
        PQ1_SK_STEP(2, o2, o1)
      }
    }
#undef PQ1_SK_STEP
  }
#pragma unroll
  for (int i = 0; i < MB; ++i) acc[i] += ps * P[i];
  // add the KS partial blocks in wave order (the LDS of the weight copies is
  // free again once every wave is past its loop)
  if constexpr (KS > 1) {
    f32x4* red = reinterpret_cast<f32x4*>(sk_lds);
    __syncthreads();
    if (wave > 0) {
#pragma unroll
      for (int i = 0; i < MB; ++i) red[((wave - 1) * MB + i) * 64 + lane] = acc[i];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int q = 0; q < KS - 1; ++q) acc[i] += red[(q * MB + i) * 64 + lane];
  }
  if (col >= N) return;
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = r0 + 16 * i + 4 * h + v;
      if (row < M) Y[static_cast<int64_t>(row) * N + col] = acc[i][v];
    }
}

struct SkinnyPlan {
  int mb, ks, pf;  // 16-row blocks per wave, waves per workgroup, groups loaded ahead
};

// Tuning override for experiments: PQ1_SKINNY_PLAN="mb,ks,pf", one of the
// instantiated plans (1,2,3 / 2,2,3 / 1,4,2 / 2,1,3; anything else is
// ignored), read once per process.  A plan with mb = 1 still covers any M up
// to kSkinnyMaxM (more row blocks).
void skinny_override(SkinnyPlan* p) {
  static const SkinnyPlan ov = [] {
    SkinnyPlan q{0, 0, 0};
    const char* e = getenv("PQ1_SKINNY_PLAN");
    if (e && sscanf(e, "%d,%d,%d", &q.mb, &q.ks, &q.pf) == 3) {
      const int known[][3] = {{1, 2, 3}, {2, 2, 3}, {1, 4, 2}, {2, 1, 3}};
      for (const auto& k : known)
        if (q.mb == k[0] && q.ks == k[1] && q.pf == k[2]) return q;
    }
    return SkinnyPlan{0, 0, 0};
  }();
  if (ov.mb > 0) *p = ov;
}

}  // namespace

hipError_t launch_gemm(const uint16_t* x_bf16, bool x_gemm_order, const uint32_t* w_bits,
                       const float* scales, float* y, int64_t M, int64_t N, int64_t K, int cus,
                       hipStream_t stream) {
  // Short prompts: the skinny kernel up to 24 rows (measured at N = 17408, K
  // = 5120, graph replay, cold weights: M = 1 11.2 us, 8 18.8, 16 27.2, 17
  // 33.4; the 128 x 128 tiles take 41 us for any M <= 128, the skinny kernel
  // 48 us at M = 32, so from 25 rows on the tiles are faster)
  if (M <= kSkinnyMaxM && K <= kSkinnyMaxK) {
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    const int C = static_cast<int>((N + 15) / 16);
    SkinnyPlan pl = M <= 16 ? SkinnyPlan{1, 2, 3} : SkinnyPlan{2, 2, 3};
    skinny_override(&pl);
    const int rows = 16 * pl.mb;
    const dim3 grid(static_cast<unsigned>(C * ((M + rows - 1) / rows)));
    // weights + scales; the final reduction reuses the same bytes (at least
    // as many as it needs)
    const size_t lds = sk_w_bytes(k) + sk_s_bytes(k);
#define PQ1_SK_CASE(MB_, KS_, PF_)                                                            \
    if (pl.mb == MB_ && pl.ks == KS_ && pl.pf == PF_) {                                       \
      const size_t red = static_cast<size_t>(KS_ - 1) * MB_ * 64 * 16;                        \
      const size_t bytes = lds > red ? lds : red;                                             \
      if (x_gemm_order)                                                                       \
        hipLaunchKernelGGL((gemm_skinny_kernel<MB_, KS_, PF_, false>), grid, dim3(64 * KS_),  \
                           bytes, stream, x_bf16, w_bits, scales, y, m, n, k, C);             \
      else                                                                                    \
        hipLaunchKernelGGL((gemm_skinny_kernel<MB_, KS_, PF_, true>), grid, dim3(64 * KS_),   \
                           bytes, stream, x_bf16, w_bits, scales, y, m, n, k, C);             \
      return hipGetLastError();                                                               \
    }
    PQ1_SK_CASE(1, 2, 3)
    PQ1_SK_CASE(2, 2, 3)
    PQ1_SK_CASE(1, 4, 2)
    PQ1_SK_CASE(2, 1, 3)
#undef PQ1_SK_CASE
    return hipErrorInvalidValue;
  }
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
