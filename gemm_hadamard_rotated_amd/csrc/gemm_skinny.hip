// Short-prompt prefill GEMM (few rows of X): see the comment of
// gemm_skinny_kernel.  gemm.hip's launcher sends a call here when
// gemm_skinny_fits(M, K).
#include <stdio.h>
#include <stdlib.h>

#include "gemm_common.h"
#include "pq1_internal.h"

namespace pq1 {

namespace {

using namespace gemm_detail;

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
constexpr int kSkinnyMaxM = 20;     // from about 21 rows on the 128 x 128 tiles are faster

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

bool gemm_skinny_fits(int64_t M, int64_t K) { return M <= kSkinnyMaxM && K <= kSkinnyMaxK; }

hipError_t launch_gemm_skinny(const uint16_t* x_bf16, bool x_gemm_order, const uint32_t* w_bits,
                              const float* scales, float* y, int64_t M, int64_t N, int64_t K,
                              hipStream_t stream) {
  // Short prompts: the skinny kernel up to 20 rows (measured at N = 17408, K
  // = 5120, graph replay, cold weights: M = 1 10.6 us, 8 18.3, 16 26.8, 17
  // 33.4, 24 42.4; the 128 x 128 tiles take 40-41 us for any M <= 128)
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

}  // namespace pq1
