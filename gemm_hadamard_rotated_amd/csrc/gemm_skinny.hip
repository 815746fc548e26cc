// Short-prompt prefill GEMM (few rows of X): see the comment of
// gemm_skinny_kernel.  gemm.hip's launcher sends a call here when
// gemm_skinny_fits(M, K).
#include <stdio.h>
#include <stdlib.h>

#include <type_traits>

#include "gemm_common.h"
#include "pq1_internal.h"

namespace pq1 {

namespace {

using namespace gemm_detail;

// ===========================================================================
// Skinny M (M <= kSkinnyMaxM): a workgroup per 16 NCB columns, K split over
// its waves, each wave's weights copied into LDS in one burst
// ===========================================================================
// With few rows of X the 128-row tiles leave the GPU to 136 long workgroup
// sequences (about 40 us for any M <= 128 at N = 17408), and the product is
// not a dense contraction: the time goes to streaming and expanding the
// 1-bit weights (each is used by one MFMA per 16 rows of X), not to the
// matrix cores.  Here:
//  * a workgroup owns NCB blocks of 16 columns; its KS waves take
//    consecutive ranges of K groups and a wave computes MB blocks of 16 rows
//    of X against all NCB column blocks with v_mfma_f32_16x16x32_bf16, so
//    every A fragment of X serves NCB MFMAs and every expanded weight
//    fragment MB of them;
//  * a wave first copies the weight words and scales of its own groups, for
//    all 16 NCB rows, into its own LDS region with buffer-to-LDS loads (one
//    burst: the whole weight stream is requested at the start, which is what
//    keeps enough bytes in flight for HBM; loading the few bytes each step
//    needs a few groups ahead kept a tenth of that in flight and ran at a
//    fraction of the bandwidth), then waits for its own copies only (no
//    barrier: no wave waits for another's);
//  * the A fragments come straight from X (small and cache-resident) PF
//    groups ahead into a ring of PF + 1 register slots, each group's words
//    are read from LDS one group ahead and its scales during its own step
//    (the loop is unrolled PF + 1 times, so the slots rotate without copies;
//    a range that is not a whole number of rounds ends in single steps);
//  * the fold acc += scale * P of a group waits one step: the first MFMAs of
//    the next group go out before it, so it does not wait for its own chain;
//  * with 16 rows per wave the workgroup has 8 waves, two per SIMD: within
//    one wave an MFMA and the vector instructions around it take turns, but
//    the other wave's vector work runs while it computes; with 32-64 rows
//    per wave (two to four times the MFMAs and A fragments) 4 waves measured
//    faster (48 and 64 rows need more than 256 VGPRs: the compiler keeps the
//    rest in AGPRs, which a single wave per SIMD has to spare);
//  * the KS partial blocks go through LDS after one barrier and block q is
//    summed in wave order and stored by wave q % KS, so results do not
//    depend on timing and no single wave does all the sums and stores.
//
// MFMA layout (wave64): lane l (h = l / 16, c = l % 16) holds
// A[c][8 h .. 8 h + 7] and B[8 h .. 8 h + 7][c]; its four outputs are
// D[4 h + v][c].  The 32 K positions of MFMA step s (0..3) of a group are
// taken so that lane h uses word h of its column's group (bits 32 h .. 32 h
// + 31 of the 128) and only bits chosen by s; which 8 of them depends on the
// X layout, and either way the lane's 16 bytes of X sit at stored elements
// 32 h + 8 s .. + 7 of the group:
//  * GEMM order (stored position 8 t' + 2 q + u of a 32-element block holds
//    element 4 t' + q + 16 u of that block): the 8 values are elements
//    4 s + q + 16 u of block h, i.e. bits {4 s + q, 4 s + q + 16} of word h
//    for dword q: one shift by 15 - 4 s - q (the same for all lanes) and the
//    three-input bit operation of sign_pair;
//  * natural order: the 8 values are elements 8 s .. 8 s + 7 of block h,
//    i.e. byte s of word h: one byte permute puts it into both 16-bit halves,
//    then per dword a packed 16-bit shift and the same bit operation.
// Every step covers 32 distinct K of the group and the four steps all 128,
// so a group's four MFMAs sum exactly the group's products.
//
// LDS: wave w's region starts at 20 * NC * gb bytes (gb = its first group)
// and holds its NC x Gw weight groups (16 bytes each, row-major: row r,
// group j at 16 (r Gw + j)), then their scales (4 bytes, same order).
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kSkinnyMaxM = 64;  // above 64 rows the 128 x 128 tiles are faster
constexpr uint32_t kSkinnyMaxLds = 64u * 1024u;

// waves whose partial blocks the final pass of the reduction adds: all KS
// where their blocks fit the LDS limit, else half of them
constexpr int skinny_red_waves(int mb, int ncb, int ks) {
  return static_cast<uint32_t>(ks * mb * ncb) * 1024u <= kSkinnyMaxLds ? ks : ks / 2;
}

template <int MB>
struct SkX {
  bf16x8 a[MB][4];  // X: the group's four steps, per 16-row block
};

template <int MB>
__device__ __forceinline__ void sk_load(SkX<MB>& o, __amdgpu_buffer_rsrc_t xr,
                                        const uint32_t (&xoff)[MB], int g) {
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      o.a[i][s] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[i], g * 256 + 16 * s, 0));
}

// B fragment of step s from the lane's weight word (see the layout above).
template <bool NAT>
__device__ __forceinline__ bf16x8 sk_b_fragment(uint32_t word, int s) {
  u32x4 d;
  if constexpr (NAT) {
    const uint32_t sel = 0x0C000C00u | static_cast<uint32_t>(s) | (static_cast<uint32_t>(s) << 16);
    const u16x2 x = __builtin_bit_cast(u16x2, __builtin_amdgcn_perm(word, word, sel));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u16x2 sh = {static_cast<unsigned short>(15 - 2 * q),
                        static_cast<unsigned short>(14 - 2 * q)};
      d[q] = (__builtin_bit_cast(uint32_t, x << sh) & 0x80008000u) ^ 0xBF80BF80u;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) d[q] = sign_pair(word, 15 - 4 * s - q);
  }
  return __builtin_bit_cast(bf16x8, d);
}

// steps J0 .. J1 - 1 of a round starting at group g (the first `count` of
// them when count is given: a uniform branch per step)
template <int J0, int J1, class F>
__device__ __forceinline__ void sk_steps(F& step, int g) {
  if constexpr (J0 < J1) {
    step(std::integral_constant<int, J0>{}, g + J0);
    sk_steps<J0 + 1, J1>(step, g);
  }
}
template <int J0, int J1, class F>
__device__ __forceinline__ void sk_steps(F& step, int g, int count) {
  if constexpr (J0 < J1) {
    if (J0 < count) step(std::integral_constant<int, J0>{}, g + J0);
    sk_steps<J0 + 1, J1>(step, g, count);
  }
}

template <int MB, int NCB, int KS, int PF, bool NAT>
__global__ __launch_bounds__(64 * KS) void gemm_skinny_kernel(const uint16_t* __restrict__ X,
                                                               const uint32_t* __restrict__ W,
                                                               const float* __restrict__ S,
                                                               float* __restrict__ Y, int M,
                                                               int N, int K, int C) {
  static_assert(PF == 1 || PF == 3, "groups of X loaded ahead: 1 or 3");
  static_assert(KS > 1, "the partial blocks are added through LDS");
  constexpr int NC = 16 * NCB;  // columns of the workgroup
  extern __shared__ __attribute__((aligned(16))) char sk_lds[];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int h = lane >> 4, lc = lane & 15;
  const int c = blockIdx.x % C, rb = blockIdx.x / C;
  const int n0 = c * NC, r0 = rb * 16 * MB;
  const int G = K / 128;
  const int gb = (G * wave) / KS, ge = (G * (wave + 1)) / KS;  // this wave's groups
  const int Gw = ge - gb;

  // X rows r0 .. M - 1 (rows past M read the last row: they only feed
  // outputs that are never stored); the lane's K position 32 h goes into its
  // per-lane offset, the group into the uniform offset
  const __amdgpu_buffer_rsrc_t xr = buffer_of(
      X + static_cast<int64_t>(r0) * K, static_cast<uint32_t>(static_cast<int64_t>(M - r0) * K * 2));
  uint32_t xoff[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
    xoff[i] = static_cast<uint32_t>(min(r0 + 16 * i + lc, M - 1) - r0) * static_cast<uint32_t>(K) * 2u +
              64u * static_cast<uint32_t>(h);

  // this wave's weight groups and scales of the workgroup's rows into its
  // LDS region (rows past N lie past the buffers' ends and read zeros; they
  // feed outputs that are never stored)
  char* const wreg = sk_lds + 20u * NC * static_cast<uint32_t>(gb);
  char* const sreg = wreg + 16u * NC * static_cast<uint32_t>(Gw);
  {
    const int ncols = min(N - n0, NC);
    const __amdgpu_buffer_rsrc_t wr = buffer_of(W + static_cast<int64_t>(n0) * (K / 32),
                                                static_cast<uint32_t>(ncols) * (K / 8));
    const __amdgpu_buffer_rsrc_t sr = buffer_of(S + static_cast<int64_t>(n0) * G,
                                                static_cast<uint32_t>(ncols) * G * 4u);
    const uint32_t units = static_cast<uint32_t>(NC * Gw);  // (row, group) pairs
    for (uint32_t i = 0; i < units; i += 64) {
      const uint32_t p = i + static_cast<uint32_t>(lane);
      const uint32_t row = p / static_cast<uint32_t>(Gw), j = p - row * static_cast<uint32_t>(Gw);
      if (p < units)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wr, (lds_void*)(wreg + 16u * i), 16,
            row * static_cast<uint32_t>(K / 8) + 16u * (static_cast<uint32_t>(gb) + j), 0, 0, 0);
    }
    for (uint32_t i = 0; i < units; i += 64) {
      const uint32_t p = i + static_cast<uint32_t>(lane);
      const uint32_t row = p / static_cast<uint32_t>(Gw), j = p - row * static_cast<uint32_t>(Gw);
      if (p < units)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            sr, (lds_void*)(sreg + 4u * i), 4,
            4u * (row * static_cast<uint32_t>(G) + static_cast<uint32_t>(gb) + j), 0, 0, 0);
    }
  }

  const f32x4 zero = {};
  f32x4 acc[MB][NCB];
  f32x4 P[2][MB][NCB];  // the chains of consecutive groups, by step parity
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NCB; ++j) {
      acc[i][j] = zero;
      P[0][i][j] = zero;
      P[1][i][j] = zero;
    }

  if (Gw > 0) {
    SkX<MB> o[PF + 1];
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      sk_load<MB>(o[p], xr, xoff, min(gb + p, ge - 1));
      // in group order: the loop's waits count on the oldest group landing first
      __builtin_amdgcn_sched_barrier(0);
    }
    // wait for the copies (and the X groups behind them): a count that
    // leaves the X loads outstanding would rely on them being issued after
    // the copies, and the compiler sinks them into the loop's preheader,
    // below this wait (a count of 4 MB PF then let copies still be in flight
    // when the LDS reads began)
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);
    __builtin_amdgcn_sched_barrier(0);
    // lane's word h and scale of row 16 j + lc, group jj of the range
    const uint32_t* wl = reinterpret_cast<const uint32_t*>(wreg) + static_cast<uint32_t>(lc * Gw) * 4u + h;
    const float* sl = reinterpret_cast<const float*>(sreg) + lc * Gw;
    const int wstride = 16 * Gw * 4, sstride = 16 * Gw;  // one column block further
    uint32_t w[2][NCB];
    float sc[2][NCB];  // scales of the groups of the last two steps, by parity
#pragma unroll
    for (int j = 0; j < NCB; ++j) {
      w[0][j] = wl[j * wstride];
      sc[1][j] = 0.0f;  // the first step folds an empty chain
    }
    // Step J of a round of PF + 1 groups (an even count, so step J always
    // has the parity of J): group g (X from slot J, words read during the
    // step before), the load of X of group g + PF into slot (J + PF) %
    // (PF + 1), the LDS reads of the words of group g + 1 (clamped to the
    // range) and of the scales of group g, and the group before folded after
    // this group's first MFMAs (so the fold does not wait for its own chain;
    // chains and scales of consecutive groups alternate between parities 0
    // and 1, so nothing is copied between steps).
    auto step = [&](auto jc, int g) {
      constexpr int J = decltype(jc)::value;
      constexpr int b = J & 1;
      sk_load<MB>(o[(J + PF) % (PF + 1)], xr, xoff, min(g + PF, ge - 1));
      {
        const int jn = min(g + 1, ge - 1) - gb;
#pragma unroll
        for (int j = 0; j < NCB; ++j) {
          w[b ^ 1][j] = wl[j * wstride + 4 * jn];
          sc[b][j] = sl[j * sstride + g - gb];
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the MFMAs
      const SkX<MB>& cur = o[J];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int j = 0; j < NCB; ++j) {
          const bf16x8 bf = sk_b_fragment<NAT>(w[b][j], s);
#pragma unroll
          for (int i = 0; i < MB; ++i)
            P[b][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.a[i][s], bf,
                                                                 s == 0 ? zero : P[b][i][j], 0, 0, 0);
        }
        if (s == 0) {
#pragma unroll
          for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NCB; ++j) acc[i][j] += sc[b ^ 1][j] * P[b ^ 1][i][j];
        }
      }
    };
    // Straight-line rounds while a whole round is left (no exits inside, so
    // the compiler counts the loads in flight exactly), then the remaining
    // groups one step each; no step runs on a group past the range.
    const int rounds = Gw / (PF + 1), rest = Gw - rounds * (PF + 1);
    int g = gb;
    for (int r = 0; r < rounds; ++r, g += PF + 1) sk_steps<0, PF + 1>(step, g);
    sk_steps<0, PF>(step, g, rest);
    // fold the last group, whose chain has the parity of the last step taken
    if (((rest > 0 ? rest - 1 : PF) & 1) == 0) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NCB; ++j) acc[i][j] += sc[0][j] * P[0][i][j];
    } else {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NCB; ++j) acc[i][j] += sc[1][j] * P[1][i][j];
    }
  }

  // Every wave puts its partial blocks into LDS (the weight regions are free
  // once every wave is past its loop); then block q is summed in wave order
  // and stored by wave q % KS, so results do not depend on timing and the
  // sums and stores are spread over the waves.  Where KS waves' blocks
  // would not fit the LDS limit, waves KS/2 .. KS-1 first hand theirs to
  // waves 0 .. KS/2-1, which add them and then go on as above.
  constexpr int RW = skinny_red_waves(MB, NCB, KS);
  f32x4* red = reinterpret_cast<f32x4*>(sk_lds);  // [RW][MB * NCB][64 lanes]
  __syncthreads();
  if constexpr (RW < KS) {
    if (wave >= RW) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NCB; ++j) red[(((wave - RW) * MB + i) * NCB + j) * 64 + lane] = acc[i][j];
    }
    __syncthreads();
    if (wave < RW) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NCB; ++j) acc[i][j] += red[((wave * MB + i) * NCB + j) * 64 + lane];
    }
    __syncthreads();
  }
  if (wave < RW) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NCB; ++j) red[((wave * MB + i) * NCB + j) * 64 + lane] = acc[i][j];
  }
  __syncthreads();
  for (int q = wave; q < MB * NCB; q += KS) {
    const int i = q / NCB, j = q - i * NCB;
    f32x4 sum = red[q * 64 + lane];
#pragma unroll
    for (int w = 1; w < RW; ++w) sum += red[(w * MB * NCB + q) * 64 + lane];
    const int col = n0 + 16 * j + lc;
    if (col >= N) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = r0 + 16 * i + 4 * h + v;
      if (row < M) Y[static_cast<int64_t>(row) * N + col] = sum[v];
    }
  }
}

struct SkinnyPlan {
  int mb, ncb, ks, pf;  // 16-row blocks per wave, 16-column blocks, waves per workgroup, X groups ahead
};

// Tuning override for experiments: PQ1_SKINNY_PLAN="mb,ncb,ks,pf", one of
// the instantiated plans (anything else is ignored), read once per process.
// A plan covers any M up to kSkinnyMaxM (more row blocks).
#define PQ1_SK_PLANS(X_)                                                                 \
  X_(1, 1, 4, 1) X_(1, 2, 4, 1) X_(1, 4, 4, 1) X_(1, 5, 4, 1) X_(2, 1, 4, 1) X_(2, 2, 4, 1) \
  X_(2, 4, 4, 1) X_(2, 5, 4, 1) X_(1, 1, 8, 1) X_(1, 2, 8, 1) X_(1, 4, 8, 1) X_(1, 5, 8, 1) \
  X_(3, 1, 4, 1) X_(3, 2, 4, 1) X_(3, 4, 4, 1) X_(3, 5, 4, 1) X_(4, 1, 4, 1) X_(4, 2, 4, 1) \
  X_(4, 4, 4, 1) X_(4, 5, 4, 1)
void skinny_override(SkinnyPlan* p) {
  static const SkinnyPlan ov = [] {
    SkinnyPlan q{0, 0, 0, 0};
    const char* e = getenv("PQ1_SKINNY_PLAN");
    if (e && sscanf(e, "%d,%d,%d,%d", &q.mb, &q.ncb, &q.ks, &q.pf) == 4) {
#define PQ1_SK_KNOWN(A, B, C_, D) \
  if (q.mb == A && q.ncb == B && q.ks == C_ && q.pf == D) return q;
      PQ1_SK_PLANS(PQ1_SK_KNOWN)
#undef PQ1_SK_KNOWN
    }
    return SkinnyPlan{0, 0, 0, 0};
  }();
  if (ov.mb > 0) *p = ov;
}

// dynamic LDS of a launch: the weight regions, or the reduction if larger
size_t skinny_lds(const SkinnyPlan& pl, int64_t K) {
  const size_t weights = static_cast<size_t>(20 * 16 * pl.ncb) * static_cast<size_t>(K / 128);
  const size_t red = static_cast<size_t>(skinny_red_waves(pl.mb, pl.ncb, pl.ks)) * pl.mb * pl.ncb * 64 * 16;
  return weights > red ? weights : red;
}

// 16-row blocks per wave for M rows: one wave covers all the rows (one row
// block up to 16 rows, two up to 32, three up to 48, four up to 64)
int skinny_row_blocks(int64_t M) { return static_cast<int>((M + 15) / 16); }

// The plan for an M x K activation block against N weight rows on `cus`
// CUs: 16 rows per wave (8 waves) up to M = 16, else all M rows rounded up
// to 16 in each of 4 waves; then the number of column blocks per workgroup
// (5, 4 or 2, as the LDS limit allows; 1 if none fits) that puts the fewest
// column blocks on the busiest CU, the workgroups being spread evenly (ties
// to more blocks, which reuse each A fragment more).  A workgroup's waves
// all run for its whole column range, so a CU with one workgroup more than
// the others sets the time: at N = 17408 (1088 blocks) five blocks give 218
// workgroups, one per CU, where four gave 272 and left 16 CUs with two.
// Measured there (K = 5120, graph replay, cold weights, row-major X, us):
// M = 1 9.8, 8 10.2, 16 10.5, 24 13.0, 32 15.0, 33 16.7, 48 20.5, 49 22.6,
// 64 26.1 (four blocks and 4 waves, 32 rows per wave: 13.5, 13.9, 15.5,
// 22.3, 26.2, -, 29.2, -, 36.3; as sets of 32-row waves: 33 22.6, 48 24.4,
// 49 24.4, 64 26.9).
SkinnyPlan skinny_plan(int64_t M, int64_t N, int64_t K, int cus) {
  const int mb = skinny_row_blocks(M);
  const int ks = mb == 1 ? 8 : 4;
  const int64_t row_blocks = (M + 16 * mb - 1) / (16 * mb);
  const int64_t col_blocks = (N + 15) / 16;
  const int64_t slots = cus > 0 ? cus : 1;
  SkinnyPlan best{mb, 1, ks, 1};
  int64_t best_cost = -1;
  for (const int ncb : {5, 4, 2}) {
    const SkinnyPlan p{mb, ncb, ks, 1};
    if (skinny_lds(p, K) > kSkinnyMaxLds) continue;
    const int64_t wgs = (col_blocks + ncb - 1) / ncb * row_blocks;
    const int64_t cost = (wgs + slots - 1) / slots * ncb;  // column blocks on the busiest CU
    if (best_cost < 0 || cost < best_cost) {
      best = p;
      best_cost = cost;
    }
  }
  skinny_override(&best);
  return best;
}

}  // namespace

bool gemm_skinny_fits(int64_t M, int64_t K) {
  // one column block per workgroup is the plan with the least LDS
  const int mb = skinny_row_blocks(M);
  return M <= kSkinnyMaxM && skinny_lds(SkinnyPlan{mb, 1, mb == 1 ? 8 : 4, 1}, K) <= kSkinnyMaxLds;
}

hipError_t launch_gemm_skinny(const uint16_t* x_bf16, bool x_gemm_order, const uint32_t* w_bits,
                              const float* scales, float* y, int64_t M, int64_t N, int64_t K,
                              int cus, hipStream_t stream) {
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
  const SkinnyPlan pl = skinny_plan(M, N, K, cus);
  const size_t lds = skinny_lds(pl, K);
  if (lds > kSkinnyMaxLds) return hipErrorInvalidValue;
  const int rows = 16 * pl.mb, cols = 16 * pl.ncb;
  const int C = static_cast<int>((N + cols - 1) / cols);
  const dim3 grid(static_cast<unsigned>(C * ((M + rows - 1) / rows)));
#define PQ1_SK_CASE(MB_, NCB_, KS_, PF_)                                                      \
  if (pl.mb == MB_ && pl.ncb == NCB_ && pl.ks == KS_ && pl.pf == PF_) {                     \
    if (x_gemm_order)                                                                       \
      hipLaunchKernelGGL((gemm_skinny_kernel<MB_, NCB_, KS_, PF_, false>), grid,            \
                         dim3(64 * KS_), lds, stream, x_bf16, w_bits, scales, y, m, n, k, C); \
    else                                                                                    \
      hipLaunchKernelGGL((gemm_skinny_kernel<MB_, NCB_, KS_, PF_, true>), grid,             \
                         dim3(64 * KS_), lds, stream, x_bf16, w_bits, scales, y, m, n, k, C); \
    return hipGetLastError();                                                               \
  }
  PQ1_SK_PLANS(PQ1_SK_CASE)
#undef PQ1_SK_CASE
  return hipErrorInvalidValue;
}

}  // namespace pq1
