// Decode GEMV kernels: y[n] = sum_k scale[n][k>>7] * (+-1)(n, k) * x_rot[k].
//
// Weight format ("Inside the One-Bit Engine", station "A weight is one bit"):
// bit (k & 31) of word (k >> 5) of row n; set = +1, clear = -1; one fp32 scale
// per 128 weights along K.
//
// Two algorithms, both split over K so that a 5120-row matrix still fills the
// 256 compute units:
//
//  LUT (default).  "Inside the One-Bit Engine", station "Four one-bit weights
//  have only sixteen possible answers": four +-1 weights against four inputs
//  can only produce 16 values.  Each workgroup tabulates, for every run of 4
//  inputs of its K-tile, the 16 signed sums +-x0 +-x1 +-x2 +-x3 in LDS (entry
//  e has +x_i where bit i of e is set), and every lane -- one lane per output
//  row -- adds one table entry per 4 weights, indexed by the nibble of its
//  weight word.  All 64 lanes of a wave read the same 16-entry table at the
//  same time, so the reads are free of bank conflicts.  The nibble-to-address
//  step costs one bit-field extract per 4 weights plus 4 ops per 32 weights;
//  with the add this is ~0.63 VALU ops per weight.  The table stores signed
//  sums directly, so no "2S - T" correction is needed.  The per-group sum is
//  multiplied by its fp32 scale once per 128 weights.
//
//  EXPAND.  Eight lanes share a row, each owning one 128-weight group of the
//  K-tile and keeping its 128 inputs in registers; each bit is expanded into a
//  select mask (masked sum S of the inputs whose bit is set, result 2S - T
//  with T the group's input sum), the group partial is multiplied by its
//  scale, and the eight partials of a row are reduced across lanes with
//  shuffles.  About 3 VALU ops per weight.
//
// Split-K: a workgroup handles `rb` rows x one K-tile.  With more than one
// K-tile, each workgroup writes its partial sums to the workspace and bumps
// the row block's arrival counter; the last workgroup to arrive adds the
// partials of all K-tiles in K order (so results do not depend on arrival
// order), stores y, and resets the counter to zero for the next call.  The
// counters sit in a fixed region at the start of the workspace, so any call
// finds them zero whatever shapes earlier calls had.
#include <algorithm>

#include "gemv_common.h"
#include "pq1.h"
#include "pq1_device.h"

namespace pq1 {

namespace {

// Per-lane weights and scales of one K-tile (one uint4 and one scale per
// 128-weight group).
template <int KT>
struct TileRegs {
  static constexpr int G = KT / kGroup;
  uint4 w[G];
  float s[G];
};

// Issue the tile's loads.  Every load is unconditional (groups past the end
// of a short last tile re-read its last group, invalid rows read row 0) so the
// compiler can wait for each group's data separately; scales go first because
// the first group's FMA needs its scale.
template <int KT, bool SCALE4>
__device__ __forceinline__ void load_tile(TileRegs<KT>& tr, const uint32_t* __restrict__ wrow,
                                          const float* __restrict__ srow, int klen) {
  constexpr int G = KT / kGroup;
  const int glast = klen / kGroup - 1;
  if constexpr (SCALE4 && G >= 4) {
    // K % 512 == 0 and KT % 512 == 0: 16-byte aligned scale quadruples, and a
    // tile covers whole quadruples
#pragma unroll
    for (int g = 0; g < G; g += 4) {
      const float4 s4 = *reinterpret_cast<const float4*>(srow + min(g, glast - 3));
      tr.s[g] = s4.x;
      tr.s[g + 1] = s4.y;
      tr.s[g + 2] = s4.z;
      tr.s[g + 3] = s4.w;
    }
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g) tr.s[g] = srow[min(g, glast)];
  }
#pragma unroll
  for (int g = 0; g < G; ++g) tr.w[g] = reinterpret_cast<const uint4*>(wrow)[min(g, glast)];
}

// Sum of scale * (table lookups) over the tile; the table must be complete.
// FULL: the tile is whole (K % KT == 0), so every group is walked with no
// condition -- a per-group condition let the compiler sink that group's
// weight load into it, behind the barrier that publishes the tables.
template <int KT, bool FULL>
__device__ __forceinline__ float lut_tile(const TileRegs<KT>& tr, int klen,
                                          const char* __restrict__ lut, uint32_t nib_mask) {
  float acc = 0.0f;
#pragma unroll
  for (int g = 0; g < TileRegs<KT>::G; ++g) {
    if (FULL || g * kGroup < klen)
      acc = fmaf(tr.s[g], lut_group<kPadTableBytes>(lut, g * 32 * kPadTableBytes, tr.w[g], nib_mask),
                 acc);
  }
  return acc;
}

template <int RB, int KT, bool SCALE4, bool FULL>
__global__ __launch_bounds__(RB) void gemv_lut_kernel(int N, int K, int nkt, int nrb,
                                                      const float* __restrict__ xr,
                                                      const uint32_t* __restrict__ wbits,
                                                      const float* __restrict__ scales,
                                                      float* __restrict__ y,
                                                      float* __restrict__ partials,
                                                      uint32_t* __restrict__ counters,
                                                      uint32_t nib_mask) {
  constexpr int NP = (KT / 4 + RB - 1) / RB;  // tables per thread
  // one spare table: threads past the last table write it, so that the table
  // writes need no branch (a branch let the compiler sink the activation load
  // into it, behind the weight loads)
  __shared__ __attribute__((aligned(16))) char lut[(KT / 4 + 1) * kPadTableBytes];
  int rblock, kt;
  tile_of(blockIdx.x, nkt, rblock, kt);
  if (rblock >= nrb) return;  // padding workgroup of the XCD mapping (uniform)
  const int t = threadIdx.x;
  const int k0 = kt * KT;
  const int klen = min(KT, K - k0);
  const int row = rblock * RB + t;
  const bool valid = row < N;
  const int64_t r = valid ? row : 0;

  // x' first, so the tables do not wait behind the weight loads (the
  // scheduling barrier keeps the compiler from moving them after the weights)
  float4 xv[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i)
    xv[i] = *reinterpret_cast<const float4*>(xr + k0 + 4 * min(t + RB * i, klen / 4 - 1));
  __builtin_amdgcn_sched_barrier(0);
  TileRegs<KT> tr;
  load_tile<KT, SCALE4>(tr, wbits + r * (K / 32) + k0 / 32,
                        scales + r * (K / kGroup) + k0 / kGroup, klen);
  __builtin_amdgcn_sched_barrier(0);  // every weight load goes out before the tables
  // (tables past klen hold clamped inputs and are never read)
#pragma unroll
  for (int i = 0; i < NP; ++i)
    write_lut_padded(lut, t + RB * i < KT / 4 ? t + RB * i : KT / 4, xv[i]);
  __syncthreads();
  const float acc = lut_tile<KT, FULL>(tr, klen, lut, nib_mask);
  finish_rows(acc, valid, row, kt, nkt, rblock, N, y, partials, counters);
}

// Fused rotation + LUT GEMV: K-tile = one 1024-block, 256 rows per workgroup.
template <bool PERM>
__global__ __launch_bounds__(256) void rotate_gemv_lut_kernel(
    int N, int K, int nkt, int nrb, const float* __restrict__ x,
    const float* __restrict__ signs, const uint32_t* __restrict__ wbits,
    const float* __restrict__ scales, float* __restrict__ y, float* __restrict__ partials,
    uint32_t* __restrict__ counters, uint32_t nib_mask, Perm perm) {
  constexpr int KT = kWhtBlock;
  __shared__ __attribute__((aligned(16))) char lut[KT / 4 * kPadTableBytes];
  __shared__ __attribute__((aligned(16))) float xs[KT];
  int rblock, kt;
  tile_of(blockIdx.x, nkt, rblock, kt);
  if (rblock >= nrb) return;
  const int t = threadIdx.x;
  const int row = rblock * 256 + t;
  const bool valid = row < N;
  const int64_t r = valid ? row : 0;

  // the activation and signs first; they are multiplied only after every
  // weight load is issued, so the wave does not wait for them in between
  const int k = kt * KT + 4 * t;
  const float4 xraw = *reinterpret_cast<const float4*>(x + (PERM ? perm_source(k, perm) : k));
  const float4 sraw = *reinterpret_cast<const float4*>(signs + k);
  __builtin_amdgcn_sched_barrier(0);
  TileRegs<KT> tr;  // K % 1024 == 0: aligned scale quadruples
  load_tile<KT, true>(tr, wbits + r * (K / 32) + kt * (KT / 32),
                      scales + r * (K / kGroup) + kt * (KT / kGroup), KT);
  __builtin_amdgcn_sched_barrier(0);
  // a multiplication by +-1 is exact
  const float4 v = make_float4(xraw.x * sraw.x, xraw.y * sraw.y, xraw.z * sraw.z, xraw.w * sraw.w);
  fwht1024(v, xs, t);
  __syncthreads();
  write_lut_padded(lut, t, reinterpret_cast<const float4*>(xs)[t]);
  __syncthreads();
  const float acc = lut_tile<KT, true>(tr, KT, lut, nib_mask);
  finish_rows(acc, valid, row, kt, nkt, rblock, N, y, partials, counters);
}

// ---------------------------------------------------------------------------
// EXPAND: bit -> select mask in registers, 8 lanes per row, shuffle reduction
// ---------------------------------------------------------------------------
// Workgroup: 256 threads = 32 rows x 8 groups (one K-tile of 1024) per step;
// `steps` row steps per workgroup (rb = 32 * steps).
template <int STEPS>
__global__ __launch_bounds__(256) void gemv_expand_kernel(int N, int K, int nkt, int nrb,
                                                          const float* __restrict__ xr,
                                                          const uint32_t* __restrict__ wbits,
                                                          const float* __restrict__ scales,
                                                          float* __restrict__ y,
                                                          float* __restrict__ partials,
                                                          uint32_t* __restrict__ counters) {
  constexpr int KT = 1024;
  constexpr int RB = 32 * STEPS;
  int rblock, kt;
  tile_of(blockIdx.x, nkt, rblock, kt);
  if (rblock >= nrb) return;
  const int t = threadIdx.x;
  const int gl = t & 7;          // group of the K-tile owned by this lane
  const int rsub = t >> 3;       // row slot 0..31
  const int k0 = kt * KT;
  const int klen = min(KT, K - k0);
  const bool gvalid = gl * kGroup < klen;

  // this lane's 128 inputs and their sum T
  float xv[kGroup];
  float T = 0.0f;
  {
    const float4* src = reinterpret_cast<const float4*>(xr + k0 + gl * kGroup);
#pragma unroll
    for (int i = 0; i < kGroup / 4; ++i) {
      const float4 v = gvalid ? src[i] : make_float4(0, 0, 0, 0);
      xv[4 * i] = v.x;
      xv[4 * i + 1] = v.y;
      xv[4 * i + 2] = v.z;
      xv[4 * i + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < kGroup; ++i) T += xv[i];
  }

  const int KW = K / 32, KG = K / kGroup;
  uint4 wv[STEPS];
  float sc[STEPS];
  float rowpart[STEPS];
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int row = rblock * RB + s * 32 + rsub;
    const bool in = gvalid && row < N;
    const int64_t r = in ? row : 0;
    wv[s] = in ? *reinterpret_cast<const uint4*>(wbits + r * KW + k0 / 32 + gl * 4)
               : make_uint4(0, 0, 0, 0);
    sc[s] = in ? scales[r * KG + k0 / kGroup + gl] : 0.0f;
  }
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const uint32_t ws[4] = {wv[s].x, wv[s].y, wv[s].z, wv[s].w};
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
#pragma unroll
      for (int j = 0; j < 32; j += 2) {
        // all-ones mask where the bit is set: keeps x, else 0
        const uint32_t m0 = static_cast<uint32_t>(static_cast<int32_t>(ws[wi] << (31 - j)) >> 31);
        const uint32_t m1 =
            static_cast<uint32_t>(static_cast<int32_t>(ws[wi] << (30 - j)) >> 31);
        s0 += __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, xv[32 * wi + j]) & m0);
        s1 += __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, xv[32 * wi + j + 1]) & m1);
      }
    }
    // group partial = scale * (2S - T); reduce the 8 groups of the row
    float part = gvalid ? sc[s] * (2.0f * (s0 + s1) - T) : 0.0f;
    part += __shfl_xor(part, 1, 64);
    part += __shfl_xor(part, 2, 64);
    part += __shfl_xor(part, 4, 64);
    rowpart[s] = part;
  }
  // write: lane gl == 0 of each row slot holds the row's partial
  __shared__ float rowsum[RB];
#pragma unroll
  for (int s = 0; s < STEPS; ++s)
    if (gl == 0) rowsum[s * 32 + rsub] = rowpart[s];
  __syncthreads();
  // redistribute: thread t < RB finishes row rblock*RB + t
  float acc = 0.0f;
  int row = rblock * RB + t;
  bool valid = false;
  if (t < RB) {
    acc = rowsum[t];
    valid = row < N;
  }
  finish_rows(acc, valid, row, kt, nkt, rblock, N, y, partials, counters);
}

// ---------------------------------------------------------------------------
// Launch helpers
// ---------------------------------------------------------------------------

template <int RB, int KT>
hipError_t launch_lut(const float* xr, const uint32_t* wb, const float* sc, float* y,
                      float* part, uint32_t* ctr, int N, int K, int nkt, int nrb,
                      hipStream_t s) {
  const dim3 grid(grid_for(nrb, nkt));
  const bool scale4 = K % 512 == 0 && KT % 512 == 0, full = K % KT == 0;
#define PQ1_LUT_CASE(S4, F)                                                                    \
  if (scale4 == S4 && full == F)                                                               \
    hipLaunchKernelGGL((gemv_lut_kernel<RB, KT, S4, F>), grid, dim3(RB), 0, s, N, K, nkt, nrb, \
                       xr, wb, sc, y, part, ctr, kNibMask);
  PQ1_LUT_CASE(true, true)
  PQ1_LUT_CASE(true, false)
  PQ1_LUT_CASE(false, true)
  PQ1_LUT_CASE(false, false)
#undef PQ1_LUT_CASE
  return hipGetLastError();
}

struct Ws {
  float* partials;
  uint32_t* counters;
};

Ws split_ws(const GemvPlan& p, void* ws) {
  Ws w{nullptr, nullptr};
  if (p.nkt > 1) {
    w.counters = static_cast<uint32_t*>(ws);
    w.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + kCounterBytes);
  }
  return w;
}

}  // namespace

// ---------------------------------------------------------------------------
// Plans
// ---------------------------------------------------------------------------
GemvPlan plan_gemv(int64_t N, int64_t K, int algo, bool fused) {
  GemvPlan p;
  p.algo = (algo == PQ1_GEMV_EXPAND) ? PQ1_GEMV_EXPAND : PQ1_GEMV_LUT;
  auto finish = [&](int rb, int kt) {
    p.rb = rb;
    p.kt = kt;
    p.nkt = static_cast<int>((K + kt - 1) / kt);
    p.nrb = static_cast<int>((N + rb - 1) / rb);
    if (p.nkt > 1 && p.nrb > kMaxRowBlocks) {
      // more row blocks than arrival counters: no plan (the caller returns
      // PQ1_ERR_SHAPE; every kernel is compiled for its K tile, so the K
      // split cannot simply be dropped)
      p.nkt = 0;
      return;
    }
    if (p.nkt > 1) p.partial_bytes = ((static_cast<size_t>(p.nkt) * N * 4 + 255) / 256) * 256;
  };
  if (fused) {
    finish(256, kWhtBlock);
    return p;
  }
  if (p.algo == PQ1_GEMV_EXPAND) {
    finish(128, 1024);
    return p;
  }
  // LUT: prefer large row blocks (cheap tables), shrink until the launch has
  // enough waves to cover the GPU a few times -- but without splitting K
  // into more than 24 tiles, whose partial sums the last-arriving workgroup
  // of a row block adds (measured on ffn_down, K = 17408: 34 tiles of 512 took
  // 15.4 us, 17 tiles of 1024 11.7 us).  Failing both, the candidate with at
  // most 24 tiles and the most waves; failing that, the fewest tiles.
  static const int cand[][2] = {{256, 1024}, {256, 512}, {128, 512}, {128, 256}, {64, 256}};
  const int64_t want_waves = 1536, max_tiles = 24;
  int best = -1;
  int64_t best_waves = -1;
  for (int i = 0; i < 5; ++i) {
    const int64_t tiles = (K + cand[i][1] - 1) / cand[i][1];
    const int64_t waves = ((N + cand[i][0] - 1) / cand[i][0]) * tiles * (cand[i][0] / 64);
    if (tiles > max_tiles) continue;
    if (waves >= want_waves) {
      finish(cand[i][0], cand[i][1]);
      return p;
    }
    if (waves >= best_waves) {  // ties: the smaller row block, as before
      best = i;
      best_waves = waves;
    }
  }
  if (best < 0) best = 0;
  finish(cand[best][0], cand[best][1]);
  return p;
}

size_t gemv_workspace_bytes(int64_t N, int64_t K) {
  size_t m = kCounterBytes;
  const GemvPlan cand[] = {plan_gemv(N, K, PQ1_GEMV_LUT, false),
                           plan_gemv(N, K, PQ1_GEMV_EXPAND, false),
                           plan_gemv(N, K, PQ1_GEMV_LUT, true), plan_gemv_packed(N, K, false),
                           plan_gemv_packed(N, K, true)};
  for (const auto& p : cand) m = std::max(m, p.workspace_bytes());
  return m;
}

hipError_t launch_gemv(const GemvPlan& p, const float* x_rot, const uint32_t* w_bits,
                       const float* scales, float* y, int64_t N, int64_t K, void* workspace,
                       hipStream_t s) {
  const Ws w = split_ws(p, workspace);
  const int n = static_cast<int>(N), k = static_cast<int>(K);
  if (p.nkt < 1) return hipErrorInvalidValue;
  if (p.algo == PQ1_GEMV_EXPAND) {
    if (p.rb != 128 || p.kt != 1024) return hipErrorInvalidValue;
    const dim3 grid(grid_for(p.nrb, p.nkt));
    hipLaunchKernelGGL((gemv_expand_kernel<4>), grid, dim3(256), 0, s, n, k, p.nkt, p.nrb, x_rot,
                       w_bits, scales, y, w.partials, w.counters);
    return hipGetLastError();
  }
  if (p.rb == 256 && p.kt == 1024)
    return launch_lut<256, 1024>(x_rot, w_bits, scales, y, w.partials, w.counters, n, k, p.nkt,
                                 p.nrb, s);
  if (p.rb == 256 && p.kt == 512)
    return launch_lut<256, 512>(x_rot, w_bits, scales, y, w.partials, w.counters, n, k, p.nkt,
                                p.nrb, s);
  if (p.rb == 128 && p.kt == 512)
    return launch_lut<128, 512>(x_rot, w_bits, scales, y, w.partials, w.counters, n, k, p.nkt,
                                p.nrb, s);
  if (p.rb == 128 && p.kt == 256)
    return launch_lut<128, 256>(x_rot, w_bits, scales, y, w.partials, w.counters, n, k, p.nkt,
                                p.nrb, s);
  if (p.rb == 64 && p.kt == 256)
    return launch_lut<64, 256>(x_rot, w_bits, scales, y, w.partials, w.counters, n, k, p.nkt,
                               p.nrb, s);
  return hipErrorInvalidValue;  // no kernel for this plan
}

hipError_t launch_rotate_gemv(const GemvPlan& p, const float* x, const float* signs, Perm perm,
                              const uint32_t* w_bits, const float* scales, float* y, int64_t N,
                              int64_t K, void* workspace, hipStream_t s) {
  const Ws w = split_ws(p, workspace);
  const int n = static_cast<int>(N), k = static_cast<int>(K);
  if (p.nkt < 1 || p.rb != 256 || p.kt != kWhtBlock) return hipErrorInvalidValue;
  const dim3 grid(grid_for(p.nrb, p.nkt));
  if (perm.on)
    hipLaunchKernelGGL((rotate_gemv_lut_kernel<true>), grid, dim3(256), 0, s, n, k, p.nkt, p.nrb,
                       x, signs, w_bits, scales, y, w.partials, w.counters, kNibMask, perm);
  else
    hipLaunchKernelGGL((rotate_gemv_lut_kernel<false>), grid, dim3(256), 0, s, n, k, p.nkt, p.nrb,
                       x, signs, w_bits, scales, y, w.partials, w.counters, kNibMask, perm);
  return hipGetLastError();
}

}  // namespace pq1
