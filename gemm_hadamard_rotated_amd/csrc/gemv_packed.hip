// Band-interleaved weight layout and the decode GEMV on it.
//
// "Inside the One-Bit Engine" describes a load-time repack of the 1-bit
// weights into a band-interleaved order that the vecmat kernel prefers; this
// file is the gfx950 version of that idea.  The GEMV kernels give each lane
// one output row (so the 16-entry tables of a wave are read conflict-free);
// in the canonical row-major layout the 64 lanes of a wave then read 64
// different rows, 16 bytes from each, which costs ~45% more time than a
// coalesced stream of the same bytes on MI355X.  In the packed layout the 64
// rows of a band are interleaved per 128-weight group, so the 64 lanes read
// 1 KB of contiguous memory per load instruction.
//
// Packed layout for N rows, K columns (nb = ceil(N / 64) bands, G = K / 128):
//   packed_bits   uint4 [nb][G][64]: element (b, g, l) holds words 4g .. 4g+3
//                 of row 64b + l, each rotated left by 2 bits (zero for rows
//                 >= N).  After the rotation byte b of a word holds 4 times
//                 nibble 2b at bits 2-5, so one byte-select AND gives that
//                 nibble's table offset, and one rotation right by 4 does the
//                 same for the odd nibbles;
//   packed_scales float or f16 [nb][G][64]: element (b, g, l) = scale[64b + l][g]
//                 (zero for rows >= N).
// Same bits and, with fp32 scales, the same scales and byte count (plus the
// last band's padding).  With f16 scales ("Inside the One-Bit Engine", station
// on a token's embedding: 640 bytes of bits and 80 bytes of f16 scales per
// 5120-wide row, 1.125 bits per weight) the repack rounds each scale to the
// nearest f16, ties to even, and the GEMV widens it back to fp32 exactly.
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <utility>

#include "gemv_common.h"
#include "pq1.h"
#include "pq1_device.h"

namespace pq1 {

namespace {

constexpr int kBand = 64;
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));  // for non-temporal loads

// Scale storage: fp32 as given, or the bit pattern of an f16 (uint16_t, so
// that kernel names demangle).  fp32 -> f16 rounds to nearest even (the
// default rounding mode); f16 -> fp32 is exact.
__device__ inline void store_scale(float* p, float v) { *p = v; }
__device__ inline void store_scale(uint16_t* p, float v) {
  *p = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}
__device__ inline float scale_value(float s) { return s; }
__device__ inline float scale_value(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// ---------------------------------------------------------------------------
// Repack
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t rotl2(uint32_t w) { return __builtin_amdgcn_alignbit(w, w, 30); }

// Source rows 0 .. Ns-1 go to rows row0 .. row0+Ns-1 of a packed matrix of
// Nt rows; the kernel walks the bands those rows touch (entry i of the walk is
// lane i % 64 of group (i / 64) % G of band b_lo + i / (64 G)), zeroes the
// entries of rows >= Nt and leaves the entries of other rows alone, so several
// matrices with the same K can be packed one after another into one.
template <typename SCT>  // float, or uint16_t holding f16 bits
__global__ __launch_bounds__(256) void pack_kernel(const uint4* __restrict__ w_bits,
                                                   const float* __restrict__ scales,
                                                   uint4* __restrict__ pbits,
                                                   SCT* __restrict__ pscales, int64_t row0,
                                                   int64_t Ns, int64_t Nt, int G, int64_t b_lo,
                                                   int64_t total) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int l = static_cast<int>(i % kBand);
    const int64_t bg = i / kBand;
    const int g = static_cast<int>(bg % G);
    const int64_t b = b_lo + bg / G;
    const int64_t n = b * kBand + l;
    const int64_t o = (b * G + g) * kBand + l;
    if (n >= row0 && n < row0 + Ns) {
      const int64_t src = n - row0;
      const uint4 v = w_bits[src * G + g];  // row src has G uint4 (4 words per 128 weights)
      pbits[o] = make_uint4(rotl2(v.x), rotl2(v.y), rotl2(v.z), rotl2(v.w));
      store_scale(&pscales[o], scales[src * G + g]);
    } else if (n >= Nt) {
      pbits[o] = make_uint4(0, 0, 0, 0);
      store_scale(&pscales[o], 0.0f);
    }
  }
}

// ---------------------------------------------------------------------------
// GEMV on the packed layout.  A workgroup (4 waves) handles BPW bands x one
// K chunk of CH groups (CH * 128 inputs, a multiple of the 1024 transform
// block); the 4 / BPW waves of a band split the chunk's groups and add their
// partial sums through LDS.
//
// Order of work, chosen from per-wave timelines of the kernel on MI355X: the
// caches are cold at every launch, so the activation comes from memory and,
// once the weight stream is in flight, queues behind it; the tables (and so
// the whole walk) wait for it.  Each wave therefore issues its activation
// loads and only its first group's weights, builds the tables, and only then
// issues the rest of its weights.  (Issuing everything up front made the
// tables ready ~0.6 us later on ffn_gate; issuing no weights before the
// tables left the memory pipe idle.)
//
// (The non-fused kernel builds its tables without a transform; there issuing
// all weights up front measured faster.)
//
// Split-K epilogue (K chunks > 1), with no state from the host: every
// (band, K chunk > 0) pair owns a generation word `gen` and a word `seen`
// in the workspace (slot band * nkt + k, at fixed offsets), equal at every
// launch boundary whatever shapes earlier calls had.  The workgroup of K chunk
// 0 reads the gen words of its bands first thing, zeroes its rows, waits until
// the zeros are stored and writes gen + 1.  The result wave of band b in K
// chunk k reads seen first thing, waits until gen == seen + 1, adds its
// partial sums into y with float atomics and writes seen + 1.  Each launch
// thus moves every pair forward by one, so a captured graph may replay the
// launch any number of times.  The polled gen words are only ever read and
// written with plain coherent loads and stores (L2 atomics on them made the
// polls ~0.4 us slower); the early reads of gen and seen are issued right
// after the activation loads, ahead of the weight stream (measured best of
// first / after the activation / after the weights).  K chunk 0 has the
// lowest workgroup index of its row block and the same XCD, so in practice it
// is dispatched first; the HIP runtime does not promise that order, so the
// wait is bounded (add_rows_after_gen): on expiry the wave reports
// kStatusWaitGaveUp in the workspace's status word and adds NaN.  K chunk 0
// also reads each pair's seen word; gen and seen must agree at a launch
// boundary, and where they do not (an earlier expired wait, or a workspace
// that was not zero-filled) it stores NaN into the band's rows, reports
// kStatusOutOfStep and publishes seen + 1, which puts the pair back in step.
// Either way the launch ends normally and the caller learns of it from the
// status word (PQ1_GEMV_STATUS_OFFSET in the header).
// ---------------------------------------------------------------------------
// (Parameter order: the sizes that place the workgroup and the pointers of its
// first loads come first, inside the 14 dwords the hardware preloads into
// SGPRs; see build.py.)
template <int BPW, int CH, bool FUSED, bool PERM, typename SCT>
__global__ __launch_bounds__(256) void gemv_packed_kernel(
    int N, int K, int nkt, int nrb, const float* __restrict__ xin,
    const float* __restrict__ signs, const uint4* __restrict__ pbits,
    const SCT* __restrict__ pscales, uint32_t* __restrict__ gens, float* __restrict__ y,
    uint32_t nib_mask, uint32_t test_flags, Perm perm) {
  constexpr int WPB = 4 / BPW;     // waves per band
  constexpr int GW = CH / WPB;     // groups per wave
  constexpr int KC = CH * kGroup;  // inputs per chunk
  constexpr int NB = CH / 8;       // transform blocks per chunk
  constexpr int NP = KC / 4 / 256; // tables per thread
  __shared__ __attribute__((aligned(16))) char lut[KC / 4 * kPadTableBytes];
  __shared__ __attribute__((aligned(16))) float xs[FUSED ? KC : 4];
  __shared__ float red[WPB > 1 ? 4 : 1][kBand];

  int rblock, kt;
  tile_of(blockIdx.x, nkt, rblock, kt);
  if (rblock >= nrb) return;  // padding workgroup (uniform)
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int band_local = wave / WPB, kq = wave % WPB;
  const int nbands = (N + kBand - 1) / kBand;
  const int band = rblock * BPW + band_local;
  const int row = band * kBand + lane;
  const bool valid = row < N;
  const int G = K / kGroup;
  const int g0 = kt * CH;
  const int glen = min(CH, G - g0);
  const int npos = glen * (kGroup / 4);  // tables in this chunk
  const bool split = nkt > 1;

  // 0. generation words: slot band * nkt + k; gen at gens[slot], seen at
  //    gens[kMaxPackedSlots + slot] (fixed offsets, so that calls of any shapes
  //    can share a workspace: each call advances both words of its slots)
  const int npub = BPW * (nkt - 1);  // (band, K chunk > 0) pairs of this row block
  uint32_t gen_old[kMaxPublish / 256], seen_old[kMaxPublish / 256];
  uint32_t seen = 0;
  auto pub_slot = [&](int k) {
    return static_cast<int64_t>(rblock * BPW + k / (nkt - 1)) * nkt + 1 + k % (nkt - 1);
  };
  // 1. the chunk's activation (the fused kernel multiplies by the signs only
  //    at the transform, after the weight loads are issued)
  float4 xv[FUSED ? NB : NP];
  float4 sv[FUSED ? NB : 1];
  if constexpr (FUSED) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int k = (kt * NB + b) * kWhtBlock + 4 * t;
      xv[b] = *reinterpret_cast<const float4*>(xin + (PERM ? perm_source(k, perm) : k));
      sv[b] = *reinterpret_cast<const float4*>(signs + k);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NP; ++i)
      xv[i] = *reinterpret_cast<const float4*>(xin + static_cast<int64_t>(kt) * KC +
                                               4 * min(t + 256 * i, npos - 1));
  }
  if (split) {
    // The loads are unconditional (slot 0 stands in where a wave or lane has
    // nothing to read): loads under a branch made the compiler wait for them
    // -- and for the activation issued before them -- where the branch joins,
    // ahead of the weight loads.
    seen = __hip_atomic_load(
        &gens[kMaxPackedSlots + (kt != 0 && kq == 0 ? static_cast<int64_t>(band) * nkt + kt : 0)],
        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (kt == 0) {
#pragma unroll
      for (int i = 0; i < kMaxPublish / 256; ++i) {
        const int64_t sl = t + 256 * i < npub ? pub_slot(t + 256 * i) : 0;
        gen_old[i] = __hip_atomic_load(&gens[sl], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        seen_old[i] = __hip_atomic_load(&gens[kMaxPackedSlots + sl], __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }

  // 2. this wave's weights: 1 KB of bits and 256 B (f16: 128 B) of scales
  //    per group, contiguous; the fused kernel issues only its first group here
  const int64_t bandc = min(band, nbands - 1);
  // (scales stay in their stored type until the FMA that uses them: an f16
  // widened at its load made the wave wait for that load right there)
  uint4 w[GW];
  SCT sc[GW];
  auto load_group = [&](int j) {
    const int g = min(g0 + kq * GW + j, G - 1);
    const int64_t idx = (bandc * G + g) * kBand + lane;
    // streamed once per launch: non-temporal loads, so they do not evict the
    // activation, the tables' inputs or the bookkeeping words from the caches
    // (output head -0.9 us, ssm_out -0.14 us, ffn_gate unchanged)
    sc[j] = __builtin_nontemporal_load(&pscales[idx]);
    const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(pbits) + idx);
    w[j] = make_uint4(v[0], v[1], v[2], v[3]);
  };
  constexpr int kPre = FUSED ? 1 : GW;
  // 3. K chunk 0 zeroes the row block's outputs (before its early weight
  //    loads) and advances the gen words once the zeros are stored.  The wait
  //    counts exactly the 2 kPre weight loads issued after the zero stores (a
  //    bits load and a scales load per group, in issue order; the scheduling
  //    barriers keep that order), so it does not wait for those loads.
  const bool zeroing = split && kt == 0;  // uniform
  if (zeroing && valid && kq == 0)
    __hip_atomic_store(&y[row], 0.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < kPre; ++j) load_group(j);
  __builtin_amdgcn_sched_barrier(0);
  if (zeroing) {
    static_assert(2 * kPre <= 63, "vmcnt holds at most 63");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kPre) : "memory");  // this wave's zeros are stored
    __syncthreads();                                                  // ... and every other wave's
#pragma unroll
    for (int i = 0; i < kMaxPublish / 256; ++i) {
      const int k = t + 256 * i;
      if (k >= npub) continue;
      if (gen_old[i] != seen_old[i]) {
        // out of step at a launch boundary: the band's sum cannot be trusted
        // this time; poison its rows (after the zeros, before the publish)
        const int b = rblock * BPW + k / (nkt - 1);
        for (int l = 0; l < kBand; ++l)
          if (b * kBand + l < N)
            __hip_atomic_store(&y[b * kBand + l], __builtin_nanf(""), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_or(&gens[kStatusWord], kStatusOutOfStep, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      // the contributors of this pair read seen at their start and wait for
      // seen + 1 (equal to gen + 1 whenever the pair is in step)
      if (!(test_flags & kTestWithholdPublish))
        __hip_atomic_store(&gens[pub_slot(k)], seen_old[i] + 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // (the transform below waits for the activation: keep it after the loads)
  __builtin_amdgcn_sched_barrier(0);
  // 4. tables
  if constexpr (FUSED) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      // a multiplication by +-1 is exact
      const float4 v = make_float4(xv[b].x * sv[b].x, xv[b].y * sv[b].y, xv[b].z * sv[b].z,
                                   xv[b].w * sv[b].w);
      if constexpr (GW > 1) {
        // the second weight group goes out as soon as this wave's activation
        // has arrived (ffn_gate 5.35 -> 5.28 us; issuing two groups here, or
        // the second one after the transform, measured slower: 5.52, 5.44)
        if (b == 0) {
          asm volatile("" ::"v"(v.x), "v"(v.w));  // the activation has landed
          __builtin_amdgcn_sched_barrier(0);
          load_group(1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      fwht1024_lanes(v, xs + b * kWhtBlock, t);
    }
    __syncthreads();
    // table 256 b + t holds inputs 1024 b + 4t .. +3: thread t's outputs
#pragma unroll
    for (int b = 0; b < NB; ++b) write_lut_padded(lut, t + 256 * b, fwht1024_out(xs + b * kWhtBlock, t));
  } else {
#pragma unroll
    for (int i = 0; i < NP; ++i)
      if (t + 256 * i < npos) write_lut_padded(lut, t + 256 * i, xv[i]);
  }
  __syncthreads();
  // 5. the rest of this wave's weights, then the walk as they arrive
  constexpr int kRest = (FUSED && GW > 1) ? 2 : kPre;  // first group not yet issued
#pragma unroll
  for (int j = kRest; j < GW; ++j) load_group(j);
  // The walk is specialised on the wave's place in its band (uniform), so
  // that every table address is a compile-time offset from the LDS array and
  // goes into the read's immediate field: each lookup address is then one
  // byte extract, with no register base to combine.
  float acc = 0.0f;
  auto walk = [&](auto kq_c) {
    constexpr int KQ = decltype(kq_c)::value;
#pragma unroll
    for (int j = 0; j < GW; ++j) {
      constexpr int kTab = 32 * kPadTableBytes;
      if (KQ * GW + j < glen)
        acc = fmaf(scale_value(sc[j]),
                   lut_group<kPadTableBytes, true, true>(lut, (KQ * GW + j) * kTab, w[j], nib_mask), acc);
    }
  };
  if constexpr (WPB == 1) {
    walk(std::integral_constant<int, 0>{});
  } else if constexpr (WPB == 2) {
    if (kq == 0) walk(std::integral_constant<int, 0>{});
    else walk(std::integral_constant<int, 1>{});
  } else {
    if (kq == 0) walk(std::integral_constant<int, 0>{});
    else if (kq == 1) walk(std::integral_constant<int, 1>{});
    else if (kq == 2) walk(std::integral_constant<int, 2>{});
    else walk(std::integral_constant<int, 3>{});
  }
  // the contributors' generation word, read after the walk (its latency
  // overlaps the reduction's barrier); unconditional, the packed bits stand in
  __builtin_amdgcn_sched_barrier(0);
  const uint32_t* gen_at =
      split ? &gens[kt != 0 && kq == 0 ? static_cast<int64_t>(band) * nkt + kt : 0]
            : reinterpret_cast<const uint32_t*>(pbits);
  const uint32_t gen_now = __hip_atomic_load(gen_at, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (WPB > 1) {
    red[wave][lane] = acc;
    __syncthreads();
    if (kq == 0) {
      acc = red[wave][lane];
#pragma unroll
      for (int q = 1; q < WPB; ++q) acc += red[wave + q][lane];
    }
  }
  // 6. results
  if (kq != 0) return;
  if (!split) {
    if (valid) y[row] = acc;
  } else if (kt == 0) {
    if (valid) __hip_atomic_fetch_add(&y[row], acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    const int64_t slot = static_cast<int64_t>(band) * nkt + kt;
    // (the empty asm keeps "seen + 1" from being folded back into the branch
    // that loaded seen, which made the wave wait for that load -- and for the
    // activation issued before it -- ahead of its first weight loads)
    asm volatile("" : "+v"(seen));
    add_rows_after_gen(acc, valid, row, y, &gens[slot], &gens[kMaxPackedSlots + slot],
                       &gens[kStatusWord], seen + 1u, gen_now);
  }
}

template <int BPW, int CH, typename SCT>
hipError_t launch_packed_t(bool fused, bool permute, const float* xin, const float* signs,
                           Perm perm, const void* pbits, const void* pscales_v, float* y,
                           uint32_t* gens, int N, int K, int nkt, int nrb, hipStream_t s) {
  const dim3 grid(grid_for(nrb, nkt));
  const uint4* pb = static_cast<const uint4*>(pbits);
  const SCT* pscales = static_cast<const SCT*>(pscales_v);
  const uint32_t tf = test_flags();
  if (!fused)
    hipLaunchKernelGGL((gemv_packed_kernel<BPW, CH, false, false, SCT>), grid, dim3(256), 0, s,
                       N, K, nkt, nrb, xin, signs, pb, pscales, gens, y, kNibMask, tf, perm);
  else if (permute)
    hipLaunchKernelGGL((gemv_packed_kernel<BPW, CH, true, true, SCT>), grid, dim3(256), 0, s,
                       N, K, nkt, nrb, xin, signs, pb, pscales, gens, y, kNibMask, tf, perm);
  else
    hipLaunchKernelGGL((gemv_packed_kernel<BPW, CH, true, false, SCT>), grid, dim3(256), 0, s,
                       N, K, nkt, nrb, xin, signs, pb, pscales, gens, y, kNibMask, tf, perm);
  return hipGetLastError();
}

// Tuning override for experiments: PQ1_PACKED_PLAN="bpw,ch" (bpw in {1,2,4},
// ch in {8,16}; anything else is ignored), read once per process (the
// initialization of a function-local static is thread-safe).
bool plan_override(int* bpw, int* ch) {
  static const std::pair<int, int> ov = [] {
    int b = 0, c = 0;
    const char* e = getenv("PQ1_PACKED_PLAN");
    if (e && sscanf(e, "%d,%d", &b, &c) == 2 && (b == 1 || b == 2 || b == 4) &&
        (c == 8 || c == 16))
      return std::pair<int, int>{b, c};
    return std::pair<int, int>{-1, -1};
  }();
  if (ov.first < 0) return false;
  *bpw = ov.first;
  *ch = ov.second;
  return true;
}

// ---------------------------------------------------------------------------
// The library's own split-K counter region, for callers that cannot allocate
// (pq1_rotate_gemv_packed_noalloc).  One copy per GPU, held until the process
// ends.  In host code `scratch` names a host-side stand-in, not the device
// copy: the device address comes from hipGetSymbolAddress, once per device,
// and only that address is ever handed to a kernel.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint32_t scratch[kScratchBytes / 4];

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

constexpr int kMaxScratchDevices = 64;
void* g_scratch[kMaxScratchDevices];
std::mutex g_scratch_mu;

}  // namespace

hipError_t packed_scratch(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    // the generation / seen pairs must start equal: zero the region once, on
    // the caller's stream, with a kernel (no memset node if it is captured)
    constexpr int n = static_cast<int>(kScratchBytes / 4);
    hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, s, static_cast<uint32_t*>(ptr),
                       n);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

size_t packed_bits_bytes(int64_t N, int64_t K) {
  return static_cast<size_t>((N + kBand - 1) / kBand) * (K / kGroup) * kBand * 16;
}

size_t packed_scales_bytes(int64_t N, int64_t K, int scale_dtype) {
  const size_t elem = scale_dtype == PQ1_SCALE_F16 ? 2 : 4;
  return static_cast<size_t>((N + kBand - 1) / kBand) * (K / kGroup) * kBand * elem;
}

hipError_t launch_pack(const uint32_t* w_bits, const float* scales, int64_t N, int64_t K,
                       void* pbits, void* pscales, int scale_dtype, int64_t N_total, int64_t row0,
                       hipStream_t s) {
  const int G = static_cast<int>(K / kGroup);
  const int64_t b_lo = row0 / kBand, b_hi = (row0 + N - 1) / kBand;
  const int64_t total = (b_hi - b_lo + 1) * G * kBand;
  const dim3 grid(static_cast<unsigned>(std::min<int64_t>((total + 255) / 256, 8192)));
  const uint4* wb = reinterpret_cast<const uint4*>(w_bits);
  uint4* pb = static_cast<uint4*>(pbits);
  if (scale_dtype == PQ1_SCALE_F16)
    hipLaunchKernelGGL(pack_kernel<uint16_t>, grid, dim3(256), 0, s, wb, scales, pb,
                       static_cast<uint16_t*>(pscales), row0, N, N_total, G, b_lo, total);
  else
    hipLaunchKernelGGL(pack_kernel<float>, grid, dim3(256), 0, s, wb, scales, pb,
                       static_cast<float*>(pscales), row0, N, N_total, G, b_lo, total);
  return hipGetLastError();
}

GemvPlan plan_gemv_packed(int64_t N, int64_t K, bool fused) {
  GemvPlan p;
  p.algo = PQ1_GEMV_LUT;
  const int64_t nbands = (N + kBand - 1) / kBand;
  // chunk of 8 groups (one transform block); bands per workgroup: share the
  // chunk's tables among more rows when the grid still has enough waves --
  // four bands only on large matrices (measured, fused step, us: output head
  // N = 248320: 42 with four, 47 with two; gate + up N = 34816: 9.2 with
  // two, 9.5 with four; ffn_gate / ffn_down: two; ssm_out N = 5120: one)
  int ch = 8, bpw = 1;
  const int64_t nkt8 = (K + 1023) / 1024;
  for (const auto& [c, min_waves] : {std::pair<int, int64_t>{4, 8192}, {2, 2048}}) {
    if (((nbands + c - 1) / c) * nkt8 * 4 >= min_waves) {
      bpw = c;
      break;
    }
  }
  plan_override(&bpw, &ch);
  if (fused && (K % (ch * kGroup)) != 0) ch = 8;  // a fused chunk must be whole blocks
  p.rb = bpw * kBand;
  p.kt = ch * kGroup;
  p.nkt = static_cast<int>((K + p.kt - 1) / p.kt);
  p.nrb = static_cast<int>((nbands + bpw - 1) / bpw);
  if (p.nkt > 1 && (static_cast<int64_t>(p.nrb) * bpw * p.nkt > kMaxPackedSlots ||
                    bpw * (p.nkt - 1) > kMaxPublish)) {
    p.nkt = 0;  // too many (band, K chunk) pairs for the generation region: the caller errors out
    return p;
  }
  p.partial_bytes = 0;  // the atomic epilogue needs only the generation region
  return p;
}

hipError_t launch_gemv_packed(const GemvPlan& p, bool fused, const float* xin, const float* signs,
                              Perm perm, const void* pbits, const void* pscales, int scale_dtype,
                              float* y, int64_t N, int64_t K, void* workspace, hipStream_t s) {
  uint32_t* gens = nullptr;
  if (p.nkt > 1) gens = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + kFlagOffset);
  const int n = static_cast<int>(N), k = static_cast<int>(K);
  const int bpw = p.rb / kBand;
  const int ch = p.kt / kGroup;
#define PQ1_PACKED_CASE(B, C)                                                                   \
  if (bpw == B && ch == C)                                                                     \
    return scale_dtype == PQ1_SCALE_F16                                                        \
               ? launch_packed_t<B, C, uint16_t>(fused, perm.on, xin, signs, perm, pbits,     \
                                                 pscales, y, gens, n, k, p.nkt, p.nrb, s)     \
               : launch_packed_t<B, C, float>(fused, perm.on, xin, signs, perm, pbits,        \
                                              pscales, y, gens, n, k, p.nkt, p.nrb, s);
  PQ1_PACKED_CASE(1, 8)
  PQ1_PACKED_CASE(2, 8)
  PQ1_PACKED_CASE(4, 8)
  PQ1_PACKED_CASE(1, 16)
  PQ1_PACKED_CASE(2, 16)
  PQ1_PACKED_CASE(4, 16)
#undef PQ1_PACKED_CASE
  return hipErrorInvalidValue;
}

}  // namespace pq1
