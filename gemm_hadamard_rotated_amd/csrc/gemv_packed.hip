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
//                 of row 64b + l (zero for rows >= N);
//   packed_scales float [nb][G][64]: element (b, g, l) = scale[64b + l][g]
//                 (zero for rows >= N).
// Same bits and scales, same byte count (plus the last band's padding).
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>

#include "gemv_common.h"
#include "pq1.h"
#include "pq1_device.h"

namespace pq1 {

namespace {

constexpr int kBand = 64;

// ---------------------------------------------------------------------------
// Repack
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_kernel(const uint4* __restrict__ w_bits,
                                                   const float* __restrict__ scales,
                                                   uint4* __restrict__ pbits,
                                                   float* __restrict__ pscales, int N, int G,
                                                   int64_t total) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int l = static_cast<int>(i % kBand);
    const int64_t bg = i / kBand;
    const int g = static_cast<int>(bg % G);
    const int64_t b = bg / G;
    const int64_t n = b * kBand + l;
    uint4 w = make_uint4(0, 0, 0, 0);
    float s = 0.0f;
    if (n < N) {
      w = w_bits[n * G + g];  // row n has G uint4 (4 words per 128 weights)
      s = scales[n * G + g];
    }
    pbits[i] = w;
    pscales[i] = s;
  }
}

// ---------------------------------------------------------------------------
// GEMV on the packed layout.  A workgroup (4 waves) handles BPW bands x one
// K chunk of CH groups (CH * 128 inputs, a multiple of the 1024 transform
// block); the 4 / BPW waves of a band split the chunk's groups and add their
// partial sums through LDS.  Order of work, chosen from a per-workgroup
// timeline of the kernel: first the loads of the chunk's activation (x_rot,
// or -- FUSED -- the raw x and the signs), so the tables do not wait behind
// the weight stream; then the weight and scale loads; then the tables (one
// per thread, padded layout), the walk as the groups arrive, and the atomic
// split-K epilogue.
// ---------------------------------------------------------------------------
template <int BPW, int CH, bool FUSED, bool PERM>
__global__ __launch_bounds__(256) void gemv_packed_kernel(
    const float* __restrict__ xin, const float* __restrict__ signs, Perm perm,
    const uint4* __restrict__ pbits, const float* __restrict__ pscales, float* __restrict__ y,
    uint32_t* __restrict__ flags, int N, int K, int nkt, int nrb, uint32_t epoch,
    uint32_t nib_mask) {
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
  const int wave = t >> 6, lane = t & 63;
  const int band_local = wave / WPB, kq = wave % WPB;
  const int nbands = (N + kBand - 1) / kBand;
  const int band = rblock * BPW + band_local;
  const int row = band * kBand + lane;
  const bool valid = row < N;
  const int G = K / kGroup;
  const int g0 = kt * CH;
  const int glen = min(CH, G - g0);
  const int npos = glen * (kGroup / 4);  // tables in this chunk

  // 1. the chunk's activation
  float4 xv[FUSED ? NB : NP];
  if constexpr (FUSED) {
#pragma unroll
    for (int b = 0; b < NB; ++b) xv[b] = load_signed4<PERM>(xin, signs, kt * NB + b, t, perm);
  } else {
#pragma unroll
    for (int i = 0; i < NP; ++i)
      xv[i] = *reinterpret_cast<const float4*>(xin + static_cast<int64_t>(kt) * KC +
                                               4 * min(t + 256 * i, npos - 1));
  }
  // 2. this wave's weights and scales: contiguous 1 KB / 256 B per group
  const int64_t bandc = min(band, nbands - 1);
  uint4 w[GW];
  float sc[GW];
#pragma unroll
  for (int j = 0; j < GW; ++j) {
    const int g = min(g0 + kq * GW + j, G - 1);
    const int64_t idx = (bandc * G + g) * kBand + lane;
    sc[j] = pscales[idx];
    w[j] = pbits[idx];
  }
  // 3. K-tile 0 zeroes the row block's outputs for the atomic epilogue
  uint32_t* flag = flags + rblock;
  if (nkt > 1 && kt == 0) zero_rows_and_publish(valid && kq == 0, row, y, flag, epoch);
  // 4. tables
  if constexpr (FUSED) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      fwht1024(xv[b], xs + b * kWhtBlock, t);
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < NP; ++i)
      write_lut_padded(lut, t + 256 * i, reinterpret_cast<const float4*>(xs)[t + 256 * i]);
  } else {
#pragma unroll
    for (int i = 0; i < NP; ++i)
      if (t + 256 * i < npos) write_lut_padded(lut, t + 256 * i, xv[i]);
  }
  __syncthreads();
  // 5. walk
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < GW; ++j) {
    const int gl = kq * GW + j;
    if (gl < glen)
      acc = fmaf(sc[j], lut_group<kPadTableBytes>(lut, gl * 32 * kPadTableBytes, w[j], nib_mask),
                 acc);
  }
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
  if (nkt == 1) {
    if (valid) y[row] = acc;
  } else {
    add_rows_atomic(acc, valid, row, y, flag, epoch);
  }
}

template <int BPW, int CH>
hipError_t launch_packed_t(bool fused, bool permute, const float* xin, const float* signs,
                           Perm perm, const void* pbits, const float* pscales, float* y,
                           uint32_t* flags, int N, int K, int nkt, int nrb, uint32_t epoch,
                           hipStream_t s) {
  const dim3 grid(grid_for(nrb, nkt));
  const uint4* pb = static_cast<const uint4*>(pbits);
  if (!fused)
    hipLaunchKernelGGL((gemv_packed_kernel<BPW, CH, false, false>), grid, dim3(256), 0, s, xin,
                       signs, perm, pb, pscales, y, flags, N, K, nkt, nrb, epoch, kNibMask);
  else if (permute)
    hipLaunchKernelGGL((gemv_packed_kernel<BPW, CH, true, true>), grid, dim3(256), 0, s, xin,
                       signs, perm, pb, pscales, y, flags, N, K, nkt, nrb, epoch, kNibMask);
  else
    hipLaunchKernelGGL((gemv_packed_kernel<BPW, CH, true, false>), grid, dim3(256), 0, s, xin,
                       signs, perm, pb, pscales, y, flags, N, K, nkt, nrb, epoch, kNibMask);
  return hipGetLastError();
}

// Tuning override for experiments: PQ1_PACKED_PLAN="bpw,ch" (bpw in {1,2,4},
// ch in {8,16}); read once.
bool plan_override(int* bpw, int* ch) {
  static int ob = -1, oc = -1;
  static bool init = false;
  if (!init) {
    init = true;
    if (const char* e = getenv("PQ1_PACKED_PLAN")) {
      int b = 0, c = 0;
      if (sscanf(e, "%d,%d", &b, &c) == 2 && (b == 1 || b == 2 || b == 4) && (c == 8 || c == 16)) {
        ob = b;
        oc = c;
      }
    }
  }
  if (ob < 0) return false;
  *bpw = ob;
  *ch = oc;
  return true;
}

}  // namespace

size_t packed_bits_bytes(int64_t N, int64_t K) {
  return static_cast<size_t>((N + kBand - 1) / kBand) * (K / kGroup) * kBand * 16;
}

size_t packed_scales_bytes(int64_t N, int64_t K) {
  return static_cast<size_t>((N + kBand - 1) / kBand) * (K / kGroup) * kBand * 4;
}

hipError_t launch_pack(const uint32_t* w_bits, const float* scales, int64_t N, int64_t K,
                       void* pbits, float* pscales, hipStream_t s) {
  const int G = static_cast<int>(K / kGroup);
  const int64_t total = ((N + kBand - 1) / kBand) * G * kBand;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 8192);
  hipLaunchKernelGGL(pack_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(w_bits), scales, static_cast<uint4*>(pbits),
                     pscales, static_cast<int>(N), G, total);
  return hipGetLastError();
}

GemvPlan plan_gemv_packed(int64_t N, int64_t K, bool fused) {
  GemvPlan p;
  p.algo = PQ1_GEMV_LUT;
  const int64_t nbands = (N + kBand - 1) / kBand;
  // chunk of 8 groups (one transform block); bands per workgroup: share the
  // chunk's tables among more rows when the grid still has enough waves
  int ch = 8, bpw = 1;
  const int64_t nkt8 = (K + 1023) / 1024;
  for (int c : {4, 2}) {
    if (((nbands + c - 1) / c) * nkt8 * 4 >= 2048) {
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
  if (p.nkt > 1 && p.nrb > kMaxRowBlocks) {
    p.nkt = 0;  // unsupported row count (> 2M rows with split K): the caller errors out
    return p;
  }
  p.partial_bytes = 0;  // the atomic epilogue needs only the flag region
  return p;
}

hipError_t launch_gemv_packed(const GemvPlan& p, bool fused, const float* xin, const float* signs,
                              Perm perm, const void* pbits, const float* pscales, float* y,
                              int64_t N, int64_t K, void* workspace, uint32_t epoch,
                              hipStream_t s) {
  uint32_t* flags = nullptr;
  if (p.nkt > 1)
    flags = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + kFlagOffset);
  const int n = static_cast<int>(N), k = static_cast<int>(K);
  const int bpw = p.rb / kBand;
  const int ch = p.kt / kGroup;
#define PQ1_PACKED_CASE(B, C)                                                                   \
  if (bpw == B && ch == C)                                                                     \
    return launch_packed_t<B, C>(fused, perm.on, xin, signs, perm, pbits, pscales, y, flags, n, \
                                 k, p.nkt, p.nrb, epoch, s);
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
