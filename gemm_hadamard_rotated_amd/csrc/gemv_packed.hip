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
#include <algorithm>

#include "gemv_common.h"
#include "pq1.h"
#include "pq1_device.h"

namespace pq1 {

namespace {

constexpr int kBand = 64;
constexpr int kChunk = 1024;                 // K per workgroup (one transform block)
constexpr int kChunkGroups = kChunk / kGroup;  // 8

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
// 1024-wide K chunk; the 4 / BPW waves of a band split the chunk's 8 groups
// and add their partial sums through LDS.  The chunk's 256 tables are built
// once per workgroup (from x_rot, or -- FUSED -- from the raw activation,
// rotated in LDS first).
// ---------------------------------------------------------------------------
template <int BPW, bool FUSED, bool PERM>
__global__ __launch_bounds__(256) void gemv_packed_kernel(
    const float* __restrict__ xin, const float* __restrict__ signs, Perm perm,
    const uint4* __restrict__ pbits, const float* __restrict__ pscales, float* __restrict__ y,
    float* __restrict__ partials, uint32_t* __restrict__ counters, int N, int K, int nkt,
    int nrb, uint32_t nib_mask) {
  constexpr int WPB = 4 / BPW;               // waves per band
  constexpr int GW = kChunkGroups / WPB;     // groups per wave
  __shared__ __attribute__((aligned(16))) float lut[kChunk / 4 * 16];
  __shared__ __attribute__((aligned(16))) float xs[FUSED ? kChunk : 4];
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
  const int g0 = kt * kChunkGroups;
  const int glen = min(kChunkGroups, G - g0);

  // this wave's weights and scales: contiguous 1 KB / 256 B per group
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

  // tables of this chunk
  if constexpr (FUSED) {
    fwht1024(load_signed4<PERM>(xin, signs, kt, t, perm), xs, t);
    __syncthreads();
    write_lut_entry(lut, t, reinterpret_cast<const float4*>(xs)[t]);
  } else {
    if (t < glen * (kGroup / 4))
      write_lut_entry(lut, t, *reinterpret_cast<const float4*>(xin + kt * kChunk + 4 * t));
  }
  __syncthreads();

  const char* lb = reinterpret_cast<const char*>(lut);
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < GW; ++j) {
    const int gl = kq * GW + j;
    if (gl < glen) acc = fmaf(sc[j], lut_group(lb, gl * 32 * 64, w[j], nib_mask), acc);
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
  finish_rows(acc, valid && kq == 0, row, kt, nkt, rblock, N, y, partials, counters);
}

template <int BPW>
hipError_t launch_packed_t(bool fused, bool permute, const float* xin, const float* signs,
                           Perm perm, const void* pbits, const float* pscales, float* y,
                           float* partials, uint32_t* counters, int N, int K, int nkt, int nrb,
                           hipStream_t s) {
  const dim3 grid(grid_for(nrb, nkt));
  const uint4* pb = static_cast<const uint4*>(pbits);
  if (!fused)
    hipLaunchKernelGGL((gemv_packed_kernel<BPW, false, false>), grid, dim3(256), 0, s, xin,
                       signs, perm, pb, pscales, y, partials, counters, N, K, nkt, nrb, kNibMask);
  else if (permute)
    hipLaunchKernelGGL((gemv_packed_kernel<BPW, true, true>), grid, dim3(256), 0, s, xin, signs,
                       perm, pb, pscales, y, partials, counters, N, K, nkt, nrb, kNibMask);
  else
    hipLaunchKernelGGL((gemv_packed_kernel<BPW, true, false>), grid, dim3(256), 0, s, xin, signs,
                       perm, pb, pscales, y, partials, counters, N, K, nkt, nrb, kNibMask);
  return hipGetLastError();
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

GemvPlan plan_gemv_packed(int64_t N, int64_t K) {
  GemvPlan p;
  p.algo = PQ1_GEMV_LUT;
  const int64_t nbands = (N + kBand - 1) / kBand;
  const int64_t nkt = (K + kChunk - 1) / kChunk;
  // bands per workgroup: share a chunk's tables among more rows when the grid
  // still has enough waves to cover the GPU
  int bpw = 1;
  for (int c : {4, 2}) {
    if (((nbands + c - 1) / c) * nkt * 4 >= 2048) {
      bpw = c;
      break;
    }
  }
  p.rb = bpw * kBand;
  p.kt = kChunk;
  p.nkt = static_cast<int>(nkt);
  p.nrb = static_cast<int>((nbands + bpw - 1) / bpw);
  if (p.nkt > 1 && p.nrb > kMaxRowBlocks) {
    p.nkt = 0;  // unsupported: far more rows than any 1-bit matrix here; caller errors out
    return p;
  }
  if (p.nkt > 1) p.partial_bytes = ((static_cast<size_t>(p.nkt) * N * 4 + 255) / 256) * 256;
  return p;
}

hipError_t launch_gemv_packed(const GemvPlan& p, bool fused, const float* xin, const float* signs,
                              Perm perm, const void* pbits, const float* pscales, float* y,
                              int64_t N, int64_t K, void* workspace, hipStream_t s) {
  float* partials = nullptr;
  uint32_t* counters = nullptr;
  if (p.nkt > 1) {
    counters = static_cast<uint32_t*>(workspace);
    partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes);
  }
  const int n = static_cast<int>(N), k = static_cast<int>(K);
  const int bpw = p.rb / kBand;
  if (bpw == 4)
    return launch_packed_t<4>(fused, perm.on, xin, signs, perm, pbits, pscales, y, partials,
                              counters, n, k, p.nkt, p.nrb, s);
  if (bpw == 2)
    return launch_packed_t<2>(fused, perm.on, xin, signs, perm, pbits, pscales, y, partials,
                              counters, n, k, p.nkt, p.nrb, s);
  return launch_packed_t<1>(fused, perm.on, xin, signs, perm, pbits, pscales, y, partials,
                            counters, n, k, p.nkt, p.nrb, s);
}

}  // namespace pq1
