// Device-side building blocks shared by the rotation and the fused
// rotation+GEMV kernels: the permuted, sign-flipped load of one 1024-block and
// its normalized Sylvester-Walsh-Hadamard transform in registers + LDS.
//
// Layout of a 1024-block inside a 256-thread workgroup: thread t owns the four
// consecutive elements i = 4t .. 4t+3 (one float4).  Index bits of i:
//   bits 0-1  -> the element inside the thread      (butterflies in registers)
//   bits 2-7  -> the lane inside the 64-wide wave     (butterflies across lanes)
//   bits 8-9  -> the wave inside the workgroup        (butterflies through LDS)
// The Sylvester matrix H[i][j] = (-1)^popcount(i & j) factors into one
// radix-2 butterfly per index bit, in any order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pq1_internal.h"

namespace pq1 {

// Position in the tiled input that feeds post-permutation position k.
// Grouped head h' = r + rep*n takes tiled head n + nk*r (hd values per head).
__device__ __forceinline__ int perm_source(int k, const Perm& p) {
  const int h = k / p.hd;
  const int d = k - h * p.hd;
  const int n = h / p.rep;
  const int r = h - n * p.rep;
  return (n + p.nk * r) * p.hd + d;
}

// Load 4 consecutive post-permutation elements of block `blk` of row `xrow`
// and multiply them by the signs.  `hd` is a multiple of 4, so the four
// elements come from one contiguous run of the source row.
template <bool PERM>
__device__ __forceinline__ float4 load_signed4(const float* __restrict__ xrow,
                                               const float* __restrict__ signs,
                                               int blk, int t, const Perm& p) {
  const int k = blk * kWhtBlock + 4 * t;
  const int src = PERM ? perm_source(k, p) : k;
  const float4 v = *reinterpret_cast<const float4*>(xrow + src);
  const float4 s = *reinterpret_cast<const float4*>(signs + k);
  // multiplication by +-1 is exact
  return make_float4(v.x * s.x, v.y * s.y, v.z * s.z, v.w * s.w);
}

// Butterfly with the partner lane `lane ^ MASK`: the lane whose index bit is
// clear keeps a + b, the other keeps a - b (here: partner - own); fmaf with a
// +-1 factor rounds exactly like the plain add / subtract.  The lane exchange
// is done in the vector ALU where gfx950 has an instruction for it (no LDS
// round trip):
//   masks 1, 2: DPP quad permutations [1,0,3,2] and [2,3,0,1];
//   mask 8:     DPP rotation of each 16-lane row by 8;
//   masks 16, 32: v_permlane16_swap / v_permlane32_swap of the value with
//               itself, which leaves every lane both members of its pair
//               (r[0] the one whose index bit is clear, r[1] the other), so
//               the result is r[0] + r[1] or r[0] - r[1] -- the same single
//               rounding of the same exact sum as fmaf(sgn, own, partner);
//   mask 4:     ds_swizzle in xor mode (no lane-address register).
template <int MASK>
__device__ __forceinline__ float lane_butterfly(float v, float sgn) {
  const int i = __builtin_bit_cast(int, v);
  if constexpr (MASK == 16 || MASK == 32) {
    const auto r = MASK == 16 ? __builtin_amdgcn_permlane16_swap(i, i, false, false)
                              : __builtin_amdgcn_permlane32_swap(i, i, false, false);
    return fmaf(sgn, __builtin_bit_cast(float, static_cast<int>(r[1])),
                __builtin_bit_cast(float, static_cast<int>(r[0])));
  } else {
    int o;
    if constexpr (MASK == 1) o = __builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, true);
    else if constexpr (MASK == 2) o = __builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, true);
    else if constexpr (MASK == 8) o = __builtin_amdgcn_mov_dpp(i, 0x128, 0xF, 0xF, true);
    else o = __builtin_amdgcn_ds_swizzle(i, (MASK << 10) | 0x1F);  // xor MASK within 32 lanes
    return fmaf(sgn, v, __builtin_bit_cast(float, o));
  }
}

// The six lane stages (bits 2..7 of the block index) of one float4.
__device__ __forceinline__ float4 lane_stages(float4 v, int lane) {
  auto stage = [&](auto m) {
    constexpr int M = decltype(m)::value;
    const float sgn = (lane & M) ? -1.0f : 1.0f;
    v.x = lane_butterfly<M>(v.x, sgn);
    v.y = lane_butterfly<M>(v.y, sgn);
    v.z = lane_butterfly<M>(v.z, sgn);
    v.w = lane_butterfly<M>(v.w, sgn);
  };
  stage(std::integral_constant<int, 1>{});
  stage(std::integral_constant<int, 2>{});
  stage(std::integral_constant<int, 4>{});
  stage(std::integral_constant<int, 8>{});
  stage(std::integral_constant<int, 16>{});
  stage(std::integral_constant<int, 32>{});
  return v;
}

// Normalized 1024-point transform of the block held as one float4 per thread
// (256 threads).  On return sh[0..1023] holds the transformed block, already
// multiplied by 1/32, in natural order; the caller must __syncthreads() before
// reading it.  `sh` must hold 1024 floats.
__device__ __forceinline__ void fwht1024(float4 v, float* __restrict__ sh, int t) {
  // bits 0 and 1: inside the thread
  {
    const float a0 = v.x + v.y, a1 = v.x - v.y;
    const float a2 = v.z + v.w, a3 = v.z - v.w;
    v = make_float4(a0 + a2, a1 + a3, a0 - a2, a1 - a3);
  }
  // bits 2..7: across the 64 lanes of the wave
  v = lane_stages(v, t & 63);
  // bits 8 and 9: across the four waves, through LDS
  reinterpret_cast<float4*>(sh)[t] = v;
  __syncthreads();
  float a[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) a[w] = sh[t + 256 * w];
  const float b0 = a[0] + a[1], b1 = a[0] - a[1];
  const float b2 = a[2] + a[3], b3 = a[2] - a[3];
  constexpr float kScale = 0.03125f;  // 1/32, exact
  sh[t] = (b0 + b2) * kScale;
  sh[t + 256] = (b1 + b3) * kScale;
  sh[t + 512] = (b0 - b2) * kScale;
  sh[t + 768] = (b1 - b3) * kScale;
}

// The same transform split for callers that want thread t's result as the
// four consecutive outputs 4t .. 4t+3 (the rows of a signed-sum table) rather
// than in LDS.  fwht1024_lanes: bits 0..7 in registers, then thread t stores
// its float4 at sh[4t .. 4t+3].  After a __syncthreads(), fwht1024_out reads
// the four float4s at positions 4 (t % 64) + 256 w, w = 0..3 (the bit-8/9
// partners of the thread's outputs) and combines them for its own bits 8-9
// (t / 64), with the same additions in the same order as fwht1024, so the
// results are identical.  One barrier fewer than fwht1024 plus a read-back.
__device__ __forceinline__ void fwht1024_lanes(float4 v, float* __restrict__ sh, int t) {
  {
    const float a0 = v.x + v.y, a1 = v.x - v.y;
    const float a2 = v.z + v.w, a3 = v.z - v.w;
    v = make_float4(a0 + a2, a1 + a3, a0 - a2, a1 - a3);
  }
  v = lane_stages(v, t & 63);
  reinterpret_cast<float4*>(sh)[t] = v;
}

__device__ __forceinline__ float4 fwht1024_out(const float* __restrict__ sh, int t) {
  const float4* s4 = reinterpret_cast<const float4*>(sh) + (t & 63);
  const float4 a0 = s4[0], a1 = s4[64], a2 = s4[128], a3 = s4[192];
  const int w = t >> 6;  // bits 8 and 9 of this thread's outputs (uniform per wave)
  const float s1 = (w & 1) ? -1.0f : 1.0f, s2 = (w & 2) ? -1.0f : 1.0f;
  constexpr float kScale = 0.03125f;  // 1/32, exact
  auto one = [&](float x0, float x1, float x2, float x3) {
    // fwht1024: b0 = x0 + x1, b1 = x0 - x1, b2 = x2 + x3, b3 = x2 - x3, then
    // b0 + b2, b1 + b3, b0 - b2, b1 - b3 for w = 0, 1, 2, 3 (fmaf with +-1
    // rounds like the plain add / subtract)
    const float lo = fmaf(s1, x1, x0), hi = fmaf(s1, x3, x2);
    return fmaf(s2, hi, lo) * kScale;
  };
  return make_float4(one(a0.x, a1.x, a2.x, a3.x), one(a0.y, a1.y, a2.y, a3.y),
                     one(a0.z, a1.z, a2.z, a3.z), one(a0.w, a1.w, a2.w, a3.w));
}

}  // namespace pq1
