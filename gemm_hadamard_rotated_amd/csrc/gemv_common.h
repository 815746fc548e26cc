// Device pieces shared by the GEMV kernels (canonical and packed layouts):
// the 16-entry signed-sum tables, the table walk over one 128-weight group,
// the workgroup -> (row block, K-tile) mapping and the split-K epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pq1_internal.h"

namespace pq1 {

// Always 0x3C3C3C3C; passed to the kernels as an argument so that the compiler
// keeps the two masked words E and O and extracts every table offset with one
// byte extract (instead of a shift and a mask per nibble).
constexpr uint32_t kNibMask = 0x3C3C3C3Cu;

// ---------------------------------------------------------------------------
// 16 signed sums of four inputs ("Inside the One-Bit Engine", station "Four
// one-bit weights have only sixteen possible answers"): entry e holds
// sum_i (bit i of e ? +x_i : -x_i), so a table read replaces four
// multiply-adds and needs no "2S - T" correction.  Table p (16 floats, 64 B)
// serves inputs 4p .. 4p+3.
//
// Padded table layout used by the packed-layout kernels: table p starts at
// byte 80 p (16 floats + 16 bytes of padding).  A lane that writes a whole
// table with four 16-byte stores then hits banks 20p .. 20p+15 (mod 32), so
// any 8 consecutive lanes -- one 16-byte store cycle -- cover all 32 banks
// once; with 64-byte tables every other lane would collide.
constexpr int kPadTableBytes = 80;

__device__ __forceinline__ void write_lut_padded(char* __restrict__ lut, int p, float4 xv) {
  const float a = xv.x + xv.y, b = xv.x - xv.y;
  const float c = xv.z + xv.w, d = xv.z - xv.w;
  const float lo[4] = {-a, b, -b, a};
  const float hi[4] = {-c, d, -d, c};
  float4* dst = reinterpret_cast<float4*>(lut + p * kPadTableBytes);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    dst[q] = make_float4(lo[0] + hi[q], lo[1] + hi[q], lo[2] + hi[q], lo[3] + hi[q]);
}

// (x >> 8B) & 0x3C in one instruction: SDWA selects byte B of x (zero
// extended) and ANDs it with m (0x3C in every byte, held in a VGPR).  The
// compiler's own pattern is a shift and an AND, or a masked word and a
// bit-field extract, per byte.
template <int B>
__device__ __forceinline__ uint32_t byte_off(uint32_t x, uint32_t m) {
  uint32_t r;
  if constexpr (B == 0)
    r = x & 0x3Cu;
  else if constexpr (B == 1)
    asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 "
        "src1_sel:DWORD" : "=v"(r) : "v"(x), "v"(m));
  else if constexpr (B == 2)
    asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2 "
        "src1_sel:DWORD" : "=v"(r) : "v"(x), "v"(m));
  else
    asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3 "
        "src1_sel:DWORD" : "=v"(r) : "v"(x), "v"(m));
  return r;
}

// Sum over one 128-weight group held as 4 words, reading the 32 tables that
// start at byte offset `tab` of `lut` (tables TS bytes apart).  Nibble q of word w (weights
// 32w + 4q .. +3, LSB first) indexes table 8w + q.  All lanes of a wave walk
// the same tables in the same order, so each read touches at most 16
// addresses in 16 distinct banks.  Table offsets: byte b of (w << 2) & 0x3C3C3C3C
// is 4 * nibble 2b, byte b of (w >> 2) & 0x3C3C3C3C is 4 * nibble 2b+1.  SDWA
// extracts each of them with one instruction (10 instead of 12 per word; it
// made the packed-layout kernels 2-3 % faster and the canonical ones slower,
// so it is a parameter).  ROT: the word is stored rotated left by 2 bits (the
// packed layout), so w itself stands in for w << 2 and a rotation right by 4
// for w >> 2 (9 per word).
template <int TS = 64, bool SDWA = false, bool ROT = false>
__device__ __forceinline__ float lut_group(const char* __restrict__ lut_bytes, int tab, uint4 w4,
                                           uint32_t nib_mask) {
  const uint32_t ws[4] = {w4.x, w4.y, w4.z, w4.w};
  float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
  for (int wi = 0; wi < 4; ++wi) {
    const uint32_t w = ws[wi];
    uint32_t off[8];  // off[2b] = 4 * nibble 2b, off[2b + 1] = 4 * nibble 2b+1
    if constexpr (SDWA) {
      const uint32_t e = ROT ? w : w << 2;
      const uint32_t o = ROT ? __builtin_amdgcn_alignbit(w, w, 4) : w >> 2;
      off[0] = byte_off<0>(e, nib_mask);
      off[1] = byte_off<0>(o, nib_mask);
      off[2] = byte_off<1>(e, nib_mask);
      off[3] = byte_off<1>(o, nib_mask);
      off[4] = byte_off<2>(e, nib_mask);
      off[5] = byte_off<2>(o, nib_mask);
      off[6] = byte_off<3>(e, nib_mask);
      off[7] = byte_off<3>(o, nib_mask);
    } else {
      static_assert(!ROT, "the rotated layout is walked with SDWA only");
      const uint32_t E = (w << 2) & nib_mask;
      const uint32_t O = (w >> 2) & nib_mask;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        off[2 * b] = (E >> (8 * b)) & 0xFFu;
        off[2 * b + 1] = (O >> (8 * b)) & 0xFFu;
      }
    }
    const char* base = lut_bytes + tab + wi * 8 * TS;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float fe = *reinterpret_cast<const float*>(base + (2 * b) * TS + off[2 * b]);
      const float fo = *reinterpret_cast<const float*>(base + (2 * b + 1) * TS + off[2 * b + 1]);
      if (wi == 0 && b == 0) {
        p0 = fe;
        p1 = fo;
      } else {
        p0 += fe;
        p1 += fo;
      }
    }
  }
  return p0 + p1;
}

// ---------------------------------------------------------------------------
// Workgroup -> (row block, K-tile).  Workgroups are dealt to the 8 XCDs round
// robin; this mapping keeps all K-tiles of a row block on one XCD.  The grid
// has round_up(nrb, 8) * nkt workgroups; those with rblock >= nrb exit.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void tile_of(int bid, int nkt, int& rblock, int& kt) {
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  kt = slot % nkt;
  rblock = (slot / nkt) * 8 + xcd;
}

inline int grid_for(int nrb, int nkt) { return ((nrb + 7) & ~7) * nkt; }

// ---------------------------------------------------------------------------
// Split-K epilogue.  With one K-tile the row result is stored directly.
// Otherwise each workgroup stores its partial sums, waits until the stores
// have completed, and bumps its row block's arrival counter; the workgroup
// that arrives last adds the partials of all K-tiles in K order (the result
// does not depend on arrival order), stores y and resets the counter to zero.
// Partials and counters are accessed as relaxed agent-scope atomics: they are
// written to and read from the device-coherent level directly, so no
// whole-cache write-back or invalidate is needed (measured: a __threadfence
// based version was 3x slower on a 14 MB GEMV).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void finish_rows(float acc, bool valid, int row, int kt, int nkt,
                                            int rblock, int N, float* __restrict__ y,
                                            float* __restrict__ partials,
                                            uint32_t* __restrict__ counters) {
  if (nkt == 1) {
    if (valid) y[row] = acc;
    return;
  }
  __shared__ int s_last;
  if (valid)
    __hip_atomic_store(&partials[static_cast<int64_t>(kt) * N + row], acc, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partials are stored
  __syncthreads();                                   // ... and every other wave's
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(&counters[rblock], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == static_cast<uint32_t>(nkt - 1));
  }
  __syncthreads();
  if (!s_last) return;
  if (valid) {
    // issue up to 32 loads at once, then add in K-tile order
    float sum = 0.0f;
    for (int j0 = 0; j0 < nkt; j0 += 32) {
      float v[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int j = min(j0 + u, nkt - 1);
        v[u] = __hip_atomic_load(&partials[static_cast<int64_t>(j) * N + row], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int u = 0; u < 32; ++u)
        if (j0 + u < nkt) sum += v[u];
    }
    y[row] = sum;
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(&counters[rblock], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Split-K epilogue by float atomics (packed-layout kernels): wait until the
// pair's gen word reaches `want` -- K chunk 0 has zeroed the rows -- add the
// partial sums into y and record `want` in the pair's seen word.  `first` is
// a value of gen the caller read earlier (gen only moves towards `want` during
// a launch, so a match there needs no further poll).  The wait is bounded
// (2^16 polls, each a short sleep and an L2 read: well under a second); on
// expiry the wave ORs kStatusWaitGaveUp into the status word, adds NaN
// instead of its partial sums and still records `want`, so every wave of the
// launch exits.  K chunk 0 checks the pair at its next launch (it
// publishes seen + 1 and poisons the band's rows if gen and seen disagreed),
// so the bookkeeping is back in step after one call.
// ---------------------------------------------------------------------------
constexpr int kMaxPolls = 1 << 16;

__device__ __forceinline__ void add_rows_after_gen(float acc, bool valid, int row,
                                                   float* __restrict__ y,
                                                   const uint32_t* __restrict__ gen,
                                                   uint32_t* __restrict__ seen,
                                                   uint32_t* __restrict__ status, uint32_t want,
                                                   uint32_t first) {
  int spins = 0;
  uint32_t g = first;
  while (g != want) {
    if (++spins > kMaxPolls) {
      acc = __builtin_nanf("");
      if ((threadIdx.x & 63) == 0)
        __hip_atomic_fetch_or(status, kStatusWaitGaveUp, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    if (spins > 1) __builtin_amdgcn_s_sleep(2);
    g = __hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (valid) __hip_atomic_fetch_add(&y[row], acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((threadIdx.x & 63) == 0)
    __hip_atomic_exchange(seen, want, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace pq1
