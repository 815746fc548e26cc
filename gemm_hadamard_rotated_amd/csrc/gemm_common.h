// Device pieces shared by the prefill GEMM kernels (gemm.hip: the 128 x 128
// tiles; gemm_skinny.hip: short prompts): the bf16 operand types, the
// expansion of 1-bit weights into bf16 +-1 matrix-core fragments, and raw
// buffer resources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pq1 {
namespace gemm_detail {

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

// Buffer resource word 3 for raw 32-bit accesses (no swizzle, no index
// stride).  Buffer loads take a uniform base and range from the resource, a
// 32-bit per-lane offset and a uniform offset, so the per-group advance costs
// no vector registers and an out-of-range offset would read zero, not fault.
constexpr int kRawBufferWord3 = 0x00020000;
// s_waitcnt immediate: vector-memory count 0, the other counters unchecked.
constexpr int kWaitVmem0 = 0x0F70;
// s_waitcnt immediate: at most n (< 64) vector-memory operations still
// outstanding (vmcnt counts them in issue order), the other counters
// unchecked.
constexpr int wait_vmem(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kRawBufferWord3);
}

}  // namespace gemm_detail

// Short prompts (gemm_skinny.hip): whether the skinny kernel takes an M x K
// activation block, and its launcher (arguments as launch_gemm; cus = the
// device's compute units, which the plan balances the workgroups over).
bool gemm_skinny_fits(int64_t M, int64_t K);
hipError_t launch_gemm_skinny(const uint16_t* x_bf16, bool x_gemm_order, const uint32_t* w_bits,
                              const float* scales, float* y, int64_t M, int64_t N, int64_t K,
                              int cus, hipStream_t stream);

}  // namespace pq1
