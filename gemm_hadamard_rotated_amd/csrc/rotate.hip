// Activation rotation kernel: x_rot = WHT_1024(signs (.) P x) / 32.
//
// Order from the Pulse ARCHITECTURE-SPEC Hadamard-fold notes: head
// permutation (tiled -> grouped, only when rep > 1), element-wise signs, then
// the normalized Sylvester-Walsh-Hadamard transform with block 1024 and scale
// 1/32.  One 256-thread workgroup transforms one 1024-block of one row: the
// permutation is folded into the load address, the signs into the load, the
// 1/32 into the last butterfly stage and the optional bf16 rounding into the
// store.  Bytes per block: 4 KB of x, 4 KB of signs (cache-resident across
// rows), 4 KB (fp32) or 2 KB (bf16) of output.
#include "pq1_device.h"

namespace pq1 {

namespace {

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // round to nearest even (hardware conversion on gfx950)
  const __bf16 a = static_cast<__bf16>(lo);
  const __bf16 b = static_cast<__bf16>(hi);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

// Output element kinds: fp32, bf16 in natural order, bf16 in the K order of
// the prefill GEMM's MFMA operand (see gemm.hip): inside every 32-wide K
// block, stored position 8c + 2q + t holds the element at offset
// 4c + q + 16t.
enum { kOutF32 = 0, kOutBf16 = 1, kOutBf16Gemm = 2 };

template <bool PERM, int OUT>
__global__ __launch_bounds__(256) void rotate_kernel(int K, int blocks_per_row,
                                                     const float* __restrict__ x,
                                                     const float* __restrict__ signs,
                                                     void* __restrict__ out, Perm perm) {
  __shared__ float sh[kWhtBlock];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x / blocks_per_row;
  const int blk = static_cast<int>(blockIdx.x - row * blocks_per_row);
  const float* xrow = x + row * K;

  const float4 v = load_signed4<PERM>(xrow, signs, blk, t, perm);
  fwht1024(v, sh, t);
  __syncthreads();

  const int64_t o = row * K + static_cast<int64_t>(blk) * kWhtBlock + 4 * t;
  if constexpr (OUT == kOutF32) {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + o) = reinterpret_cast<const float4*>(sh)[t];
  } else {
    float4 r;
    if constexpr (OUT == kOutBf16) {
      r = reinterpret_cast<const float4*>(sh)[t];
    } else {
      // stored positions 4t .. 4t+3: 32-block (4t & ~31), chunk c, elements e
      const int base = (4 * t) & ~31;
      const int c = (t >> 1) & 3;
      const int e0 = (t & 1) * 4;  // e = e0 .. e0+3, q = e / 2, half = e % 2
      const int src = base + 4 * c + (e0 >> 1);
      r = make_float4(sh[src], sh[src + 16], sh[src + 1], sh[src + 17]);
    }
    uint2 p;
    p.x = pack_bf16x2(r.x, r.y);
    p.y = pack_bf16x2(r.z, r.w);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + o) = p;
  }
}

// Embedding gather with the inverse rotation (Pulse ARCHITECTURE-SPEC,
// Hadamard-fold notes: the embedding table stores rotated rows, and the lookup
// applies the transform first and the signs second,
// h = signs * WHT_1024(z) / 32).  z is the token's 1-bit row dequantized as
// in "Inside the One-Bit Engine", station "A token's embedding is 5,120
// numbers with at most 80 different values": +-scale of the 128-group.  One
// workgroup per (token, 1024-block); thread t dequantizes elements 4t .. 4t+3
// (one nibble of one word, one scale).  A token id outside [0, V) yields a
// row of NaNs (and reads nothing of the table).
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tokens,
                                                    const uint32_t* __restrict__ w_bits,
                                                    const float* __restrict__ scales,
                                                    const float* __restrict__ signs,
                                                    float* __restrict__ out, int64_t V, int K,
                                                    int blocks_per_row) {
  __shared__ float sh[kWhtBlock];
  const int t = threadIdx.x;
  const int64_t m = blockIdx.x / blocks_per_row;
  const int blk = static_cast<int>(blockIdx.x - m * blocks_per_row);
  const int64_t row = tokens[m];  // the same for the whole workgroup
  float4* orow = reinterpret_cast<float4*>(out + m * K + static_cast<int64_t>(blk) * kWhtBlock);
  if (row < 0 || row >= V) {
    const float nan = __builtin_nanf("");
    orow[t] = make_float4(nan, nan, nan, nan);
    return;
  }
  const int KW = K / 32, G = K / kGroup;
  const uint32_t word = w_bits[row * KW + blk * (kWhtBlock / 32) + (t >> 3)];
  const float sc = scales[row * G + blk * (kWhtBlock / kGroup) + (t >> 5)];
  const uint32_t nib = word >> (4 * (t & 7));
  const float4 z = make_float4((nib & 1u) ? sc : -sc, (nib & 2u) ? sc : -sc,
                               (nib & 4u) ? sc : -sc, (nib & 8u) ? sc : -sc);
  fwht1024(z, sh, t);
  __syncthreads();
  const float4 r = reinterpret_cast<const float4*>(sh)[t];
  const float4 sg = reinterpret_cast<const float4*>(signs + static_cast<int64_t>(blk) * kWhtBlock)[t];
  orow[t] = make_float4(r.x * sg.x, r.y * sg.y, r.z * sg.z, r.w * sg.w);
}

template <bool PERM, int OUT>
hipError_t launch_rotate_t(const float* x, const float* signs, Perm perm, void* out,
                           int64_t M, int64_t K, hipStream_t stream) {
  const int bpr = static_cast<int>(K / kWhtBlock);
  const dim3 grid(static_cast<unsigned>(M * bpr));
  hipLaunchKernelGGL((rotate_kernel<PERM, OUT>), grid, dim3(256), 0, stream, static_cast<int>(K),
                     bpr, x, signs, out, perm);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rotate(const float* x, const float* signs, Perm perm, void* out, int out_kind,
                         int64_t M, int64_t K, hipStream_t stream) {
  if (perm.on) {
    if (out_kind == kOutBf16Gemm)
      return launch_rotate_t<true, kOutBf16Gemm>(x, signs, perm, out, M, K, stream);
    return out_kind == kOutBf16 ? launch_rotate_t<true, kOutBf16>(x, signs, perm, out, M, K, stream)
                                : launch_rotate_t<true, kOutF32>(x, signs, perm, out, M, K, stream);
  }
  if (out_kind == kOutBf16Gemm)
    return launch_rotate_t<false, kOutBf16Gemm>(x, signs, perm, out, M, K, stream);
  return out_kind == kOutBf16 ? launch_rotate_t<false, kOutBf16>(x, signs, perm, out, M, K, stream)
                              : launch_rotate_t<false, kOutF32>(x, signs, perm, out, M, K, stream);
}

hipError_t launch_embed(const int32_t* tokens, const uint32_t* w_bits, const float* scales,
                        const float* signs, float* out, int64_t M, int64_t V, int64_t K,
                        hipStream_t stream) {
  const int bpr = static_cast<int>(K / kWhtBlock);
  hipLaunchKernelGGL(embed_kernel, dim3(static_cast<unsigned>(M * bpr)), dim3(256), 0, stream,
                     tokens, w_bits, scales, signs, out, V, static_cast<int>(K), bpr);
  return hipGetLastError();
}

}  // namespace pq1
