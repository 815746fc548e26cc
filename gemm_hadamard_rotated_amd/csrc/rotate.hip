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

template <bool PERM, bool BF16>
__global__ __launch_bounds__(256) void rotate_kernel(const float* __restrict__ x,
                                                     const float* __restrict__ signs,
                                                     Perm perm, void* __restrict__ out,
                                                     int K, int blocks_per_row) {
  __shared__ float sh[kWhtBlock];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x / blocks_per_row;
  const int blk = static_cast<int>(blockIdx.x - row * blocks_per_row);
  const float* xrow = x + row * K;

  const float4 v = load_signed4<PERM>(xrow, signs, blk, t, perm);
  fwht1024(v, sh, t);
  __syncthreads();

  const float4 r = reinterpret_cast<const float4*>(sh)[t];
  const int64_t o = row * K + static_cast<int64_t>(blk) * kWhtBlock + 4 * t;
  if constexpr (BF16) {
    uint2 p;
    p.x = pack_bf16x2(r.x, r.y);
    p.y = pack_bf16x2(r.z, r.w);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + o) = p;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + o) = r;
  }
}

template <bool PERM, bool BF16>
hipError_t launch_rotate_t(const float* x, const float* signs, Perm perm, void* out,
                           int64_t M, int64_t K, hipStream_t stream) {
  const int bpr = static_cast<int>(K / kWhtBlock);
  const dim3 grid(static_cast<unsigned>(M * bpr));
  hipLaunchKernelGGL((rotate_kernel<PERM, BF16>), grid, dim3(256), 0, stream, x, signs, perm,
                     out, static_cast<int>(K), bpr);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rotate(const float* x, const float* signs, Perm perm, void* out,
                         bool out_bf16, int64_t M, int64_t K, hipStream_t stream) {
  if (perm.on) {
    return out_bf16 ? launch_rotate_t<true, true>(x, signs, perm, out, M, K, stream)
                    : launch_rotate_t<true, false>(x, signs, perm, out, M, K, stream);
  }
  return out_bf16 ? launch_rotate_t<false, true>(x, signs, perm, out, M, K, stream)
                  : launch_rotate_t<false, false>(x, signs, perm, out, M, K, stream);
}

}  // namespace pq1
