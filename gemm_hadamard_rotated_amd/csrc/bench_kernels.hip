// ---------------------------------------------------------------------------
// Measurement kernels for bench.py (not part of the pq1 library): what this
// GPU actually sustains, for the roofline figures next to the published peaks.
//
//  * pq1b_mfma_loop: every wave runs a long chain of v_mfma_f32_32x32x16_bf16
//    on eight independent accumulators, with no memory traffic in the loop.
//    FLOPs per launch = blocks * 4 waves * iters * 8 * 2 * 32 * 32 * 16.
//  * pq1b_read: a grid-stride streaming read of `bytes` (16 bytes per lane
//    per load, four loads in flight per lane), folded into a value that is
//    stored only when `store` is set, so nothing but the reads is timed.
// Both return a hipError_t (0 on success) and never allocate.
// ---------------------------------------------------------------------------
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_loop_kernel(float* out, int iters, int store) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = static_cast<__bf16>(static_cast<float>((lane + j) & 7) - 3.0f);
    b[j] = static_cast<__bf16>(static_cast<float>((3 * lane + j) & 7) - 4.0f);
  }
  f32x16 c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int v = 0; v < 16; ++v) c[k][v] = 0.0f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
  }
  if (store) {
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += c[k][v];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  }
}

__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                   float* out, int store) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
    acc ^= v0.x ^ v1.y ^ v2.z ^ v3.w;
  }
  for (; i < n16; i += stride) acc ^= src[i].x;
  if (store) out[blockIdx.x * blockDim.x + threadIdx.x] = static_cast<float>(acc);
}

}  // namespace

extern "C" {

int pq1b_mfma_loop(float* out, int blocks, int iters, int store, void* stream) {
  if (blocks < 1 || iters < 1 || (store && out == nullptr)) return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     out, iters, store);
  return static_cast<int>(hipGetLastError());
}

int pq1b_read(const void* src, int64_t bytes, float* out, int blocks, int store, void* stream) {
  if (src == nullptr || bytes < 16 || (bytes & 15) != 0 || blocks < 1 || (store && out == nullptr) ||
      (reinterpret_cast<uintptr_t>(src) & 15) != 0)
    return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), bytes / 16, out, store);
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
