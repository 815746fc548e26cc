// ---------------------------------------------------------------------------
// Measurement kernels for bench.py (not part of the pq1 library): what this
// GPU actually sustains, for the roofline figures next to the published peaks.
//
//  * pq1b_mfma_loop: every wave runs a long chain of v_mfma_f32_32x32x16_bf16
//    on eight independent accumulators, with no memory traffic in the loop.
//    FLOPs per launch = blocks * 4 waves * iters * 8 * 2 * 32 * 32 * 16.
//  * pq1b_mfma_loop_random: the same loop on operands that change from one
//    MFMA to the next: each lane holds 8 A fragments of pseudo-random bf16
//    values (random sign and 7-bit mantissa, exponents over 2^-3 .. 2^4) and
//    8 B fragments of random +-1, the shapes of the prefill GEMM's operands,
//    and chain k of step j takes A (k + j) % 8 and B (k + 3 j + 1) % 8.  The
//    matrix datapath's switching sets its power draw and with it the clock,
//    so this is the rate the matrix cores sustain on data like the GEMM's.
//    `iters` must be a multiple of 8; FLOPs as pq1b_mfma_loop.
//  * pq1b_read: a grid-stride streaming read of `bytes` (16 bytes per lane
//    per load, four loads in flight per lane), folded into a value that is
//    stored only when `store` is set, so nothing but the reads is timed.
//  * pq1b_read_chunks: the strongest plain read this file offers for the
//    same byte count: a workgroup reads whole chunks of 256 lanes x L loads
//    x 16 bytes (lanes coalesced, all L loads issued before any is used),
//    chunk c, c + grid, ...; L in {1, 2, 4, 8, 16}, loads plain or
//    non-temporal.  bench.py times a set of (L, grid, nt) shapes and reports
//    the fastest as the floor a GEMV streaming those bytes can be held to.
//  * pq1b_mark: an empty one-wave kernel.  bench.py launches it right before
//    and right after every timed region, so a kernel trace of a run can be
//    cut down to the timed dispatches.
//  * pq1b_empty: the same empty kernel under another name; graph-replayed on
//    its own it gives the cost of a launch that does nothing.
// All return a hipError_t (0 on success) and never allocate.
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

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(256) void mfma_loop_random_kernel(float* out, int iters, int store) {
  const uint32_t id = blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t u = mix32(id * 131u + static_cast<uint32_t>(f * 8 + e) * 0x9E3779B9u);
      const uint32_t v = mix32(u ^ 0x5bd1e995u);
      const unsigned short ab = static_cast<unsigned short>(((u >> 31) << 15) | ((124u + ((u >> 8) & 7u)) << 7) | (u & 0x7Fu));
      const unsigned short bb = static_cast<unsigned short>(0x3F80u | ((v & 1u) << 15));
      a[f][e] = __builtin_bit_cast(__bf16, ab);
      b[f][e] = __builtin_bit_cast(__bf16, bb);
    }
  f32x16 c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int v = 0; v < 16; ++v) c[k][v] = 0.0f;
  for (int i = 0; i < iters; i += 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(k + j) & 7], b[(k + 3 * j + 1) & 7], c[k], 0, 0, 0);
  }
  if (store) {
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += c[k][v];
    out[id] = s;
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

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int L, bool NT>
__global__ __launch_bounds__(256) void read_chunks_kernel(const u32x4* __restrict__ src,
                                                          int64_t n16, float* out, int store) {
  uint32_t acc = 0;
  const int64_t nchunks = (n16 + 256 * L - 1) / (256 * L);
  for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const int64_t base = c * 256 * L + threadIdx.x;
    u32x4 v[L];
#pragma unroll
    for (int j = 0; j < L; ++j) {
      const int64_t i = min(base + 256 * j, n16 - 1);  // the tail re-reads the last element
      v[j] = NT ? __builtin_nontemporal_load(src + i) : src[i];
    }
#pragma unroll
    for (int j = 0; j < L; ++j) acc ^= v[j][j & 3];
  }
  if (store) out[blockIdx.x * blockDim.x + threadIdx.x] = static_cast<float>(acc);
}

__global__ __launch_bounds__(64) void mark_kernel(float* out, int store) {
  if (store) out[threadIdx.x] = 0.0f;
}

__global__ __launch_bounds__(64) void empty_kernel(float* out, int store) {
  if (store) out[threadIdx.x] = 0.0f;
}

template <int L>
hipError_t launch_chunks(const void* src, int64_t n16, float* out, int blocks, int nt, int store,
                         hipStream_t s) {
  const u32x4* p = static_cast<const u32x4*>(src);
  if (nt)
    hipLaunchKernelGGL((read_chunks_kernel<L, true>), dim3(blocks), dim3(256), 0, s, p, n16, out,
                       store);
  else
    hipLaunchKernelGGL((read_chunks_kernel<L, false>), dim3(blocks), dim3(256), 0, s, p, n16, out,
                       store);
  return hipGetLastError();
}

}  // namespace

extern "C" {

int pq1b_read_chunks(const void* src, int64_t bytes, float* out, int loads, int blocks, int nt,
                     int store, void* stream) {
  if (src == nullptr || bytes < 16 || (bytes & 15) != 0 || blocks < 1 ||
      (store && out == nullptr) || (reinterpret_cast<uintptr_t>(src) & 15) != 0)
    return static_cast<int>(hipErrorInvalidValue);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t n16 = bytes / 16;
  switch (loads) {
    case 1: return static_cast<int>(launch_chunks<1>(src, n16, out, blocks, nt, store, s));
    case 2: return static_cast<int>(launch_chunks<2>(src, n16, out, blocks, nt, store, s));
    case 4: return static_cast<int>(launch_chunks<4>(src, n16, out, blocks, nt, store, s));
    case 8: return static_cast<int>(launch_chunks<8>(src, n16, out, blocks, nt, store, s));
    case 16: return static_cast<int>(launch_chunks<16>(src, n16, out, blocks, nt, store, s));
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

int pq1b_empty(void* stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), nullptr,
                     0);
  return static_cast<int>(hipGetLastError());
}

int pq1b_mark(void* stream) {
  hipLaunchKernelGGL(mark_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), nullptr,
                     0);
  return static_cast<int>(hipGetLastError());
}


int pq1b_mfma_loop(float* out, int blocks, int iters, int store, void* stream) {
  if (blocks < 1 || iters < 1 || (store && out == nullptr)) return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     out, iters, store);
  return static_cast<int>(hipGetLastError());
}

int pq1b_mfma_loop_random(float* out, int blocks, int iters, int store, void* stream) {
  if (blocks < 1 || iters < 8 || (iters & 7) != 0 || (store && out == nullptr))
    return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(mfma_loop_random_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), out, iters, store);
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
