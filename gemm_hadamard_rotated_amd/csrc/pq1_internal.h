// Internal declarations shared by the HIP translation units of libpq1.
// Not part of the public ABI (include/pq1.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pq1 {

constexpr int kWhtBlock = 1024;  // transform block length
constexpr int kGroup = 128;      // weights per scale
// Split-K workspace: a counter region first (zero-filled once by the caller;
// every call leaves it in a state the next call accepts), partials after.
// Bytes [0, 32 KB) hold the arrival counters of the canonical-layout kernels
// (one per row block, left zero); bytes [32 KB, kStatusOffset) the generation
// and seen words of the packed-layout kernels (one pair per (band, K chunk));
// the word at kStatusOffset collects the status bits below.
constexpr size_t kCounterBytes = 262144;
constexpr size_t kFlagOffset = 32768;
constexpr size_t kStatusOffset = kCounterBytes - 256;
constexpr int kMaxRowBlocks = static_cast<int>(kFlagOffset / 4);
constexpr int64_t kMaxPackedSlots = static_cast<int64_t>((kStatusOffset - kFlagOffset) / 8);
constexpr int64_t kStatusWord = 2 * kMaxPackedSlots;  // its index from the generation words
constexpr int kMaxPublish = 512;  // (band, K chunk) pairs one K-chunk-0 workgroup advances
// Status bits (the words are only ever OR-ed into; the caller clears them):
constexpr uint32_t kStatusWaitGaveUp = 1u;  // a K chunk's bounded wait for chunk 0 expired
constexpr uint32_t kStatusOutOfStep = 2u;   // a generation / seen pair disagreed at launch
// Test flags of the packed GEMV (set through pq1_set_test_flags; zero in use).
constexpr uint32_t kTestWithholdPublish = 1u;  // K chunk 0 never advances its gen words
uint32_t test_flags();

struct Perm {
  int hd = 0, nk = 0, rep = 0;
  bool on = false;  // rep > 1
};

// ---------------------------------------------------------------------------
// GEMV launch plan (shared by the launcher and the workspace-size query)
// ---------------------------------------------------------------------------
struct GemvPlan {
  int algo = 0;     // PQ1_GEMV_LUT or PQ1_GEMV_EXPAND
  int rb = 0;       // rows per workgroup
  int kt = 0;       // K-tile (elements) handled by one workgroup
  int nkt = 0;      // number of K-tiles = ceil(K / kt)
  int nrb = 0;      // number of row blocks = ceil(N / rb)
  size_t partial_bytes = 0;   // nkt * N * 4, rounded up to 256 (0 when nkt == 1)
  size_t workspace_bytes() const { return nkt > 1 ? kCounterBytes + partial_bytes : 0; }
};

GemvPlan plan_gemv(int64_t N, int64_t K, int algo, bool fused);
size_t gemv_workspace_bytes(int64_t N, int64_t K);

// ---------------------------------------------------------------------------
// Launchers (arguments already validated; return the launch error)
// ---------------------------------------------------------------------------
// out_kind: PQ1_F32, PQ1_BF16 or PQ1_BF16_GEMM
hipError_t launch_rotate(const float* x, const float* signs, Perm perm, void* out, int out_kind,
                         int64_t M, int64_t K, hipStream_t stream);

// Embedding rows with the inverse rotation: out[m] = signs * WHT(dequant(row tokens[m])) / 32.
hipError_t launch_embed(const int32_t* tokens, const uint32_t* w_bits, const float* scales,
                        const float* signs, float* out, int64_t M, int64_t V, int64_t K,
                        hipStream_t stream);

hipError_t launch_gemv(const GemvPlan& plan, const float* x_rot, const uint32_t* w_bits,
                       const float* scales, float* y, int64_t N, int64_t K,
                       void* workspace, hipStream_t stream);

hipError_t launch_rotate_gemv(const GemvPlan& plan, const float* x, const float* signs,
                              Perm perm, const uint32_t* w_bits, const float* scales,
                              float* y, int64_t N, int64_t K, void* workspace,
                              hipStream_t stream);

// Band-interleaved ("packed") weight layout, see gemv_packed.hip.
size_t packed_bits_bytes(int64_t N, int64_t K);
// scale_dtype PQ1_SCALE_F32 or PQ1_SCALE_F16 (validated by the caller).
size_t packed_scales_bytes(int64_t N, int64_t K, int scale_dtype);
GemvPlan plan_gemv_packed(int64_t N, int64_t K, bool fused);
// Rows 0 .. N-1 of w_bits / scales into rows row0 .. row0+N-1 of a packed
// matrix of N_total rows.
hipError_t launch_pack(const uint32_t* w_bits, const float* scales, int64_t N, int64_t K,
                       void* pbits, void* pscales, int scale_dtype, int64_t N_total,
                       int64_t row0, hipStream_t stream);
// The library's own counter region on the current device (for callers that
// cannot allocate): its device address, zeroed by a kernel enqueued on `s`
// at the first call on the device.  kScratchBytes is the counter region: the
// packed-layout plans need nothing beyond it.
constexpr size_t kScratchBytes = kCounterBytes;
hipError_t packed_scratch(hipStream_t s, void** out);
hipError_t launch_gemv_packed(const GemvPlan& plan, bool fused, const float* xin,
                              const float* signs, Perm perm, const void* pbits,
                              const void* pscales, int scale_dtype, float* y, int64_t N,
                              int64_t K, void* workspace, hipStream_t stream);

// x_gemm_order: X is in the GEMM K order (PQ1_X_GEMM_ORDER), else row-major
// cus: compute units of the current device (sizes the GEMM-order tail split).
hipError_t launch_gemm(const uint16_t* x_bf16, bool x_gemm_order, const uint32_t* w_bits,
                       const float* scales, float* y, int64_t M, int64_t N, int64_t K, int cus,
                       hipStream_t stream);

}  // namespace pq1
