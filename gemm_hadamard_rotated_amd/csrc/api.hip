// C ABI of libpq1: argument validation and launches (see include/pq1.h).
//
// Every entry point validates all arguments on the host before it touches the
// HIP runtime, so invalid calls return an error without a device.  Kernels
// are launched on the caller's stream; nothing synchronizes the host.
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <unordered_map>

#include "pq1.h"
#include "pq1_internal.h"

static_assert(PQ1_GEMV_COUNTER_BYTES == pq1::kCounterBytes, "workspace layout mismatch");
static_assert(PQ1_GEMV_STATUS_OFFSET == pq1::kStatusOffset, "workspace layout mismatch");
static_assert(PQ1_SPLITK_WAIT_GAVE_UP == pq1::kStatusWaitGaveUp &&
                  PQ1_SPLITK_OUT_OF_STEP == pq1::kStatusOutOfStep,
              "status bits mismatch");
static_assert(PQ1_TEST_WITHHOLD_PUBLISH == pq1::kTestWithholdPublish, "test flag mismatch");

namespace {

thread_local int32_t g_last_hip_error = 0;
std::atomic<uint32_t> g_test_flags{0};

// Largest sizes the kernels index with 32-bit ints.
constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;
constexpr int64_t kMaxElems = (int64_t{1} << 31) - 1;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bn && b0 < a0 + an;
}

// Per-device "is this a gfx950" cache (and its compute-unit count); checked
// once per device.
constexpr int kMaxDevices = 64;
int g_dev_state[kMaxDevices];  // 0 unknown, 1 ok, 2 wrong architecture
int g_dev_cus[kMaxDevices];
std::mutex g_dev_mu;

pq1_status check_device(int* cus = nullptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    g_last_hip_error = static_cast<int32_t>(e);
    return PQ1_ERR_DEVICE;
  }
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_state[dev] == 1) {
      if (cus) *cus = g_dev_cus[dev];
      return PQ1_OK;
    }
    if (g_dev_state[dev] == 2) return PQ1_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int32_t>(e);
    return PQ1_ERR_DEVICE;
  }
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  g_dev_cus[dev] = prop.multiProcessorCount;
  g_dev_state[dev] = ok ? 1 : 2;
  if (cus) *cus = prop.multiProcessorCount;
  return ok ? PQ1_OK : PQ1_ERR_DEVICE;
}

pq1_status launched(hipError_t e) {
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int32_t>(e);
    return PQ1_ERR_LAUNCH;
  }
  return PQ1_OK;
}

pq1_status check_perm(const pq1_perm* perm, int64_t K, pq1::Perm* out) {
  *out = pq1::Perm{};
  if (perm == nullptr || perm->rep <= 1) return PQ1_OK;
  if (perm->hd < 1 || perm->nk < 1) return PQ1_ERR_PERM;
  if (perm->hd % 4 != 0) return PQ1_ERR_PERM;
  if (static_cast<int64_t>(perm->hd) * perm->nk * perm->rep != K) return PQ1_ERR_PERM;
  out->hd = perm->hd;
  out->nk = perm->nk;
  out->rep = perm->rep;
  out->on = true;
  return PQ1_OK;
}

pq1_status check_weights(const uint32_t* w_bits, const float* scales, int64_t N, int64_t K) {
  if (w_bits == nullptr || scales == nullptr) return PQ1_ERR_NULL;
  if (N < 1 || K < 128 || K % 128 != 0) return PQ1_ERR_SHAPE;
  if (N > kMaxDim || K > kMaxDim || N * (K / 32) > kMaxElems) return PQ1_ERR_SHAPE;
  if (!aligned16(w_bits) || !aligned16(scales)) return PQ1_ERR_ALIGN;
  return PQ1_OK;
}

pq1_status check_workspace(const pq1::GemvPlan& plan, void* workspace, size_t ws_bytes) {
  if (plan.nkt <= 1) return PQ1_OK;  // single K-tile: workspace unused
  if (workspace == nullptr) return PQ1_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PQ1_ERR_ALIGN;
  if (ws_bytes < plan.workspace_bytes()) return PQ1_ERR_ARG;
  return PQ1_OK;
}

}  // namespace

uint32_t pq1::test_flags() { return g_test_flags.load(std::memory_order_relaxed); }

extern "C" {

const char* pq1_status_str(pq1_status s) {
  switch (s) {
    case PQ1_OK: return "ok";
    case PQ1_ERR_NULL: return "a required pointer is NULL";
    case PQ1_ERR_SHAPE: return "invalid shape (size < 1, too large, or K not a multiple of the block)";
    case PQ1_ERR_ALIGN: return "an array is not 16-byte aligned (workspace: 256-byte)";
    case PQ1_ERR_PERM: return "invalid head permutation";
    case PQ1_ERR_ALIAS: return "an output overlaps an input";
    case PQ1_ERR_DEVICE: return "no HIP device, or the current device is not gfx950";
    case PQ1_ERR_LAUNCH: return "kernel launch failed";
    case PQ1_ERR_ARG: return "invalid enumerated argument, or workspace too small";
    case PQ1_ERR_SPLITK:
      return "a split-K wait gave up or the workspace bookkeeping was out of step (outputs NaN)";
  }
  return "unknown status";
}

int32_t pq1_abi_version(void) { return PQ1_ABI_VERSION; }

int32_t pq1_last_hip_error(void) { return g_last_hip_error; }

size_t pq1_gemv_workspace_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 128 || K % 128 != 0 || N > kMaxDim || K > kMaxDim) return 0;
  return pq1::gemv_workspace_bytes(N, K);
}

pq1_status pq1_rotate(const float* x, const float* signs, const pq1_perm* perm, void* x_rot,
                      int32_t out_dtype, int64_t M, int64_t K, void* stream) {
  if (x == nullptr || signs == nullptr || x_rot == nullptr) return PQ1_ERR_NULL;
  if (out_dtype != PQ1_F32 && out_dtype != PQ1_BF16 && out_dtype != PQ1_BF16_GEMM)
    return PQ1_ERR_ARG;
  if (M < 1 || K < pq1::kWhtBlock || K % pq1::kWhtBlock != 0) return PQ1_ERR_SHAPE;
  if (K > kMaxDim || M > kMaxDim || M * (K / pq1::kWhtBlock) > kMaxDim) return PQ1_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(signs) || !aligned16(x_rot)) return PQ1_ERR_ALIGN;
  pq1::Perm p;
  if (pq1_status st = check_perm(perm, K, &p); st != PQ1_OK) return st;
  const size_t out_bytes = static_cast<size_t>(M * K) * (out_dtype == PQ1_F32 ? 4 : 2);
  if (overlaps(x_rot, out_bytes, x, static_cast<size_t>(M * K) * 4) ||
      overlaps(x_rot, out_bytes, signs, static_cast<size_t>(K) * 4))
    return PQ1_ERR_ALIAS;
  if (pq1_status st = check_device(); st != PQ1_OK) return st;
  return launched(pq1::launch_rotate(x, signs, p, x_rot, out_dtype, M, K,
                                     static_cast<hipStream_t>(stream)));
}

pq1_status pq1_gemv_ex(const float* x_rot, const uint32_t* w_bits, const float* scales, float* y,
                       int64_t N, int64_t K, int32_t algo, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (x_rot == nullptr || y == nullptr) return PQ1_ERR_NULL;
  if (pq1_status st = check_weights(w_bits, scales, N, K); st != PQ1_OK) return st;
  if (!aligned16(x_rot) || !aligned16(y)) return PQ1_ERR_ALIGN;
  if (algo != PQ1_GEMV_AUTO && algo != PQ1_GEMV_LUT && algo != PQ1_GEMV_EXPAND)
    return PQ1_ERR_ARG;
  const pq1::GemvPlan plan = pq1::plan_gemv(N, K, algo, false);
  if (plan.nkt == 0) return PQ1_ERR_SHAPE;  // too many row blocks for a K split
  if (pq1_status st = check_workspace(plan, workspace, workspace_bytes); st != PQ1_OK) return st;
  const size_t yb = static_cast<size_t>(N) * 4;
  if (overlaps(y, yb, x_rot, static_cast<size_t>(K) * 4) ||
      overlaps(y, yb, w_bits, static_cast<size_t>(N) * (K / 8)) ||
      overlaps(y, yb, scales, static_cast<size_t>(N) * (K / 128) * 4))
    return PQ1_ERR_ALIAS;
  if (plan.nkt > 1) {
    const size_t wsb = plan.workspace_bytes();
    if (overlaps(workspace, wsb, y, yb) || overlaps(workspace, wsb, x_rot, static_cast<size_t>(K) * 4) ||
        overlaps(workspace, wsb, w_bits, static_cast<size_t>(N) * (K / 8)) ||
        overlaps(workspace, wsb, scales, static_cast<size_t>(N) * (K / 128) * 4))
      return PQ1_ERR_ALIAS;
  }
  if (pq1_status st = check_device(); st != PQ1_OK) return st;
  return launched(pq1::launch_gemv(plan, x_rot, w_bits, scales, y, N, K, workspace,
                                   static_cast<hipStream_t>(stream)));
}

pq1_status pq1_gemv(const float* x_rot, const uint32_t* w_bits, const float* scales, float* y,
                    int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  return pq1_gemv_ex(x_rot, w_bits, scales, y, N, K, PQ1_GEMV_AUTO, workspace, workspace_bytes,
                     stream);
}

pq1_status pq1_rotate_gemv(const float* x, const float* signs, const pq1_perm* perm,
                           const uint32_t* w_bits, const float* scales, float* y, int64_t N,
                           int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  if (x == nullptr || signs == nullptr || y == nullptr) return PQ1_ERR_NULL;
  if (pq1_status st = check_weights(w_bits, scales, N, K); st != PQ1_OK) return st;
  if (K % pq1::kWhtBlock != 0) return PQ1_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(signs) || !aligned16(y)) return PQ1_ERR_ALIGN;
  pq1::Perm p;
  if (pq1_status st = check_perm(perm, K, &p); st != PQ1_OK) return st;
  const pq1::GemvPlan plan = pq1::plan_gemv(N, K, PQ1_GEMV_LUT, true);
  if (plan.nkt == 0) return PQ1_ERR_SHAPE;  // too many row blocks for a K split
  if (pq1_status st = check_workspace(plan, workspace, workspace_bytes); st != PQ1_OK) return st;
  const size_t yb = static_cast<size_t>(N) * 4;
  if (overlaps(y, yb, x, static_cast<size_t>(K) * 4) ||
      overlaps(y, yb, signs, static_cast<size_t>(K) * 4) ||
      overlaps(y, yb, w_bits, static_cast<size_t>(N) * (K / 8)) ||
      overlaps(y, yb, scales, static_cast<size_t>(N) * (K / 128) * 4))
    return PQ1_ERR_ALIAS;
  if (plan.nkt > 1) {
    const size_t wsb = plan.workspace_bytes();
    if (overlaps(workspace, wsb, y, yb) || overlaps(workspace, wsb, x, static_cast<size_t>(K) * 4) ||
        overlaps(workspace, wsb, signs, static_cast<size_t>(K) * 4) ||
        overlaps(workspace, wsb, w_bits, static_cast<size_t>(N) * (K / 8)) ||
        overlaps(workspace, wsb, scales, static_cast<size_t>(N) * (K / 128) * 4))
      return PQ1_ERR_ALIAS;
  }
  if (pq1_status st = check_device(); st != PQ1_OK) return st;
  return launched(pq1::launch_rotate_gemv(plan, x, signs, p, w_bits, scales, y, N, K, workspace,
                                          static_cast<hipStream_t>(stream)));
}

size_t pq1_packed_bits_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 128 || K % 128 != 0 || N > kMaxDim || K > kMaxDim) return 0;
  return pq1::packed_bits_bytes(N, K);
}

size_t pq1_packed_scales_bytes_ex(int64_t N, int64_t K, int32_t scale_dtype) {
  if (N < 1 || K < 128 || K % 128 != 0 || N > kMaxDim || K > kMaxDim) return 0;
  if (scale_dtype != PQ1_SCALE_F32 && scale_dtype != PQ1_SCALE_F16) return 0;
  return pq1::packed_scales_bytes(N, K, scale_dtype);
}

size_t pq1_packed_scales_bytes(int64_t N, int64_t K) {
  return pq1_packed_scales_bytes_ex(N, K, PQ1_SCALE_F32);
}

pq1_status pq1_pack_weights_ex(const uint32_t* w_bits, const float* scales, int64_t N, int64_t K,
                               void* packed_bits, void* packed_scales, int32_t scale_dtype,
                               int64_t N_total, int64_t row0, void* stream) {
  if (packed_bits == nullptr || packed_scales == nullptr) return PQ1_ERR_NULL;
  if (scale_dtype != PQ1_SCALE_F32 && scale_dtype != PQ1_SCALE_F16) return PQ1_ERR_ARG;
  if (pq1_status st = check_weights(w_bits, scales, N, K); st != PQ1_OK) return st;
  if (N_total > kMaxDim || N_total * (K / 32) > kMaxElems || row0 < 0 || row0 + N > N_total)
    return PQ1_ERR_SHAPE;
  if (!aligned16(packed_bits) || !aligned16(packed_scales)) return PQ1_ERR_ALIGN;
  const size_t pb = pq1::packed_bits_bytes(N_total, K),
               ps = pq1::packed_scales_bytes(N_total, K, scale_dtype);
  const size_t wb = static_cast<size_t>(N) * (K / 8), sb = static_cast<size_t>(N) * (K / 128) * 4;
  if (overlaps(packed_bits, pb, w_bits, wb) || overlaps(packed_bits, pb, scales, sb) ||
      overlaps(packed_scales, ps, w_bits, wb) || overlaps(packed_scales, ps, scales, sb) ||
      overlaps(packed_bits, pb, packed_scales, ps))
    return PQ1_ERR_ALIAS;
  if (pq1_status st = check_device(); st != PQ1_OK) return st;
  return launched(pq1::launch_pack(w_bits, scales, N, K, packed_bits, packed_scales, scale_dtype,
                                   N_total, row0, static_cast<hipStream_t>(stream)));
}

pq1_status pq1_pack_weights_rows(const uint32_t* w_bits, const float* scales, int64_t N, int64_t K,
                                 void* packed_bits, float* packed_scales, int64_t N_total,
                                 int64_t row0, void* stream) {
  return pq1_pack_weights_ex(w_bits, scales, N, K, packed_bits, packed_scales, PQ1_SCALE_F32,
                             N_total, row0, stream);
}

pq1_status pq1_pack_weights(const uint32_t* w_bits, const float* scales, int64_t N, int64_t K,
                            void* packed_bits, float* packed_scales, void* stream) {
  return pq1_pack_weights_ex(w_bits, scales, N, K, packed_bits, packed_scales, PQ1_SCALE_F32, N,
                             0, stream);
}

pq1_status pq1_embed(const int32_t* tokens, int64_t M, const uint32_t* w_bits, const float* scales,
                     const float* signs, float* out, int64_t V, int64_t K, void* stream) {
  if (tokens == nullptr || signs == nullptr || out == nullptr) return PQ1_ERR_NULL;
  if (pq1_status st = check_weights(w_bits, scales, V, K); st != PQ1_OK) return st;
  if (K % pq1::kWhtBlock != 0 || M < 1 || M > kMaxDim || M * K > kMaxElems) return PQ1_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(tokens) & 3u) != 0 || !aligned16(signs) || !aligned16(out))
    return PQ1_ERR_ALIGN;
  const size_t ob = static_cast<size_t>(M) * K * 4;
  if (overlaps(out, ob, tokens, static_cast<size_t>(M) * 4) ||
      overlaps(out, ob, w_bits, static_cast<size_t>(V) * (K / 8)) ||
      overlaps(out, ob, scales, static_cast<size_t>(V) * (K / 128) * 4) ||
      overlaps(out, ob, signs, static_cast<size_t>(K) * 4))
    return PQ1_ERR_ALIAS;
  if (pq1_status st = check_device(); st != PQ1_OK) return st;
  return launched(pq1::launch_embed(tokens, w_bits, scales, signs, out, M, V, K,
                                    static_cast<hipStream_t>(stream)));
}

namespace {

// own_scratch: the workspace is the library's own counter region (no
// workspace argument; the pointer is fetched after validation).
pq1_status gemv_packed_common(bool fused, const float* xin, const float* signs,
                              const pq1_perm* perm, const void* pbits, const void* pscales,
                              int32_t scale_dtype, float* y, int64_t N, int64_t K,
                              void* workspace, size_t workspace_bytes, void* stream,
                              bool own_scratch = false) {
  if (xin == nullptr || y == nullptr || pbits == nullptr || pscales == nullptr)
    return PQ1_ERR_NULL;
  if (fused && signs == nullptr) return PQ1_ERR_NULL;
  if (scale_dtype != PQ1_SCALE_F32 && scale_dtype != PQ1_SCALE_F16) return PQ1_ERR_ARG;
  if (N < 1 || K < 128 || K % 128 != 0 || N > kMaxDim || K > kMaxDim ||
      N * (K / 32) > kMaxElems)
    return PQ1_ERR_SHAPE;
  if (fused && K % pq1::kWhtBlock != 0) return PQ1_ERR_SHAPE;
  if (!aligned16(xin) || !aligned16(y) || !aligned16(pbits) || !aligned16(pscales) ||
      (fused && !aligned16(signs)))
    return PQ1_ERR_ALIGN;
  pq1::Perm p;
  if (fused) {
    if (pq1_status st = check_perm(perm, K, &p); st != PQ1_OK) return st;
  }
  const pq1::GemvPlan plan = pq1::plan_gemv_packed(N, K, fused);
  if (plan.nkt == 0) return PQ1_ERR_SHAPE;
  if (own_scratch) {
    static_assert(pq1::kScratchBytes >= pq1::kCounterBytes, "scratch holds the counter region");
    if (plan.workspace_bytes() > pq1::kScratchBytes) return PQ1_ERR_SHAPE;
  } else if (pq1_status st = check_workspace(plan, workspace, workspace_bytes); st != PQ1_OK) {
    return st;
  }
  const size_t yb = static_cast<size_t>(N) * 4, xb = static_cast<size_t>(K) * 4;
  const size_t pb = pq1::packed_bits_bytes(N, K), ps = pq1::packed_scales_bytes(N, K, scale_dtype);
  if (overlaps(y, yb, xin, xb) || overlaps(y, yb, pbits, pb) || overlaps(y, yb, pscales, ps) ||
      (fused && overlaps(y, yb, signs, xb)))
    return PQ1_ERR_ALIAS;
  if (plan.nkt > 1 && !own_scratch) {
    const size_t wsb = plan.workspace_bytes();
    if (overlaps(workspace, wsb, y, yb) || overlaps(workspace, wsb, xin, xb) ||
        overlaps(workspace, wsb, pbits, pb) || overlaps(workspace, wsb, pscales, ps) ||
        (fused && overlaps(workspace, wsb, signs, xb)))
      return PQ1_ERR_ALIAS;
  }
  if (pq1_status st = check_device(); st != PQ1_OK) return st;
  if (own_scratch && plan.nkt > 1) {
    const hipError_t e = pq1::packed_scratch(static_cast<hipStream_t>(stream), &workspace);
    if (e != hipSuccess) return launched(e);
  }
  return launched(pq1::launch_gemv_packed(plan, fused, xin, signs, p, pbits, pscales, scale_dtype,
                                          y, N, K, workspace, static_cast<hipStream_t>(stream)));
}

}  // namespace

pq1_status pq1_gemv_packed(const float* x_rot, const void* packed_bits, const float* packed_scales,
                           float* y, int64_t N, int64_t K, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return gemv_packed_common(false, x_rot, nullptr, nullptr, packed_bits, packed_scales,
                            PQ1_SCALE_F32, y, N, K, workspace, workspace_bytes, stream);
}

pq1_status pq1_rotate_gemv_packed(const float* x, const float* signs, const pq1_perm* perm,
                                  const void* packed_bits, const float* packed_scales, float* y,
                                  int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  return gemv_packed_common(true, x, signs, perm, packed_bits, packed_scales, PQ1_SCALE_F32, y, N,
                            K, workspace, workspace_bytes, stream);
}

pq1_status pq1_gemv_packed_ex(const float* x_rot, const void* packed_bits,
                              const void* packed_scales, int32_t scale_dtype, float* y,
                              int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return gemv_packed_common(false, x_rot, nullptr, nullptr, packed_bits, packed_scales,
                            scale_dtype, y, N, K, workspace, workspace_bytes, stream);
}

pq1_status pq1_rotate_gemv_packed_ex(const float* x, const float* signs, const pq1_perm* perm,
                                     const void* packed_bits, const void* packed_scales,
                                     int32_t scale_dtype, float* y, int64_t N, int64_t K,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return gemv_packed_common(true, x, signs, perm, packed_bits, packed_scales, scale_dtype, y, N,
                            K, workspace, workspace_bytes, stream);
}

pq1_status pq1_rotate_gemv_packed_noalloc(const float* x, const float* signs,
                                          const pq1_perm* perm, const void* packed_bits,
                                          const void* packed_scales, int32_t scale_dtype, float* y,
                                          int64_t N, int64_t K, void* stream) {
  return gemv_packed_common(true, x, signs, perm, packed_bits, packed_scales, scale_dtype, y, N,
                            K, nullptr, 0, stream, true);
}

pq1_status pq1_gemm_ex(const uint16_t* x_rot_bf16, const uint32_t* w_bits, const float* scales,
                       float* y, int64_t M, int64_t N, int64_t K, int32_t x_layout,
                       void* stream) {
  if (x_rot_bf16 == nullptr || y == nullptr) return PQ1_ERR_NULL;
  if (x_layout != PQ1_X_ROW_MAJOR && x_layout != PQ1_X_GEMM_ORDER) return PQ1_ERR_ARG;
  if (pq1_status st = check_weights(w_bits, scales, N, K); st != PQ1_OK) return st;
  if (M < 1 || M > kMaxDim || M * K > kMaxElems || M * N > kMaxElems) return PQ1_ERR_SHAPE;
  if (K >= (int64_t{1} << 28)) return PQ1_ERR_SHAPE;  // 32-bit offsets in a tile's weights
  if (!aligned16(x_rot_bf16) || !aligned16(y)) return PQ1_ERR_ALIGN;
  const size_t yb = static_cast<size_t>(M) * N * 4;
  if (overlaps(y, yb, x_rot_bf16, static_cast<size_t>(M) * K * 2) ||
      overlaps(y, yb, w_bits, static_cast<size_t>(N) * (K / 8)) ||
      overlaps(y, yb, scales, static_cast<size_t>(N) * (K / 128) * 4))
    return PQ1_ERR_ALIAS;
  int cus = 0;
  if (pq1_status st = check_device(&cus); st != PQ1_OK) return st;
  return launched(pq1::launch_gemm(x_rot_bf16, x_layout == PQ1_X_GEMM_ORDER, w_bits, scales, y,
                                   M, N, K, cus, static_cast<hipStream_t>(stream)));
}

pq1_status pq1_gemm(const uint16_t* x_rot_bf16, const uint32_t* w_bits, const float* scales,
                    float* y, int64_t M, int64_t N, int64_t K, void* stream) {
  return pq1_gemm_ex(x_rot_bf16, w_bits, scales, y, M, N, K, PQ1_X_ROW_MAJOR, stream);
}

uint32_t pq1_set_test_flags(uint32_t flags) {
  return g_test_flags.exchange(flags, std::memory_order_relaxed);
}

}  // extern "C"
