/*
 * pq1.h -- C ABI of the Hadamard-rotated 1-bit GEMV/GEMM library for AMD
 * MI355X (gfx950).
 *
 * The library computes y = W . WHT(s (.) P x), the product the Pulse
 * ARCHITECTURE-SPEC Hadamard-fold notes describe for a model whose weights
 * had the rotation folded into them: the activation is head-permuted
 * (tiled -> grouped, only when the repetition factor is above one),
 * multiplied by an explicit +-1 sign vector, passed through a normalized
 * Sylvester-Walsh-Hadamard transform (block 1024, scale 1/32), and only then
 * multiplied by the 1-bit weight matrix.
 *
 * Weight format ("Inside the One-Bit Engine", station "A weight is one bit"
 * and the addressing lines of station "A token's embedding is 5,120
 * numbers"): row-major [N][K/32] uint32 words; weight (n, k) is bit
 * (k & 31) of word (k >> 5) of row n; a set bit is +1 and a clear bit is -1.
 * Scales: row-major [N][K/128] fp32; scale (n, g) multiplies the weights of
 * row n with k in [128 g, 128 g + 128).
 *
 * Conventions shared by every call:
 *  - Every array argument is a DEVICE pointer on the current HIP device,
 *    owned by the caller, contiguous and row-major, 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued on it; the call returns without waiting for the GPU.
 *    The library never synchronizes the host and never allocates device
 *    memory.  The only host-side state is a per-device architecture check;
 *    GEMV workspaces carry the split-K bookkeeping (see below).
 *  - Arguments are validated before anything is enqueued; on any error
 *    nothing is enqueued and no output is touched.  Nothing is truncated.
 *  - Outputs may not overlap inputs (PQ1_ERR_ALIAS).
 *  - Calls are thread-safe.  Two calls that share a workspace must be
 *    ordered on one stream.
 */
#ifndef PQ1_H
#define PQ1_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PQ1_ABI_VERSION 4

typedef enum {
    PQ1_OK = 0,
    PQ1_ERR_NULL = 1,    /* a required pointer is NULL                         */
    PQ1_ERR_SHAPE = 2,   /* a size is < 1, too large, or K is not a multiple of
                            1024 (rotate) / 128 (gemv, gemm)                    */
    PQ1_ERR_ALIGN = 3,   /* an array is not 16-byte aligned                     */
    PQ1_ERR_PERM = 4,    /* permutation with rep > 1 whose hd*nk*rep != K, or
                            hd not a multiple of 4, or a non-positive factor    */
    PQ1_ERR_ALIAS = 5,   /* an output overlaps an input                         */
    PQ1_ERR_DEVICE = 6,  /* no HIP device, or the current device is not gfx950  */
    PQ1_ERR_LAUNCH = 7,  /* the HIP runtime reported an error when launching    */
    PQ1_ERR_ARG = 8,     /* an enumerated argument has an unknown value, or the
                            workspace is too small                              */
    PQ1_ERR_SPLITK = 9,  /* never returned by a call: the code a binding reports
                            when a workspace's status word (below) is non-zero  */
} pq1_status;

/* Head permutation of the ssm_out input (Pulse ARCHITECTURE-SPEC, ssm_out
 * permutation paragraph).  The input is in the tiled layout [hd, nk, rep]
 * (axes listed fastest first: head n + nk*r holds hd contiguous values); the
 * output is the grouped layout [hd, rep, nk] (head r + rep*n).  Output head
 * r + rep*n is a copy of input head n + nk*r.  NULL or rep <= 1 means no
 * permutation. */
typedef struct {
    int32_t hd;
    int32_t nk;
    int32_t rep;
} pq1_perm;

/* Output element type of pq1_rotate.  PQ1_BF16_GEMM is bf16 stored in the K
 * order of the prefill GEMM's matrix-core operand (pq1_gemm_ex with
 * PQ1_X_GEMM_ORDER): inside every 32-wide K block, stored position
 * 8c + 2q + t (c, q < 4, t < 2) holds the element at offset 4c + q + 16t. */
enum { PQ1_F32 = 0, PQ1_BF16 = 1, PQ1_BF16_GEMM = 2 };

/* Layout of the bf16 activation of pq1_gemm_ex. */
enum { PQ1_X_ROW_MAJOR = 0, PQ1_X_GEMM_ORDER = 1 };

/* GEMV algorithm selector for pq1_gemv_ex. */
enum {
    PQ1_GEMV_AUTO = 0,    /* the library's choice (currently PQ1_GEMV_LUT)      */
    PQ1_GEMV_LUT = 1,     /* 16-entry signed-sum table per 4 inputs, one lookup
                             per 4 weights ("Inside the One-Bit Engine", station
                             "Four one-bit weights have only sixteen possible
                             answers")                                          */
    PQ1_GEMV_EXPAND = 2,  /* every bit expanded to +-1 in registers, fp32
                             partial per 128-group times its scale, wave-wide
                             reduction per row                                  */
};

/* Activation rotation: x_rot = WHT_1024(signs (.) P x) / 32 for every row.
 *   x      [M][K] fp32 input (read only).
 *   out_dtype  PQ1_F32, PQ1_BF16 or PQ1_BF16_GEMM (see above).
 *   signs  [K] fp32, every entry +1 or -1, indexed in the post-permutation
 *          order (Pulse ARCHITECTURE-SPEC: one sign vector per activation
 *          width, applied before the transform).
 *   perm   NULL, or the permutation above (applied first).
 *   x_rot  [M][K] output: fp32 (out_dtype PQ1_F32) or bfloat16 bit patterns
 *          (PQ1_BF16; each fp32 result rounded to nearest, ties to even).
 *   M >= 1, K >= 1024 and a multiple of 1024 (the transform block).
 * The transform is block-diagonal: each contiguous 1024-block of a row is
 * transformed on its own with the natural-order Sylvester matrix
 * H[i][j] = (-1)^popcount(i & j). */
pq1_status pq1_rotate(const float* x, const float* signs, const pq1_perm* perm,
                      void* x_rot, int32_t out_dtype, int64_t M, int64_t K,
                      void* stream);

/* Bytes of device workspace pq1_gemv / pq1_gemv_ex / pq1_rotate_gemv need
 * for an [N][K] weight matrix (0 for an invalid shape).
 * Layout: bytes [0, PQ1_GEMV_COUNTER_BYTES) hold the split-K bookkeeping
 * (the first 32 KB per-row-block arrival counters of the canonical layout,
 * which every call leaves zero; the rest a generation word and a "seen" word
 * per (band, K chunk) of the packed layout, which every call advances
 * together); the rest holds partial sums.  Before its first use a workspace
 * must be zero-filled by the caller.  Every call leaves the counter bytes in
 * a state the next call accepts and never reads a partial sum it has not
 * written, so one workspace can serve any sequence of calls (any shapes)
 * ordered on one stream, as long as each call's workspace_bytes is at least
 * pq1_gemv_workspace_bytes of its shape.  Calls that may overlap in time
 * (different streams) need different workspaces. */
#define PQ1_GEMV_COUNTER_BYTES 262144
size_t pq1_gemv_workspace_bytes(int64_t N, int64_t K);

/* Status word of a workspace: a uint32 at byte PQ1_GEMV_STATUS_OFFSET, inside
 * the counter region.  The packed-layout GEMVs OR these bits into it (they
 * never clear it; zero means no trouble since the caller last cleared it):
 *   PQ1_SPLITK_WAIT_GAVE_UP: a K chunk waited too long (2^16 polls) for K
 *     chunk 0 to zero its rows -- the GPU did not dispatch chunk 0 first,
 *     which nothing guarantees but which this library has never seen -- and
 *     added NaN instead of its partial sums;
 *   PQ1_SPLITK_OUT_OF_STEP: at a launch a generation word disagreed with its
 *     seen word (after a wait that gave up, or in a workspace that was not
 *     zero-filled); K chunk 0 set the band's outputs to NaN for that call and
 *     put the pair back in step, so the next call is correct.
 * Either way every kernel ends normally.  Reading the word needs the stream
 * to have finished the calls; the Python binding does that on request and
 * raises PQ1_ERR_SPLITK.  Clearing it (zero-filling the whole counter region
 * is always safe between calls) is the caller's. */
#define PQ1_GEMV_STATUS_OFFSET 261888
#define PQ1_SPLITK_WAIT_GAVE_UP 1u
#define PQ1_SPLITK_OUT_OF_STEP 2u

/* Decode GEMV (M = 1): y[n] = sum_k scale[n][k>>7] * (+-1)(n, k) * x_rot[k],
 * the product y = W x that the Pulse ARCHITECTURE-SPEC Hadamard-fold notes
 * ("Order" block) apply to the rotated activation, with the 1-bit weights and
 * per-128 scales of "Inside the One-Bit Engine", station "A weight is one
 * bit".  Unlike the bare (x, w, scales, y, N, K, stream) form, the call takes
 * a workspace: the K dimension is split over workgroups to fill the GPU, and
 * the split's partial sums and arrival counters live in caller-owned memory
 * (the library never allocates).
 *   x_rot      [K] fp32 rotated activation (output of pq1_rotate).
 *   w_bits     [N][K/32] uint32 packed weights (format above).
 *   scales     [N][K/128] fp32.
 *   y          [N] fp32 output (overwritten).
 *   workspace  device buffer of workspace_bytes >= pq1_gemv_workspace_bytes(N,
 *              K) bytes, 256-byte aligned, zeroed before its first use (see
 *              above).  PQ1_ERR_ARG if it is too small.
 *   K >= 128 and a multiple of 128; N >= 1.
 * Results do not depend on the order in which workgroups finish: the split-K
 * partial sums are added in K order. */
pq1_status pq1_gemv(const float* x_rot, const uint32_t* w_bits, const float* scales,
                    float* y, int64_t N, int64_t K, void* workspace,
                    size_t workspace_bytes, void* stream);
/* (When K is split -- K above 1024 for the rotate_gemv kernel and the
 * default plans -- N may have at most 8192 row blocks: 2,097,152 rows, or
 * 1,048,576 with PQ1_GEMV_EXPAND; larger shapes return PQ1_ERR_SHAPE.  The
 * packed-layout calls below have their own, larger limit.) */

/* pq1_gemv with an explicit algorithm (PQ1_GEMV_*).  Same arguments and
 * results; PQ1_ERR_ARG for an unknown algorithm. */
pq1_status pq1_gemv_ex(const float* x_rot, const uint32_t* w_bits, const float* scales,
                       float* y, int64_t N, int64_t K, int32_t algo,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Rotation and GEMV in a single launch, for one activation (M = 1):
 * y = W . WHT_1024(signs (.) P x) / 32.  Arguments as pq1_rotate (with
 * M = 1, output not materialized) and pq1_gemv; K a multiple of 1024.  Each
 * workgroup transforms the 1024-block it needs in shared memory. */
pq1_status pq1_rotate_gemv(const float* x, const float* signs, const pq1_perm* perm,
                           const uint32_t* w_bits, const float* scales, float* y,
                           int64_t N, int64_t K, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Band-interleaved ("packed") weights.  "Inside the One-Bit Engine" describes
 * repacking the 1-bit weights once at load time into a band-interleaved order
 * the vecmat kernel prefers.  Here the 64 rows of each band are interleaved
 * per 128-weight group so that a wave (one lane per row) reads contiguous
 * memory.  For N rows and K columns, nb = ceil(N / 64), G = K / 128:
 *   packed_bits   [nb][G][64] x 16 bytes: element (b, g, l) holds words
 *                 4g .. 4g+3 of row 64b + l of w_bits, each rotated left by
 *                 2 bits (zero when 64b+l >= N);
 *   packed_scales [nb][G][64] fp32 (or f16, see pq1_scale_dtype): element
 *                 (b, g, l) = scales[64b+l][g] (zero when 64b+l >= N).
 * The packed arrays carry exactly the same bits (rotated within each word:
 * the even nibbles then sit at bits 2-5 of each byte, which is where the
 * GEMV's table offsets are read) and, with fp32 scales, the same scales. */
size_t pq1_packed_bits_bytes(int64_t N, int64_t K);    /* 0 for an invalid shape */
size_t pq1_packed_scales_bytes(int64_t N, int64_t K);  /* fp32 scales; 0 for an invalid shape */

/* Storage type of packed_scales.  PQ1_SCALE_F16 is the weight format "Inside
 * the One-Bit Engine" ships (station on a token's embedding: a 5120-wide row
 * is 640 bytes of sign bits and 80 bytes of f16 scales, 720 bytes, 1.125 bits
 * per weight; the bits-per-weight table lists one-bit g128 at 1.125).  The
 * repack rounds each fp32 scale to the nearest f16, ties to even (magnitudes
 * that round above 65504 become infinities, small ones f16 subnormals or
 * zero); the GEMV widens it back to fp32 exactly and computes as with fp32
 * scales, so its result is the fp32-scale result for the rounded scales. */
typedef enum {
    PQ1_SCALE_F32 = 0,   /* 4 bytes per scale (the canonical scales' values)  */
    PQ1_SCALE_F16 = 1,   /* 2 bytes per scale, rounded to nearest even        */
} pq1_scale_dtype;

/* Bytes of packed_scales for the given storage type (0 for an invalid shape
 * or an unknown scale_dtype). */
size_t pq1_packed_scales_bytes_ex(int64_t N, int64_t K, int32_t scale_dtype);

/* Repack canonical weights (w_bits [N][K/32], scales [N][K/128]) into the
 * packed layout.  Outputs are caller-owned device buffers of the sizes above.
 * K >= 128, K % 128 == 0, N >= 1. */
pq1_status pq1_pack_weights(const uint32_t* w_bits, const float* scales, int64_t N, int64_t K,
                            void* packed_bits, float* packed_scales, void* stream);

/* Stacking: pack the N rows of one matrix into rows row0 .. row0+N-1 of a
 * packed matrix of N_total rows (the same K), whose packed_bits and
 * packed_scales are sized for N_total.  Matrices that take the same rotated
 * activation (ffn_gate and ffn_up: Pulse ARCHITECTURE-SPEC, per-weight
 * convention table) packed one after another are served by one
 * pq1_gemv_packed / pq1_rotate_gemv_packed launch over N_total rows, whose y
 * holds their outputs one after another.  Only the entries of rows
 * row0 .. row0+N-1 are written, plus zeros for rows >= N_total in the bands
 * those rows touch, so calls for disjoint row ranges do not disturb one
 * another.  row0 >= 0 and row0 + N <= N_total, else PQ1_ERR_SHAPE.
 * pq1_pack_weights(...) is the case row0 = 0, N_total = N. */
pq1_status pq1_pack_weights_rows(const uint32_t* w_bits, const float* scales, int64_t N, int64_t K,
                                 void* packed_bits, float* packed_scales, int64_t N_total,
                                 int64_t row0, void* stream);

/* pq1_pack_weights_rows with a choice of scale storage: packed_scales holds
 * pq1_packed_scales_bytes_ex(N_total, K, scale_dtype) bytes of fp32 or f16
 * scales (16-byte aligned).  An unknown scale_dtype gives PQ1_ERR_ARG.  Rows
 * packed into one matrix must all use the same scale_dtype. */
pq1_status pq1_pack_weights_ex(const uint32_t* w_bits, const float* scales, int64_t N, int64_t K,
                               void* packed_bits, void* packed_scales, int32_t scale_dtype,
                               int64_t N_total, int64_t row0, void* stream);

/* pq1_gemv on packed weights: y = W x_rot, same result definition, same
 * workspace rules.  When K > 1024 the K dimension is split over workgroups and
 * ceil(N / 64) x (K / 1024) must not exceed 28640 (about 360K rows at K =
 * 5120); larger shapes return PQ1_ERR_SHAPE.  The partial sums of
 * the K chunks are added into y with float atomics in arrival order, so the
 * last bits of y may differ from run to run (within the fp32 tolerance). */
pq1_status pq1_gemv_packed(const float* x_rot, const void* packed_bits,
                           const float* packed_scales, float* y, int64_t N, int64_t K,
                           void* workspace, size_t workspace_bytes, void* stream);

/* pq1_rotate_gemv on packed weights (one launch; K a multiple of 1024). */
pq1_status pq1_rotate_gemv_packed(const float* x, const float* signs, const pq1_perm* perm,
                                  const void* packed_bits, const float* packed_scales, float* y,
                                  int64_t N, int64_t K, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* pq1_gemv_packed / pq1_rotate_gemv_packed on packed weights whose scales are
 * stored as scale_dtype (the type they were packed with; an unknown value
 * gives PQ1_ERR_ARG).  PQ1_SCALE_F32 is exactly the calls above. */
pq1_status pq1_gemv_packed_ex(const float* x_rot, const void* packed_bits,
                              const void* packed_scales, int32_t scale_dtype, float* y,
                              int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                              void* stream);
pq1_status pq1_rotate_gemv_packed_ex(const float* x, const float* signs, const pq1_perm* perm,
                                     const void* packed_bits, const void* packed_scales,
                                     int32_t scale_dtype, float* y, int64_t N, int64_t K,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory or pass a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): pq1_rotate_gemv_packed_ex with the split-K counter region
 * taken from the library's own static device array (256 KB per GPU, held
 * until the process ends) instead of a workspace.  Same arguments otherwise,
 * same results, same shape limit (a shape whose split needs more
 * (band, K chunk) pairs than the region holds gives PQ1_ERR_SHAPE); it
 * allocates nothing.  The first call on a device zeroes the region with a
 * kernel enqueued on `stream`.  Every call on a GPU shares that GPU's region,
 * so calls that may overlap in time on one GPU (different streams or
 * threads) race and must not be made; calls ordered on one stream are fine,
 * whatever their shapes.  The region's status word is not reported: a
 * split-K failure shows only as NaN outputs. */
pq1_status pq1_rotate_gemv_packed_noalloc(const float* x, const float* signs,
                                          const pq1_perm* perm, const void* packed_bits,
                                          const void* packed_scales, int32_t scale_dtype, float* y,
                                          int64_t N, int64_t K, void* stream);

/* Prefill GEMM: Y[m][n] = sum_k scale[n][k>>7] * (+-1)(n, k) * X[m][k], the
 * same product as pq1_gemv (Pulse ARCHITECTURE-SPEC Hadamard-fold notes,
 * "Order" block; "Inside the One-Bit Engine", station "A weight is one bit")
 * for a block of M rotated activations, each rotated then rounded to bf16.
 *   x_rot_bf16  [M][K] bfloat16 bit patterns, row-major in natural K order
 *               (pq1_rotate with PQ1_BF16).
 *   w_bits, scales as pq1_gemv.
 *   y           [M][N] fp32 output (overwritten).
 * Products of bf16 activations with +-1 are exact; they are accumulated in
 * fp32 on the matrix cores per 128-wide K group and each group's sum is
 * multiplied by its fp32 scale.  M, N >= 1; K >= 128, a multiple of 128 and
 * below 2^28; M * K and M * N below 2^31 (else PQ1_ERR_SHAPE).  The result
 * does not depend on how the kernel splits the work (it is the same for any
 * device size). */
pq1_status pq1_gemm(const uint16_t* x_rot_bf16, const uint32_t* w_bits, const float* scales,
                    float* y, int64_t M, int64_t N, int64_t K, void* stream);

/* pq1_gemm with the activation's layout given: x_layout PQ1_X_ROW_MAJOR is
 * pq1_gemm; PQ1_X_GEMM_ORDER takes X in the GEMM K order (pq1_rotate with
 * PQ1_BF16_GEMM), which saves the kernel one byte permute per matrix-core
 * step when it expands the weights (both layouts run at about the same
 * rate).  Any other x_layout gives PQ1_ERR_ARG.  The K order inside a group
 * changes only the order of the fp32 additions. */
pq1_status pq1_gemm_ex(const uint16_t* x_rot_bf16, const uint32_t* w_bits, const float* scales,
                       float* y, int64_t M, int64_t N, int64_t K, int32_t x_layout,
                       void* stream);

/* Embedding lookup with the inverse rotation (Pulse ARCHITECTURE-SPEC,
 * Hadamard-fold notes: the table stores rotated rows; the lookup applies the
 * transform first, then the signs):
 *   out[m][k] = signs[k] * (WHT_1024(z_m) / 32)[k],
 *   z_m[k] = scales[r][k >> 7] * (bit k of row r of w_bits ? +1 : -1),  r = tokens[m].
 *   tokens   [M] int32 device array (4-byte aligned): rows of the table; an id
 *            outside [0, V) gives a row of NaNs (the table is not read).
 *   w_bits   [V][K/32], scales [V][K/128]: the table, in the weight layout.
 *   signs    [K] fp32, out [M][K] fp32 (16-byte aligned, not overlapping the
 *            inputs).  K a multiple of 1024, M * K < 2^31. */
pq1_status pq1_embed(const int32_t* tokens, int64_t M, const uint32_t* w_bits, const float* scales,
                     const float* signs, float* out, int64_t V, int64_t K, void* stream);

/* Static description of a status code (never NULL). */
const char* pq1_status_str(pq1_status s);

/* PQ1_ABI_VERSION of the loaded library. */
int32_t pq1_abi_version(void);

/* The last HIP error code the calling thread's most recent failed call saw
 * (0 if none); useful after PQ1_ERR_LAUNCH or PQ1_ERR_DEVICE. */
int32_t pq1_last_hip_error(void);

/* Tests of the failure handling only; 0 (the default) in any other use.
 * PQ1_TEST_WITHHOLD_PUBLISH makes K chunk 0 of the packed-layout GEMVs skip
 * its publish, so every other K chunk's bounded wait expires (each launch
 * then takes a fraction of a second and reports PQ1_SPLITK_WAIT_GAVE_UP;
 * the calls after it report PQ1_SPLITK_OUT_OF_STEP once and are then back in
 * step).  Process-wide; returns the previous flags. */
#define PQ1_TEST_WITHHOLD_PUBLISH 1u
uint32_t pq1_set_test_flags(uint32_t flags);

#ifdef __cplusplus
}
#endif

#endif /* PQ1_H */
