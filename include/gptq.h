/*
 * gptq.h — C ABI of the MI355X (gfx950) GPTQ layer quantizer.
 *
 * The library quantizes one linear layer W [d_out, d_in] (or a batch of independent
 * layers, e.g. the experts of a mixture-of-experts block) to a uniform 2..8-bit grid by
 * the GPTQ procedure:
 *
 *   minimise || W X - What X ||_F^2 over grid-restricted What
 *     ("04 — GPTQ: Hessian-Weighted Rounding, the OBS Lineage, and Why It Still Ships",
 *      section 1; "GPTQ Architecture, in depth", "The algorithm on one page")
 *
 * in four calls that follow the pages' split of the work:
 *   gptq_accumulate_hessian  H += 2 X^T X per calibration batch
 *   gptq_prepare_hinv        dead inputs, ActOrder, damping, U with H_p^-1 = U^T U
 *   gptq_quantize_layer      blocked column sweep with lazy trailing updates
 *   gptq_pack_int4           checkpoint tensors (qweight, qzeros, fp16 scales)
 *
 * Conventions shared by every call
 *   - All array arguments are DEVICE pointers owned by the caller.  The library never
 *     allocates or frees memory; scratch memory comes in through `workspace`, whose
 *     required size is returned by gptq_workspace_size().  Nothing is retained between
 *     calls.
 *   - Every call enqueues its kernels on `stream` and returns without waiting, except
 *     gptq_prepare_hinv, which waits for its own kernels to read the factorisation
 *     status.  Outputs are valid once the stream reaches the end of the call's work.
 *   - Arrays are dense row-major; "stride" arguments count ELEMENTS of the array's own
 *     type.  `batch` independent problems are addressed by the batch strides.
 *   - Errors are returned, never printed; on an error the outputs are unspecified.
 *     Argument errors are detected before anything is enqueued.
 *   - Calls on different streams that share a workspace race; calls on one stream do
 *     not.
 */
#ifndef GPTQ_MI355X_H
#define GPTQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPTQ_OK = 0,
  GPTQ_ERR_INVALID_ARG = -1, /* bad sizes, strides, null pointers or parameters          */
  GPTQ_ERR_NOT_SPD = -2,     /* the damped Hessian has no Cholesky factor                 */
  GPTQ_ERR_HIP = -3,         /* a HIP runtime call failed                                  */
  GPTQ_ERR_WORKSPACE = -4,   /* workspace missing or smaller than gptq_workspace_size()   */
  GPTQ_ERR_UNSUPPORTED = -5, /* valid request outside what this build implements          */
  GPTQ_ERR_TOO_LARGE = -6    /* problem exceeds the fixed scratch of the allocation-free
                                entry point (gptq_quantize_layer_noalloc)                  */
} gptq_status;

typedef enum { GPTQ_F32 = 0, GPTQ_BF16 = 1, GPTQ_F16 = 2 } gptq_dtype;

/* Quantizer knobs ("GPTQ Architecture, in depth", "The algorithm in code" and
 * "Groups, act-order and other knobs"; damping: "Same Ruler, Smarter Placement:
 * GPTQ", 1.6).
 *   bits          2..8; codes lie in [0, 2^bits - 1]
 *   group_size    -1: one grid per row, fitted once on the whole row; otherwise 16, 32,
 *                 64 or 128 dividing d_in: the grid of each group of consecutive
 *                 columns IN PROCESSING ORDER is refitted on the current (already
 *                 compensated) weights when the sweep reaches its first column
 *   block_size    columns per lazy batch; must be 128
 *   damp          lambda = damp * mean(diag H) is added to the diagonal (>= 0)
 *   act_order     nonzero: process columns by descending Hessian diagonal
 *   sym           0: asymmetric min-max grid, scale = (hi - lo) / maxq with
 *                 [lo, hi] = [min(0, min w), max(0, max w)], zero = rne(-lo / scale);
 *                 nonzero: symmetric grid, scale = max|w| / (2^(bits-1) - 1), zero fixed
 *                 at the middle level 2^(bits-1) (the grid of "Same Ruler, Smarter
 *                 Placement: GPTQ", 1.11, stored with an unsigned code); scales are never
 *                 below 1e-8 ("Groups, act-order and other knobs": symmetric or asymmetric)
 *   static_groups nonzero (with group_size > 0): groups are runs of group_size
 *                 consecutive ORIGINAL columns, each fitted once on the dead-zeroed W
 *                 before the sweep; every column is quantized on its original group's grid
 *                 wherever act_order puts it, and g_idx[c] = c / group_size ("Groups,
 *                 act-order and other knobs": static groups keep the scale reads of the
 *                 serving kernel contiguous)                                               */
typedef struct {
  int bits;
  int group_size;
  int block_size;
  float damp;
  int act_order;
  int sym;
  int static_groups;
} gptq_params;

/* Which call a workspace is sized for. */
typedef enum {
  GPTQ_WS_HESSIAN = 0,
  GPTQ_WS_PREPARE = 1,
  GPTQ_WS_QUANTIZE = 2,
  GPTQ_WS_W4A16_REPACK = 3,
  GPTQ_WS_W4A16 = 4
} gptq_ws_call;

/*
 * Hessian accumulation — "Same Ruler, Smarter Placement: GPTQ", 1.4 (H = 2 X X^T, the
 * same matrix for every output row) and "GPTQ Architecture, in depth", "The algorithm
 * in code" (accumulated over calibration batches).
 *
 * For every problem e < batch:
 *   H[e]        += 2 * X[e]^T X[e]          fp32, full symmetric [d_in, d_in]
 *   diag_key[e] += 2 * sum_t X[e][t,:]^2    fp64 [d_in]; the exact-to-fp64 diagonal,
 *                                           used for the dead-input test, the ActOrder
 *                                           order and the damping mean
 *   n_seen[e]   += n_tokens                 int64
 * X[e] is token-major [n_tokens, d_in] with row stride ldx (>= d_in) and batch stride
 * batch_stride_x; dtype bf16, fp16 or fp32 (products are exact in fp32, sums are fp32;
 * the fp64 key sums the same products in fp64).  H[e] starts at H + e*batch_stride_h
 * (>= d_in*d_in).  Zero H, diag_key and n_seen before the first batch.  n_tokens may be
 * 0 (no-op) and need not be a multiple of any tile.  Requires d_in % 8 == 0.
 */
gptq_status gptq_accumulate_hessian(int batch, int d_in, int64_t n_tokens, gptq_dtype x_dtype,
                                    const void* X, int64_t ldx, int64_t batch_stride_x,
                                    float* H, int64_t batch_stride_h, double* diag_key,
                                    int64_t* n_seen, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/*
 * Grouped Hessian accumulation — the same sums as gptq_accumulate_hessian for `batch`
 * problems whose calibration tokens lie in one token-major buffer X [total_tokens, d_in]
 * (row stride ldx), problem e owning rows token_offsets[e] .. token_offsets[e + 1] - 1: the
 * tokens a mixture-of-experts router sends to expert e ("GPTQ Architecture, in depth",
 * "Failure modes": experts that receive few tokens are starved, so their counts are
 * reported).  token_offsets: DEVICE int64 [batch + 1]; each range is clamped to [0,
 * total_tokens] (a decreasing pair is empty) and to its first max_tokens_per_problem rows,
 * which sizes the launch (gptq_workspace_size(GPTQ_WS_HESSIAN, batch, 0, d_in,
 * max_tokens_per_problem, ...)).  For every problem: H[e] += 2 X_e^T X_e, diag_key[e] +=
 * 2 sum x^2 (fp64), n_seen[e] += the number of rows accumulated (0 for a problem that got
 * no token: its H stays 0 and every input is then dead).  One launch per kernel covers
 * all problems.  Requires d_in % 8 == 0 and a 16-byte aligned X.
 */
gptq_status gptq_accumulate_hessian_grouped(int batch, int d_in, int64_t total_tokens,
                                            int64_t max_tokens_per_problem, gptq_dtype x_dtype,
                                            const void* X, int64_t ldx, const int64_t* token_offsets,
                                            float* H, int64_t batch_stride_h, double* diag_key,
                                            int64_t* n_seen, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream);

/*
 * Inverse-Hessian factor — "GPTQ Architecture, in depth", "The algorithm in code"
 * (dead inputs, act-order, damping) and "Same Ruler, Smarter Placement: GPTQ", 1.6,
 * 1.7 and 1.9.
 *
 * For every problem e:
 *   dead[c] = (diag_key[c] == 0)            uint8 [d_in]; such inputs get H_cc = 1
 *   perm    = columns by descending key (dead inputs count as key 1), ties by ascending
 *             index; the identity when act_order == 0            int32 [d_in]
 *   H_p     = H[perm][:, perm] with diagonal key[perm] + lambda,
 *             lambda = damp * mean(key)  (key after the dead-input fix, fp64)
 *   U       = the upper-triangular factor with positive diagonal and H_p^-1 = U^T U,
 *             fp32 [d_in, d_in] in processing (permuted) order; the strictly lower part
 *             is written as zero.
 * The off-diagonal of H_p comes from the fp32 H (only its lower triangle is read); the
 * diagonal from diag_key.  H is not modified.  Computed through H_p = Ut Ut^T (Ut upper:
 * the Cholesky factor of the index-reversed H_p) and U = Ut^-1; positive-diagonal
 * factors are unique, so this is the same U as the pages' chol / cholesky_inverse /
 * chol route.  Returns GPTQ_ERR_NOT_SPD (after waiting for the stream) when a pivot is
 * not positive or not finite; the caller may retry with a larger damp.
 * Requires d_in % 128 == 0.
 * For one to three problems per call, parts of the factorisation and of the inverse run
 * on two streams that the library creates per device (kept for the life of the process),
 * forked from `stream` with events and joined back into it before the call returns; where
 * the process's other streams already hold the device's hardware queues, those parts run
 * serialized with the rest and take longer, with the same results.
 */
gptq_status gptq_prepare_hinv(int batch, int d_in, const float* H, int64_t batch_stride_h,
                              const double* diag_key, const gptq_params* p, float* U,
                              int64_t batch_stride_u, int32_t* perm, uint8_t* dead,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Column sweep — "Same Ruler, Smarter Placement: GPTQ", 1.5 (Steps 1-3), 1.7 (rows of
 * U), 1.8 (lazy batch update, block 128); "GPTQ Architecture, in depth", "The algorithm
 * in code" (min-max grid, in-block updates, lazy update, undoing the permutation).
 *
 * For every problem e, with W_p = W[:, perm] in fp32 and dead columns zeroed:
 *   for each column j in processing order:
 *     at a group start (not with static groups): the grid of the params above is fitted
 *       per row on the current values of the group's columns
 *     code = clamp(rne(W_p[r, j] / scale) + zero, 0, maxq)
 *     err  = (W_p[r, j] - scale * (code - zero)) / U[j, j]
 *     W_p[r, later columns of the block] -= err * U[j, later columns of the block]
 *   after each block of 128 columns: W_p[:, later] -= Err_block @ U[block, later]
 * Outputs (rne = round half to even):
 *   codes  uint8 [d_out, d_in] in ORIGINAL column order (batch stride d_out*d_in)
 *   scales fp32 [n_groups, d_out], zeros uint8 [n_groups, d_out]; n_groups = d_in /
 *          group_size, or 1 per row; group g holds processing positions [g*gs, (g+1)*gs),
 *          or original columns [g*gs, (g+1)*gs) with static groups
 *   g_idx  int32 [d_in]: group of each original column (0 per row)
 * W is bf16, fp16 or fp32 with row stride ldw and batch stride batch_stride_w; U, perm
 * and dead are the outputs of gptq_prepare_hinv (U batch stride batch_stride_u).
 * Requires d_in % 128 == 0, d_out >= 1.
 */
gptq_status gptq_quantize_layer(int batch, int d_out, int d_in, gptq_dtype w_dtype, const void* W,
                                int64_t ldw, int64_t batch_stride_w, const float* U,
                                int64_t batch_stride_u, const int32_t* perm, const uint8_t* dead,
                                const gptq_params* p, uint8_t* codes, float* scales,
                                uint8_t* zeros, int32_t* g_idx, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * Allocation-free variant of gptq_quantize_layer, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and kernels as gptq_quantize_layer, without the
 * workspace: the call's scratch (per problem: fp32 working weights and errors, codes in
 * processing order, 9 bytes per weight, plus the inverse permutation) lives in a fixed
 * device array of GPTQ_NOALLOC_SCRATCH_BYTES (64 MiB) inside the library, one per GPU,
 * held until the process ends; the call itself allocates and frees nothing.  A problem
 * that needs more (about 7.4 million weights over all problems of the batch) is rejected
 * with GPTQ_ERR_TOO_LARGE before anything is enqueued.  The array's address is looked up
 * once per device, on the first call there.  Every call on one GPU shares that GPU's
 * array, which keeps the last call's contents: calls that overlap in time on one GPU
 * (different streams, or different host threads) race; calls in order on one stream do
 * not.  Nothing in the array needs to start at zero.  The timing hook does not bracket
 * this variant's kernels.
 */
#define GPTQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gptq_status gptq_quantize_layer_noalloc(int batch, int d_out, int d_in, gptq_dtype w_dtype,
                                        const void* W, int64_t ldw, int64_t batch_stride_w,
                                        const float* U, int64_t batch_stride_u,
                                        const int32_t* perm, const uint8_t* dead,
                                        const gptq_params* p, uint8_t* codes, float* scales,
                                        uint8_t* zeros, int32_t* g_idx, hipStream_t stream);

/*
 * Checkpoint packing — "04 — GPTQ: ...", section 8, and "GPTQ Architecture, in
 * depth", "Packing, tooling and serving": eight 4-bit values per int32, element k in
 * bits [4k, 4k + 4).
 *   qweight    int32 [d_in/8, d_out]       qweight[i, o] = sum_k codes[o, 8i + k] << 4k
 *   qzeros     int32 [n_groups, d_out/8]   qzeros[g, i]  = sum_k zeros[g, 8i + k] << 4k
 *   scales_f16 fp16 bits [n_groups, d_out] round-to-nearest-even of scales
 * codes / scales / zeros as written by gptq_quantize_layer (values < 16; 3-bit codes are
 * stored in nibbles too).  Batch strides are the dense sizes of each array.
 * Requires d_in % 8 == 0 and d_out % 8 == 0.  Values are masked to their low 4 bits;
 * no range check is made.
 */
gptq_status gptq_pack_int4(int batch, int d_out, int d_in, int n_groups, const uint8_t* codes,
                           const float* scales, const uint8_t* zeros, int32_t* qweight,
                           int32_t* qzeros, uint16_t* scales_f16, hipStream_t stream);

/*
 * Serving layout for the W4A16 product — "Same Ruler, Smarter Placement: GPTQ", 1.9 (with
 * act-order the weight columns are permuted and the activations are permuted the same way
 * at inference time) and "GPTQ Architecture, in depth", "Groups, act-order and other
 * knobs" (groups formed in permuted order scatter the scale reads).
 *
 * For every problem e < batch (qweight and g_idx as written by gptq_pack_int4 and
 * gptq_quantize_layer, batch strides the dense sizes):
 *   order[e]     int32 [d_in]: the inputs sorted by group, g_idx ascending, ties by
 *                ascending input index (the position of input c is g_idx[c] * gs + the
 *                number of earlier inputs of its group, gs = d_in / n_groups)
 *   qweight_s[e] int32 [d_in/8, d_out]: qweight with its inputs in that order (nibble t of
 *                word i holds input order[8 i + t])
 * Every group must have exactly gs members and every g_idx lie in [0, n_groups); the
 * call waits for its kernels to read that check and returns GPTQ_ERR_INVALID_ARG
 * otherwise (outputs then unspecified).  workspace: at least
 * gptq_workspace_size(GPTQ_WS_W4A16_REPACK, ...) bytes of device memory (a flag).
 * Requires d_out % 8 == 0, d_in % 8 == 0 and n_groups dividing d_in.  When g_idx[c] = c /
 * gs already (static groups, or no act-order), order is the identity and qweight_s equals
 * qweight: gptq_w4a16_matmul then takes the checkpoint's qweight with order = NULL.
 */
gptq_status gptq_w4a16_repack(int batch, int d_out, int d_in, int n_groups, const int32_t* qweight,
                              const int32_t* g_idx, int32_t* qweight_s, int32_t* order,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * W4A16 product — "GPTQ Architecture, in depth", "Packing, tooling and serving": 4-bit
 * weights stay packed and are dequantized in registers right before the product with
 * 16-bit activations (decode is bound by reading the weights):
 *   Y[r, o] = sum_c X[r, c] * scale[g_idx[c], o] * (code[o, c] - zero[g_idx[c], o])
 * X [m, d_in] bf16 or fp16 bits, row stride ldx (>= d_in); Y fp32 [m, d_out], row stride
 * ldy (>= d_out, a multiple of 4, Y 16-byte aligned).  qweight_s / order from
 * gptq_w4a16_repack (order = NULL: qweight_s is in input order and g_idx[c] = c / gs);
 * qzeros int32 [n_groups, d_out/8] and scales_f16 [n_groups, d_out] as written by
 * gptq_pack_int4.  The codes enter 16-bit matrix-core products exactly; the group's scale
 * and zero are applied in fp32 once per group (sums in fp32).  Rows are processed 16 at a
 * time.  workspace: gptq_workspace_size(GPTQ_WS_W4A16, batch = 1, d_out, d_in,
 * n_tokens_hint = m, p with the group size) bytes (K-split partial sums; 256 when unsplit).
 * Requires m >= 1, d_out % 8 == 0, d_in % 128 == 0, a group size gs = d_in / n_groups of
 * 32, 64 or 128, or n_groups = 1 (one grid per row), and qweight_s 16-byte aligned.
 */
gptq_status gptq_w4a16_matmul(int m, int d_out, int d_in, int n_groups, gptq_dtype x_dtype,
                              const void* X, int64_t ldx, const int32_t* qweight_s,
                              const int32_t* order, const int32_t* qzeros,
                              const uint16_t* scales_f16, float* Y, int64_t ldy, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace the given call needs (0 on invalid arguments).  For
 * GPTQ_WS_HESSIAN `d_out` is ignored and `n_tokens_hint` is the largest n_tokens per call
 * (it only sizes the split over tokens); for GPTQ_WS_W4A16 `n_tokens_hint` is the number
 * of activation rows m and p->group_size the group size (-1: one grid per row); for the
 * other calls it is ignored. */
size_t gptq_workspace_size(gptq_ws_call which, int batch, int d_out, int d_in,
                           int64_t n_tokens_hint, const gptq_params* p);

/* Measurement hook for the kernels the roofline figures are quoted on.
 *   GPTQ_TIME_SYRK       the Hessian SYRK kernel of gptq_accumulate_hessian (the matrix-core
 *                        kernel for bf16/fp16 inputs, the vector-ALU kernel for fp32 inputs)
 *   GPTQ_TIME_LAZY_GEMM  every lazy trailing-update product of gptq_quantize_layer
 *   GPTQ_TIME_SWEEP      every 128-column sweep kernel of gptq_quantize_layer
 *   GPTQ_TIME_PACK       the packing kernels of one gptq_pack_int4 call (one pair per call)
 *   GPTQ_TIME_W4A16      the kernels of one gptq_w4a16_matmul call (one pair per call)
 * gptq_timing_enable(mask) times the classes whose bit (1 << class) is set in mask (0: none,
 * -1: all): every launch of such a class is bracketed by a pair of HIP events recorded on
 * the call's stream immediately around it (each pair adds a few microseconds between
 * launches, so a class left unset costs nothing).  gptq_timing_read waits for the recorded
 * events of one class, returns their summed elapsed milliseconds and the number of
 * bracketed launches since the previous read of that class, and forgets them.  Events are
 * created by the library on first use and reused; the hook is process-wide and not meant
 * for concurrent callers.  Returns GPTQ_ERR_INVALID_ARG for an unknown class or null
 * outputs. */
typedef enum {
  GPTQ_TIME_SYRK = 0,
  GPTQ_TIME_LAZY_GEMM = 1,
  GPTQ_TIME_SWEEP = 2,
  GPTQ_TIME_PACK = 3,
  GPTQ_TIME_W4A16 = 4
} gptq_timed_kernel;
gptq_status gptq_timing_enable(int mask);
gptq_status gptq_timing_read(gptq_timed_kernel which, double* total_ms, int64_t* launches);

/* Static description of a status code. */
const char* gptq_status_string(gptq_status s);

/* Library version, "major.minor.patch". */
const char* gptq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_MI355X_H */
