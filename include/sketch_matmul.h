/*
 * sketch_matmul.h - C ABI of the sketched-weight matrix multiply for AMD
 * Instinct MI355X (gfx950).
 *
 * The method ("SpaLLM: Unified Compressive Adaptation of Large Language Models
 * with Sketching", section 2.2, Eq. (1), and "Sketch to Adapt: Fine-Tunable
 * Sketches for Efficient LLM Adaptation", reply W2 on sub-rows) stores each
 * weight row of an n x d layer as gpr contiguous groups of G = d / gpr columns.
 * Every (row, group) owns a lookup table of k = 2^b values and every weight
 * stores a b-bit index into its group's table:
 *
 *     W[i][j] = lut[i][j / G][idx[i][j]]                         (dequantise)
 *     Y[t][i] = sum_j X[t][j] * W[i][j]                          (forward)
 *     dX[t][j] = sum_i dY[t][i] * W[i][j]                        (input grad)
 *     dLUT[i][g][c] = sum_{j in g, idx[i][j] == c} sum_t dY[t][i] * X[t][j]
 *                                                                (table grad,
 *                     corrected Eq. (6) of the Sketch to Adapt discussion)
 *
 * Data layout (all row-major, all pointers are DEVICE pointers):
 *   idx_packed  uint8 [n][d*b/8]   row i's indices as one little-endian
 *                                  bitstream: index j occupies bits
 *                                  b*j .. b*j+b-1, stream bit p is bit p%8 of
 *                                  byte p/8 (b=4: low nibble = even column;
 *                                  b=3: contiguous 3-bit stream).
 *   lut         [n][gpr][2^b]      table values, dtype lut_dtype.
 *   X           [m][d]             activations, dtype x_dtype.
 *   Y           [m][n]             forward output, dtype x_dtype, rounded to
 *                                  nearest-even from an fp32 accumulator.
 *   dY          [m][n]             output gradient, dtype io_dtype.
 *   dX          [m][d]   fp32      input gradient.
 *   dLUT        [n][gpr][2^b] fp32 table gradient.
 *
 * Supported shapes: b in {2,3,4}; gpr >= 1 with d % gpr == 0 and
 * (d / gpr) % 32 == 0; n >= 1; m >= 0 (m == 0 is a no-op that returns OK).
 * Supported dtype pairs (x_dtype, lut_dtype): (F32,F32) fp32 path with fp32
 * products; (F16,F16), (BF16,F16), (F16,BF16), (BF16,BF16) matrix-core path
 * whose operands are in the lut dtype (activations are converted to it) with
 * fp32 accumulation. The table gradient's dY^T X product always uses the
 * activations' own dtype.
 *
 * Range of the (BF16, F16) pair: f16 holds a far narrower range than bf16,
 * so every token row of X (forward) or dY (dX) whose largest magnitude M
 * lies outside [2^-2, 2^16) is multiplied by a power of two 2^-e before the
 * conversion, with e = floor(log2 M) - 14 clamped to [-126, 113] (so that
 * M 2^-e lands in [2^14, 2^15)), and the fp32 results of that row are
 * multiplied by 2^e afterwards; rows inside the window are converted as they
 * are (e = 0). Both steps are exact. After them every bf16 value of the row
 * at or above 2^-17 (in the scaled row) converts to f16 exactly, and a
 * smaller one with an absolute error below 2^-23 M, for any finite bf16
 * input; infinities and NaNs propagate. The exponents come from a pre-pass
 * into the workspace (forward GEMM, dX, and a decode that reads its
 * activations per slot instead of staging them in LDS) or are found inside
 * the decode kernel. The decode stages them when m * d <= 32768, and when
 * m < 8, m * d <= 49152, n <= 4096 and the block's tables, activations and
 * partial sums fit in 160 KB of LDS.
 *
 * Alignment: every pointer must be 16-byte aligned.
 *
 * Ownership and threading: the caller allocates and owns every buffer; the
 * library never allocates or frees device memory and, apart from
 * sketch_matmul_bwd_noalloc's static scratch array, keeps none and holds no
 * mutable global state, so calls are thread-safe. Work is enqueued on `stream`
 * (NULL = the default stream) and runs asynchronously; no call synchronises.
 *
 * Errors: argument checks run on the host before anything is launched; a
 * failed check returns its status and launches nothing. A launch failure
 * returns SKM_EHIP. Device-side faults surface at the caller's next
 * synchronisation of `stream`.
 */
#ifndef SKETCH_MATMUL_H
#define SKETCH_MATMUL_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SKM_F32 = 0,
  SKM_F16 = 1,
  SKM_BF16 = 2
} skm_dtype;

typedef enum {
  SKM_OK = 0,
  SKM_EINVAL = -1,        /* bad size, bit width, group count or NULL pointer */
  SKM_EUNSUPPORTED = -2,  /* dtype combination not provided                   */
  SKM_EALIGN = -3,        /* a pointer is not 16-byte aligned                  */
  SKM_EWORKSPACE = -4,    /* workspace smaller than the size query returns      */
  SKM_EHIP = -5,          /* the HIP runtime reported a launch error           */
  SKM_EALIAS = -6         /* an output buffer overlaps an input buffer         */
} skm_status;

/*
 * Forward pass Y = X * W^T (SpaLLM abstract and section 2.3: one compressed
 * matrix multiplication per layer; W is never materialised).
 *   X          [m][d] x_dtype     idx_packed [n][d*b/8]   lut [n][gpr][2^b]
 *   Y          [m][n] x_dtype (written, must not overlap any input)
 * workspace/workspace_bytes: device scratch of at least
 * sketch_matmul_fwd_workspace(...) bytes, 16-byte aligned, not overlapping
 * any other buffer; may be NULL when that size is 0 (every dtype pair except
 * (BF16, F16), and that pair's decode-sized calls that stage their
 * activations, see "Range" above). It
 * holds the row exponents of X (see "Range" above) during the call only.
 * Decode-sized m streams the indices once; larger m runs a tiled matrix-core
 * GEMM. Returns SKM_OK or an error status (see above).
 */
int sketch_matmul_fwd(const void* X, int x_dtype,
                      const uint8_t* idx_packed,
                      const void* lut, int lut_dtype,
                      int64_t m, int64_t n, int64_t d, int b, int gpr,
                      void* Y, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* Bytes of device workspace sketch_matmul_fwd needs for these sizes (0 for
 * invalid arguments, which the call itself then rejects). */
size_t sketch_matmul_fwd_workspace(int64_t m, int64_t n, int64_t d, int b, int gpr,
                                   int x_dtype, int lut_dtype);

/*
 * Forward pass with one table set per token, over one shared index stream
 * (SpaLLM section 2.3, multiple adapters: each adapter is a set of tables in
 * the same format over the frozen mapping, so requests of different tasks can
 * share a batch):
 *   luts     [n_sets][n][gpr][2^b] lut_dtype   (set s at luts + s*n*gpr*2^b)
 *   lut_set  [m] int32 (device): token t uses set lut_set[t]; values outside
 *            [0, n_sets) are clamped to that range
 *   Y[t][i] = sum_j X[t][j] * luts[lut_set[t]][i][j/G][idx[i][j]]
 * Decode-sized batches (1 <= m <= 16, tables of a 16-row block within the
 * decode limit) with a 16-bit dtype pair; other sizes, the fp32 pair and, for
 * (BF16, F16), rows of more than 32768 columns with one token (or with more
 * than 8 tokens and more than 128 table entries per row) return
 * SKM_EUNSUPPORTED. Row exponents of the (BF16, F16) pair are found inside the
 * kernel, so no workspace is needed. The index stream is read from memory once
 * and each set that some token uses adds its tables. Table lookups: from two
 * tokens on, with n_sets >= 2 (any n_sets for (BF16, F16)), when at most 224
 * table entries per row (gpr * 2^b) are used, or at most 128 when more than 8
 * sets can occur (min(m, n_sets) > 8), the tables of all sets in use are
 * interleaved in LDS and one lookup serves up to 8 sets; n_sets == 1 with the
 * other pairs, and one token (m == 1, its row staged for (BF16, F16)), run the
 * single-set forward on that set (read from lut_set on the device, so the
 * results equal sketch_matmul_fwd's on that set); otherwise each set in use takes one
 * round of lookups (one per 32768 / d of its tokens when more of them than
 * that share the set). lut_set must
 * be 4-byte aligned, the other pointers 16-byte aligned; Y must not overlap
 * any input. m == 0 returns OK.
 */
int sketch_matmul_fwd_multi(const void* X, int x_dtype,
                            const uint8_t* idx_packed,
                            const void* luts, int lut_dtype,
                            const int32_t* lut_set, int n_sets,
                            int64_t m, int64_t n, int64_t d, int b, int gpr,
                            void* Y, hipStream_t stream);

/*
 * Backward pass (the mapping is frozen, SpaLLM section 2.3, so there is no
 * index gradient):
 *   dX   = dY * W                      [m][d] fp32, NULL = skip
 *   dLUT = table gradient (see top)    [n][gpr][2^b] fp32, NULL = skip;
 *          accumulate == 0 overwrites dLUT, accumulate == 1 adds to it.
 *   dY [m][n] and X [m][d] are in io_dtype; X may be NULL when dLUT is NULL.
 * workspace/workspace_bytes: device scratch of at least
 * sketch_matmul_bwd_workspace(...) bytes, 16-byte aligned, not overlapping
 * any other buffer (may be NULL when that is 0). It holds, during the call
 * only: with (BF16, F16), the row exponents of dY; and, when the table
 * gradient's grid of (128-row block, group) pairs has fewer than 256 blocks
 * (e.g. 4096 rows in one group), one partial dLUT per (column range, token
 * range) the gradient is split into, at most 6 MiB in all, added in range
 * order at the end (deterministic; no atomics).
 * Gradients are sums over the columns that share an entry (chain rule of the
 * corrected Eq. (6)), not averages. With m == 0 and accumulate == 0 the
 * requested gradients are written as zeros.
 */
int sketch_matmul_bwd(const void* dY, const void* X, int io_dtype,
                      const uint8_t* idx_packed,
                      const void* lut, int lut_dtype,
                      int64_t m, int64_t n, int64_t d, int b, int gpr,
                      float* dX,
                      float* dLUT, int accumulate,
                      void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * sketch_matmul_bwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving or
 * training loops, harnesses that forbid allocation). Same arguments, results
 * and errors as sketch_matmul_bwd, whose kernels it runs; the workspace is a
 * library-owned scratch array of 8 MiB per GPU (a static device array, held
 * until the process ends; its address is looked up once per device on the
 * first call). Sizes whose sketch_matmul_bwd_workspace(...) exceeds 8 MiB
 * return SKM_EWORKSPACE (the need is 4 bytes per token with (BF16, F16),
 * rounded up to 256, plus at most 6 MiB of split table-gradient partials, so
 * every call with up to 524288 tokens fits). Allocates nothing. Calls that overlap in time on one GPU (several
 * host threads, or streams running concurrently) share that GPU's array and
 * race; serialise them. Nothing from an earlier call is read back (every
 * scratch entry a call reads was written by that call).
 */
int sketch_matmul_bwd_noalloc(const void* dY, const void* X, int io_dtype,
                              const uint8_t* idx_packed,
                              const void* lut, int lut_dtype,
                              int64_t m, int64_t n, int64_t d, int b, int gpr,
                              float* dX, float* dLUT, int accumulate,
                              hipStream_t stream);

/* Bytes of device workspace sketch_matmul_bwd needs for these sizes (>= 0). */
size_t sketch_matmul_bwd_workspace(int64_t m, int64_t n, int64_t d, int b, int gpr,
                                   int io_dtype, int lut_dtype);

/*
 * Dequantise W[i][j] = lut[i][j/G][idx[i][j]] into a dense [n][d] array of
 * lut_dtype (SpaLLM Eq. (1) with groups per row). A checking aid: the matmul
 * entry points never build W.
 */
int sketch_dequant(const uint8_t* idx_packed, const void* lut, int lut_dtype,
                   int64_t n, int64_t d, int b, int gpr,
                   void* W, hipStream_t stream);

/*
 * Unpack the b-bit index stream into one uint8 per weight: idx [n][d].
 * A checking aid for the bit layout described at the top of this file.
 */
int sketch_unpack_indices(const uint8_t* idx_packed, int64_t n, int64_t d, int b,
                          uint8_t* idx, hipStream_t stream);

/*
 * Sketch construction, the step before the matmul (SpaLLM section 2.2,
 * "Weighted Lloyd's algorithm for learning sketched parameters" and
 * "Learning the sketching matrix"; Sketch to Adapt, reply to Concern 1).
 * From a layer's dense weights W [n][d] fp32 and sample inputs X_s [s][d] of
 * the layer, with H = X_s^T X_s (damped so that it is invertible; the caller
 * chooses the damping) and the upper-triangular factor U of its inverse,
 * H^-1 = U^T U ([d][d] fp32, row-major; entries below the diagonal are not
 * read):
 *   1. sketch_column_weights: h[j] = 1 / [H^-1]_jj = 1 / sum_{k<=j} U[k][j]^2
 *   2. sketch_lloyd: the table of each (row i, group g) holds the 2^b
 *      centroids of weighted Lloyd's algorithm over W[i][j], j in g, weight
 *      h[j]. Start: centroid r at lo + (r + 1/2) (hi - lo) / 2^b, lo and hi
 *      the group's smallest and largest weight. Each iteration assigns every
 *      weight to its nearest centroid (ties to the lower index) and moves
 *      each centroid to the weighted mean of its weights (a centroid with no
 *      weights stays); at most `iters` iterations, fewer when the centroids
 *      stop changing. Written to lut [n][gpr][2^b] in lut_dtype (F32, F16 or
 *      BF16, rounded to nearest even).
 *   3. sketch_map: columns j = 0 .. d-1 in order; weight j of every row goes
 *      to the nearest entry q of its group's table (ties to the lower index,
 *      the table as stored in lut_dtype) and its error is spread over the
 *      later columns: err = (w_j - q) / U[j][j], w_j' -= err * U[j][j'] for
 *      j' > j (the update of Frantar et al., GPTQ). Writes idx_packed in the
 *      layout above. W is overwritten with the compensated weights (it is the
 *      working buffer). workspace: sketch_map_workspace(n) bytes. U must
 *      have a positive diagonal (a Cholesky factor does).
 * All arithmetic is fp32. Shapes as for the matmul (b in {2,3,4}, d % gpr ==
 * 0, (d / gpr) % 32 == 0); d <= 2^20, and n <= 2^22 for sketch_map. Pointers
 * 16-byte aligned; outputs must
 * not overlap inputs (SKM_EALIAS).
 */
int sketch_column_weights(const float* U, int64_t d, float* h, hipStream_t stream);

int sketch_lloyd(const float* W, const float* h, int64_t n, int64_t d, int b, int gpr, int iters,
                 void* lut, int lut_dtype, hipStream_t stream);

size_t sketch_map_workspace(int64_t n);

int sketch_map(float* W, const float* U, const void* lut, int lut_dtype,
               int64_t n, int64_t d, int b, int gpr,
               uint8_t* idx_packed, void* workspace, size_t workspace_bytes,
               hipStream_t stream);

/*
 * The factor U that sketch_column_weights and sketch_map take, from the Gram
 * matrix of the sample inputs (the mapping's error update of Frantar et al.
 * needs the upper Cholesky factor of the inverse Hessian):
 *   U upper triangular with U^T U = (H + damp * mean(diag H) * I)^-1.
 * H: [d][d] float64, row-major, symmetric (H = X_s^T X_s; only entries with
 * i <= j are read). damp >= 0 (1 % is the usual choice). U: [d][d] fp32,
 * written in full (zeros below the diagonal). Computed in float64: with P the
 * exchange matrix and P H P = L L^T, U = P L^-1 P (one blocked Cholesky
 * factorization and one triangular inverse). workspace:
 * sketch_hessian_factor_workspace(d) bytes (16-byte aligned; 8 (D^2 + D * 64
 * + 32) bytes with D = d rounded up to a multiple of 64). 1 <= d <= 65536.
 * A matrix that is not positive definite after the damping gives NaN entries
 * in U (the factorization runs on the device; nothing is read back).
 */
size_t sketch_hessian_factor_workspace(int64_t d);

int sketch_hessian_factor(const double* H, int64_t d, double damp, float* U,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Fused optimizer steps for the trainable tables (SpaLLM section 2.3: only the
 * table values are fine-tuned; the mapping stays frozen). The pages give the
 * learning rates searched (SpaLLM appendix B.1, Table 7) but no optimizer;
 * these are the textbook rules. One pass over `count` table entries (count =
 * n * gpr * 2^b for one layer; any count >= 0 is accepted, 0 is a no-op):
 *   master     [count] fp32, updated in place (the trained values)
 *   grad       [count] fp32, read only (e.g. dLUT of sketch_matmul_bwd), used
 *              as grad * grad_scale
 *   lut        [count] compute copy in lut_dtype (SKM_F16 or SKM_BF16),
 *              written as the new master rounded to nearest even; NULL = none
 *              (lut_dtype is then ignored)
 * Adam with decoupled weight decay (Kingma & Ba, Algorithm 1; Loshchilov &
 * Hutter), step = 1, 2, ... counts this call among the steps taken so far:
 *   g = grad * grad_scale
 *   master *= 1 - lr * weight_decay
 *   exp_avg    = beta1 * exp_avg    + (1 - beta1) * g
 *   exp_avg_sq = beta2 * exp_avg_sq + (1 - beta2) * g * g
 *   master -= lr / (1 - beta1^step) * exp_avg
 *             / (sqrt(exp_avg_sq) / sqrt(1 - beta2^step) + eps)
 * exp_avg and exp_avg_sq [count] fp32 start as zeros before step 1.
 * Requires lr, eps, weight_decay >= 0, 0 <= beta1, beta2 < 1, all finite.
 * All pointers 16-byte aligned; the written buffers must not overlap each
 * other or grad (SKM_EALIAS). Computed in fp32.
 */
int sketch_lut_adam_step(float* master, void* lut, int lut_dtype,
                         const float* grad, float* exp_avg, float* exp_avg_sq,
                         int64_t count, int64_t step,
                         float lr, float beta1, float beta2, float eps,
                         float weight_decay, float grad_scale,
                         hipStream_t stream);

/*
 * SGD with heavy-ball momentum and coupled weight decay, over the same
 * buffers as above:
 *   g = grad * grad_scale + weight_decay * master
 *   momentum_buf = momentum * momentum_buf + g;  g = momentum_buf
 *                                               (only when momentum != 0)
 *   master -= lr * g
 * momentum_buf [count] fp32 starts as zeros (then step 1 stores g, as
 * torch.optim.SGD does); it may be NULL when momentum == 0. Requires lr,
 * momentum, weight_decay >= 0 and finite. Alignment and overlap rules as for
 * sketch_lut_adam_step.
 */
int sketch_lut_sgd_step(float* master, void* lut, int lut_dtype,
                        const float* grad, float* momentum_buf,
                        int64_t count,
                        float lr, float momentum, float weight_decay, float grad_scale,
                        hipStream_t stream);

/* Static, human-readable text for a status code. */
const char* sketch_status_str(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int sketch_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SKETCH_MATMUL_H */
