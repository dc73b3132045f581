/*
 * llm_int8.h - C ABI of the LLM.int8() mixed-precision linear layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer computes Y = X . W^T for fp16 activations X[T,K] and a weight
 * W[N,K] that has been quantized once to int8 with one scale per output
 * feature.  Each call:
 *   1. finds the outlier feature columns of X: columns j in which some
 *      |X[t,j]| > threshold (the pages use 6.0)
 *        -- hncyxsy.com/news/230290 (LLM quantization, part 2), section 2.1;
 *           lowentro.cn "model quantization" notes, Q4;
 *   2. quantizes every token row of X over its normal columns with a
 *      symmetric absmax scale, sX[t] = max|x| / 127, code round(x / sX[t])
 *      clipped to [-127, 127]; outlier columns get code 0
 *        -- notes Q2 (symmetric formulas) and Q11 (range); tqpw.cn/news/5683,
 *           section 2.1 (scale = max/127, round, clip);
 *   3. multiplies the int8 codes, int8 x int8 -> int32, and dequantizes with
 *      acc * sX[t] * sW[n];
 *   4. multiplies the outlier columns of X (fp16) with the same columns of
 *      the dequantized weight in floating point and adds the two parts; the
 *      sum is stored as fp16
 *        -- hncyxsy.com/news/230290, section 2.1; tqpw.cn/news/5683,
 *           section 3.1.
 *
 * Conventions for every entry point:
 *   - All tensors are dense row-major, in device memory owned by the caller.
 *     fp16 tensors are passed as raw IEEE binary16 bit patterns (void*).
 *     Pointers must be 16-byte aligned.
 *   - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL is
 *     the default stream).  No entry point synchronizes, allocates or frees
 *     device memory, or copies anything to the host.  The library keeps no
 *     mutable global state: calls on different streams with different
 *     workspaces may overlap.
 *   - Validation happens on the host, before anything is launched; a
 *     non-LI8_OK status means nothing was enqueued, except LI8_ERR_HIP,
 *     which reports a launch failure.  Device-side faults surface at the
 *     caller's next synchronization.
 *   - Shapes: T >= 0 tokens, N >= 0 output features, K >= 0 features with
 *     K a multiple of 16 and K <= 133144 (so that the int32 sum of K
 *     products of magnitude <= 127*127 cannot overflow), T*K < 2^31 and
 *     N*K < 2^31.  T == 0 or N == 0 is an empty call that enqueues nothing.
 *   - Inputs must be finite; NaN or Inf in X or W is outside the contract.
 */
#ifndef LLM_INT8_H
#define LLM_INT8_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum li8_status {
    LI8_OK = 0,
    LI8_ERR_INVALID_ARG = 1, /* null pointer, NaN or negative threshold     */
    LI8_ERR_SHAPE = 2,       /* negative dim, K % 16 != 0, K > 133144,
                                T*K or N*K >= 2^31                         */
    LI8_ERR_ALIGN = 3,       /* a pointer not 16-byte aligned               */
    LI8_ERR_WORKSPACE = 4,   /* workspace null or smaller than required     */
    LI8_ERR_HIP = 5,         /* a HIP launch or copy failed to enqueue (for
                                example: no gfx950 code for this device)   */
    LI8_ERR_SCRATCH = 6      /* llm_int8_linear_noalloc: the shape needs more
                                than its fixed scratch array               */
} li8_status;

/* Human-readable name of a status code (static string, never NULL). */
const char *li8_status_str(li8_status status);

/*
 * Vector-wise weight quantization, done once per weight, off the per-call
 * path (tqpw.cn/news/5683, section 2.1; hncyxsy.com/news/230290, section
 * 2.1: one scale per output feature; notes Q3: per-channel scales).
 *   W   [N,K] fp16, read only.
 *   Wq  [N,K] int8 out:  Wq[n,k] = clamp(rne(fl32(W[n,k] / sW[n])), -127, 127)
 *   sW  [N]  fp32 out:   sW[n]   = fl32(max_k |W[n,k]| / 127)
 *   (rne: round half to even; fl32: IEEE fp32 rounding; a row of zeros gets
 *   sW = 0 and codes 0.)
 */
li8_status int8_quantize_weight(const void *W, int64_t N, int64_t K,
                                int8_t *Wq, float *sW, hipStream_t stream);

/*
 * Bytes of device workspace that is enough for every entry point below that
 * takes one, for this shape.  It covers the worst case, every column an
 * outlier, so the size never depends on the data; it is sized for the
 * fp16-weight variant, whose gathered outlier weight columns are fp16.
 * The int8 and SmoothQuant-style entry points (llm_int8_linear, _prepare,
 * _gemm, _*_cached, smoothquant_prepare, smoothquant_linear) accept a
 * workspace of llm_int8_linear_workspace_bytes(T, K, N) bytes for shapes on
 * the tiled path, about N*K bytes less.  Returns 0 if the shape is invalid.
 */
size_t llm_int8_workspace_bytes(int64_t T, int64_t K, int64_t N);

/*
 * Bytes of device workspace that llm_int8_linear itself needs for this
 * shape (see llm_int8_plan): 0 on the fused few-token path; on the split
 * few-token path about 2*T*K bytes plus 1 KB per slice of K and 16 output
 * features; else the int8 layout (about 3*T*K + N*K bytes, the worst case
 * of every column an outlier).  Returns 0 for an invalid shape too.
 */
size_t llm_int8_linear_workspace_bytes(int64_t T, int64_t K, int64_t N);

/*
 * Which kernels a call of this shape runs (introspection for tests and
 * benchmarks; nothing is enqueued):
 *   *path    LI8_PATH_EMPTY      T == 0 or N == 0, nothing is launched;
 *            LI8_PATH_FEW_TOKENS T <= 16 and 16 <= K <= 8192: llm_int8_linear
 *                                is one fused kernel, and llm_int8_gemm a
 *                                kernel of the same structure reading the
 *                                prepared workspace; *tile_m = T,
 *                                *tile_n = 16 output features per row group;
 *            LI8_PATH_TILED      the prepare kernels and the tiled int8 MFMA
 *                                GEMM with output tiles of *tile_m x *tile_n;
 *            LI8_PATH_FEW_TOKENS_SPLIT  T <= 16 and K > 8192: K is split
 *                                across workgroups; llm_int8_linear is a
 *                                scan of X, the split int8 MFMA product and
 *                                a finishing kernel (three launches), and
 *                                llm_int8_gemm the last two on the prepared
 *                                workspace; *tile_m = T, *tile_n = 16.
 *   *fold_lo, *fold_hi  on the tiled path, a call whose outlier count n has
 *            fold_lo < n <= fold_hi has its GEMM copy the weight's outlier
 *            columns out of the K stages it streams, and its prepare kernel
 *            skips that gather; for other counts the prepare kernel gathers
 *            them (both 0 when the GEMM never copies them).  This holds for
 *            llm_int8_linear and llm_int8_prepare + _gemm; the fp16-weight
 *            and cached calls always gather.  On the few-token paths both
 *            are 0: their kernels read the outlier columns of Wq by index
 *            and nothing gathers them.
 * Returns LI8_ERR_SHAPE for an invalid shape, LI8_ERR_INVALID_ARG for a
 * null pointer.
 */
enum { LI8_PATH_EMPTY = 0, LI8_PATH_FEW_TOKENS = 1, LI8_PATH_TILED = 2,
       LI8_PATH_FEW_TOKENS_SPLIT = 3 };
li8_status llm_int8_plan(int64_t T, int64_t K, int64_t N, int32_t *path, int32_t *tile_m,
                         int32_t *tile_n, int32_t *fold_lo, int32_t *fold_hi);

/*
 * The whole layer: Y[T,N] = decomposed X[T,K] . W^T.
 *   X          [T,K] fp16, read only.
 *   Wq, sW     the outputs of int8_quantize_weight for W[N,K], read only.
 *   threshold  outlier threshold, >= 0; +inf disables the decomposition (the
 *              pure vector-wise int8 product); 0 makes every column that has
 *              a non-zero value an outlier.
 *   Y          [T,N] fp16 out, fully overwritten; must not alias an input.
 *   workspace  device buffer of at least llm_int8_linear_workspace_bytes(T,K,N)
 *              bytes, owned by the caller; its contents on entry do not
 *              matter.  Two calls in flight at once need two workspaces.
 *              On the fused few-token path (llm_int8_plan) none is used,
 *              and NULL is accepted.
 * Equivalent to llm_int8_prepare followed by llm_int8_gemm on the same
 * stream and workspace.
 */
li8_status llm_int8_linear(const void *X, const int8_t *Wq, const float *sW,
                           float threshold, int64_t T, int64_t K, int64_t N,
                           void *Y, void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * llm_int8_linear for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and the same result bit for bit, with the
 * workspace taken from a fixed array that the library holds on each GPU it
 * runs on, LI8_NOALLOC_SCRATCH_BYTES bytes (128 MiB) for the life of the
 * process.  Nothing is allocated or freed on any call.
 *   - Arguments as for llm_int8_linear, without the workspace.
 *   - Shapes whose workspace (llm_int8_linear_workspace_bytes) exceeds the
 *     array return LI8_ERR_SCRATCH and enqueue nothing (4096 x 4096 x 11008
 *     needs about 96 MB; few-token shapes need none).
 *   - Every call on one GPU uses that GPU's one array, so calls that
 *     overlap on one GPU (two streams, two host threads) race and give
 *     wrong results: order them.  Nothing carries over from one call to
 *     the next: no kernel reads a word of the array that its call has not
 *     written first.
 *   - The first call on a device looks the array's address up (a host-side
 *     query, no allocation); a failure there returns LI8_ERR_HIP.
 */
#define LI8_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
li8_status llm_int8_linear_noalloc(const void *X, const int8_t *Wq, const float *sW,
                                   float threshold, int64_t T, int64_t K, int64_t N,
                                   void *Y, hipStream_t stream);

/*
 * First half of llm_int8_linear (steps 1-2 above): outlier detection,
 * token-wise quantization of X, and the gathering of the outlier columns of
 * X and of Wq into compact matrices (those of Wq only where llm_int8_gemm
 * does not copy them itself: see llm_int8_plan's fold range, and the
 * few-token paths, whose kernels read them by index).  Everything it
 * produces stays in `workspace`, which llm_int8_gemm then consumes.
 * Arguments as for llm_int8_linear.
 */
li8_status llm_int8_prepare(const void *X, const int8_t *Wq, float threshold,
                            int64_t T, int64_t K, int64_t N,
                            void *workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * Second half of llm_int8_linear (steps 3-4): the int8 GEMM with its
 * dequantizing epilogue and the outlier product.  `workspace` must hold
 * the result of llm_int8_prepare for the same X, Wq, T, K, N, enqueued
 * earlier on the same stream (or otherwise ordered before this call).
 *   acc  optional [T,N] int32 out (NULL to skip): the exact int8 sums
 *        acc[t,n] = sum_j Xq[t,j] * Wq[n,j], stored by the same kernel that
 *        computes Y (a test hook; it costs 4*T*N bytes of writes).
 */
li8_status llm_int8_gemm(const int8_t *Wq, const float *sW,
                         int64_t T, int64_t K, int64_t N, void *Y,
                         int32_t *acc, const void *workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * The fp16-weight variant (hncyxsy.com/news/230290, section 2.1: the weight
 * sub-matrix of the outlier columns is extracted and multiplied in fp16 with
 * the outlier columns of X).  The outlier columns multiply the original
 * fp16 weight W instead of the dequantized codes Wq*sW:
 *   Y[t,n] = fp16( fl32(fl32(acc[t,n] * sX[t]) * sW[n]) + sum_{j in O} X[t,j] * W[n,j] )
 * (the outlier sum accumulated in fp32 on the GPU).  With threshold 0 every
 * column that has a non-zero value is an outlier and Y is the fp16 product
 * X . W^T; with threshold +inf it equals llm_int8_linear bit for bit.
 *   W   [N,K] fp16, read only: the weight that Wq and sW were quantized
 *       from (16-byte aligned; may be NULL only when T, N or K is 0).
 * Everything else as for llm_int8_linear; the workspace size is the same.
 * Equivalent to llm_int8_prepare_fp16w followed by llm_int8_gemm_fp16w.
 */
li8_status llm_int8_linear_fp16w(const void *X, const int8_t *Wq, const float *sW,
                                 const void *W, float threshold, int64_t T, int64_t K,
                                 int64_t N, void *Y, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * First half of llm_int8_linear_fp16w: as llm_int8_prepare, but the outlier
 * columns gathered on the weight side are those of the fp16 W.
 */
li8_status llm_int8_prepare_fp16w(const void *X, const void *W, float threshold,
                                  int64_t T, int64_t K, int64_t N,
                                  void *workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * Second half of llm_int8_linear_fp16w: as llm_int8_gemm on a workspace
 * prepared by llm_int8_prepare_fp16w (W is read directly when T <= 16).
 */
li8_status llm_int8_gemm_fp16w(const int8_t *Wq, const float *sW, const void *W,
                               int64_t T, int64_t K, int64_t N, void *Y,
                               int32_t *acc, const void *workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * Outlier-column cache (lowentro.cn "model quantization" notes, Q4: the
 * outlier features sit on the same few channels from token to token, so the
 * set found by step 1 tends to repeat across calls).  A cache is a device
 * buffer owned by the caller and bound to one quantized weight (Wq); it holds
 * the last outlier set and the outlier columns of Wq gathered for it.  A call
 * whose set equals the cached one skips that gather (which reads about all of
 * Wq when the outlier columns are spread over K) and the GEMM reads the
 * cached columns.  Detection still runs on every call, so the result is
 * always that of llm_int8_linear, bit for bit, whatever the cache holds.
 *
 * Layout, for tests and inspection: the cache starts with int32 hdr[64],
 * hdr[0] = 1 when it holds a set, hdr[1] = that set's nO, hdr[2] = calls
 * that reused it (hits), hdr[3] = calls that gathered (misses); hits and
 * misses count tiled calls only.  For few tokens (the fused path: T <= 16,
 * K <= 8192) the cache is neither read nor written.
 *
 * Ownership: one cache per weight, and one call in flight per cache (calls
 * that share it must be ordered, e.g. on one stream).  After Wq changes, or
 * before first use, llm_int8_cache_reset must run; a cache used with a
 * weight other than the one it was filled from gives wrong outputs.
 */

/* Bytes of a cache for a weight [N,K] (about N*K); 0 if the shape is invalid. */
size_t llm_int8_cache_bytes(int64_t K, int64_t N);

/* Marks the cache empty (and zeroes its counters); enqueued on `stream`. */
li8_status llm_int8_cache_reset(void *cache, size_t cache_bytes, int64_t K, int64_t N,
                                hipStream_t stream);

/*
 * llm_int8_linear with an outlier-column cache; same arguments, plus the
 * cache (16-byte aligned, at least llm_int8_cache_bytes(K, N) bytes).
 * Y is bit-identical to llm_int8_linear's.
 */
li8_status llm_int8_linear_cached(const void *X, const int8_t *Wq, const float *sW,
                                  float threshold, int64_t T, int64_t K, int64_t N, void *Y,
                                  void *workspace, size_t workspace_bytes, void *cache,
                                  size_t cache_bytes, hipStream_t stream);

/* The two halves of llm_int8_linear_cached (as llm_int8_prepare / _gemm). */
li8_status llm_int8_prepare_cached(const void *X, const int8_t *Wq, float threshold, int64_t T,
                                   int64_t K, int64_t N, void *workspace, size_t workspace_bytes,
                                   void *cache, size_t cache_bytes, hipStream_t stream);
li8_status llm_int8_gemm_cached(const int8_t *Wq, const float *sW, int64_t T, int64_t K, int64_t N,
                                void *Y, int32_t *acc, const void *workspace,
                                size_t workspace_bytes, const void *cache, size_t cache_bytes,
                                hipStream_t stream);

/*
 * SmoothQuant-style W8A8 (lowentro.cn "model quantization" notes, Q9 and
 * Q10; hncyxsy.com/news/230290, section 5.1): instead of splitting off the
 * outlier columns, one factor s_j per input feature moves their range from
 * the activation to the weight through the exact rewrite
 * X . W^T = (X / s) . (W * s)^T; both sides are then quantized with the
 * absmax scheme above and multiplied in int8, with no floating-point part.
 * The factor is
 *   s_j = ax_j^alpha / aw_j^(1 - alpha)
 * with ax_j = max_t |X_cal[t,j]| over a calibration batch of activations,
 * aw_j = max_n |W[n,j]|, and the migration strength alpha in [0, 1].  (Q10
 * prints a garbled product form whose alpha = 0 value is aw_j; the quotient
 * is what makes its own description hold: alpha = 0.5 balances the smoothed
 * ranges ax_j / s_j and aw_j * s_j, alpha = 1 gives s_j = ax_j, and
 * alpha = 0 flattens the weight range to 1 with s_j = 1 / aw_j.)
 * Offline, once per layer: smoothquant_column_absmax (of the calibration
 * batch and of W), smoothquant_factors, smoothquant_quantize_weight.  Per
 * call: smoothquant_linear, or smoothquant_prepare + llm_int8_gemm.
 */

/*
 * absmax[j] = max_r |A[r,j]| (exact, as fp32) for fp16 A [rows,K]; 0 for a
 * column of zeros.  0 <= rows < 2^31 (rows*K may exceed 2^31); K as for
 * every call.  absmax [K] fp32 out.
 */
li8_status smoothquant_column_absmax(const void *A, int64_t rows, int64_t K, float *absmax,
                                     hipStream_t stream);

/*
 * The smoothing factors and their reciprocals, [K] fp32 each:
 *   s[j]     = fl32(ax[j]^alpha / aw[j]^(1-alpha))  (evaluated in fp64),
 *              or 1 where ax[j] or aw[j] is 0;
 *   s_inv[j] = fl32(1 / s[j]).
 * ax, aw [K] fp32 in (>= 0, finite); alpha in [0, 1], else
 * LI8_ERR_INVALID_ARG.  The fp64 power is the device library's (within an
 * ulp or so of fp64), so s[j] can differ from a correctly rounded
 * evaluation only where the fp64 quotient lies that close to the midpoint
 * of two fp32 values.
 */
li8_status smoothquant_factors(const float *ax, const float *aw, double alpha, int64_t K,
                               float *s, float *s_inv, hipStream_t stream);

/*
 * Absmax quantization of the smoothed weight W' = fl32(W * s) (per column):
 *   sW[n]   = fl32(max_k |W'[n,k]| / 127)
 *   Wq[n,k] = clamp(rne(fl32(W'[n,k] / sW[n])), -127, 127)   (0 if sW[n] = 0)
 * W [N,K] fp16 in, s [K] fp32 in, Wq [N,K] int8 out, sW [N] fp32 out.
 */
li8_status smoothquant_quantize_weight(const void *W, const float *s, int64_t N, int64_t K,
                                       int8_t *Wq, float *sW, hipStream_t stream);

/*
 * Per-call token side: X' = fl32(X * s_inv) per column, then
 *   sX[t]   = fl32(max_k |X'[t,k]| / 127)
 *   Xq[t,k] = clamp(rne(fl32(X'[t,k] / sX[t])), -127, 127)   (0 if sX[t] = 0)
 * written into `workspace` (sized by llm_int8_workspace_bytes(T, K, N)) with
 * no outlier column, so that llm_int8_gemm on it computes
 *   Y[t,n] = fp16(fl32(fl32(acc[t,n] * sX[t]) * sW[n])).
 * X [T,K] fp16 in, s_inv [K] fp32 in (as written by smoothquant_factors).
 */
li8_status smoothquant_prepare(const void *X, const float *s_inv, int64_t T, int64_t K,
                               int64_t N, void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * The whole per-call layer: smoothquant_prepare followed by llm_int8_gemm
 * (Wq, sW from smoothquant_quantize_weight).  Y [T,N] fp16 out.
 */
li8_status smoothquant_linear(const void *X, const float *s_inv, const int8_t *Wq,
                              const float *sW, int64_t T, int64_t K, int64_t N, void *Y,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Copies the intermediate results of the last llm_int8_prepare on
 * `workspace` into caller buffers (device-to-device, on `stream`).  A test
 * hook: the product path never needs it.  Any output pointer may be NULL.
 *   outlier_bits [ceil(K/32)] uint32: bit (j % 32) of word j / 32 set iff
 *                column j is an outlier.
 *   n_outliers   [1] int32: number of outlier columns nO.
 *   outlier_idx  [K] int32: the outlier columns in ascending order; entries
 *                from nO on are unspecified.
 *   Xq           [T,K] int8: token codes (0 in outlier columns).
 *   sX           [T] fp32: token scales.
 *   X_out        T*K fp16 elements: the gathered outlier values in chunks
 *                of 16 columns, X[t, outlier_idx[i]] at element
 *                ((i / 16) * T + t) * 16 + i % 16 for i < nO; ranks nO ..
 *                round_up(nO,16)-1 are zero; the rest is unspecified.
 */
li8_status llm_int8_export_stages(const void *workspace, size_t workspace_bytes,
                                  int64_t T, int64_t K, int64_t N,
                                  uint32_t *outlier_bits, int32_t *n_outliers,
                                  int32_t *outlier_idx, int8_t *Xq, float *sX,
                                  void *X_out, hipStream_t stream);

/*
 * Every intermediate result of one linear call, for tests: the rows of the
 * method one by one (hncyxsy.com/news/230290, section 2.1: the outlier
 * columns, the vector-wise int8 quantization of the rest and their int8
 * product, the fp16 product of the outlier columns; tqpw.cn/news/5683,
 * section 2.1: scale and codes).  It runs llm_int8_prepare and
 * llm_int8_gemm on `workspace` (the kernels of llm_int8_linear on the tiled
 * path; on the few-token paths the two-call route, whose Y equals the
 * one-call kernel's bit for bit), writes Y, and copies out:
 *   flags        [K] uint8: 1 if column j is an outlier column, else 0.
 *   n_outliers   [1] int32: nO, the number of outlier columns.
 *   outlier_idx  [K] int32: the outlier columns in ascending order;
 *                entries from nO on are unspecified.
 *   Xq           [T,K] int8: token codes (0 in outlier columns).
 *   sX           [T] fp32: token scales.
 *   X_out        [T,K] fp16, row stride K: X[t, outlier_idx[i]] at
 *                t*K + i for i < nO; the rest of each row is unspecified.
 *   acc          [T,N] int32: the exact int8 sums, as llm_int8_gemm's acc.
 * Any of these output pointers may be NULL (that output is skipped).  The
 * other arguments are those of llm_int8_linear; the workspace must be at
 * least llm_int8_workspace_bytes(T, K, N) (it is the int8 layout of
 * llm_int8_prepare).  Outputs are device memory owned by the caller.
 * Errors as for llm_int8_prepare and llm_int8_gemm, from host checks made
 * before anything is enqueued; LI8_ERR_ALIGN also for a misaligned Xq, sX,
 * X_out or acc.
 */
li8_status llm_int8_stages(const void *X, const int8_t *Wq, const float *sW,
                           float threshold, int64_t T, int64_t K, int64_t N,
                           void *Y, void *workspace, size_t workspace_bytes,
                           uint8_t *flags, int32_t *n_outliers,
                           int32_t *outlier_idx, int8_t *Xq, float *sX,
                           void *X_out, int32_t *acc, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LLM_INT8_H */
