// Internal declarations shared by the HIP sources of libllm_int8.so.
// Not part of the public ABI (include/llm_int8.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace li8 {

// Largest K for which sum_{j<K} |q_x q_w| <= K * 127 * 127 fits in int32.
constexpr int64_t kMaxK = 133144;
// Largest T*K and N*K: the GEMM reads the int8 operands through buffer
// resources with 32-bit offsets.
constexpr int64_t kMaxOperandBytes = ((int64_t)1 << 31) - 1;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Few-token path (one fused kernel): T <= kDecodeMaxT token rows, whose
// codes for all of K stay in LDS, hence the bound on K.
constexpr int kDecodeMaxT = 16;
constexpr int kDecodeMaxK = 8192;
constexpr int kDecodeMaxBlocks = 256;   // one workgroup per CU

// Row strips of the outlier detection: each writes its own partial bit
// set, and the quantization kernel ORs the strips' words.
constexpr int kDetectParts = 16;

// Device workspace carved into fixed regions.  Offsets depend only on the
// shape (T, K, N), never on the data, so the host needs no readback.
//   part : uint32[kDetectParts][ceil(K/32)]  per-row-strip partial bit sets
//                              (every word of the strips in use written by
//                              the detection kernel, none read before)
//   bits : uint32[ceil(K/32)]  outlier column bit set (the strips' OR)
//   meta : int32[64]           meta[0] = nO
//   idx  : int32[K]            outlier columns, ascending
//   sX   : fp32[T]             token scales
//   Xq   : int8[T,K]           token codes, 0 in outlier columns
//   wpre : int32[ceil(K/32)+1] outlier columns before bit-set word w
//                              (column 32 w); wpre[ceil(K/32)] = nO
//   XO   : fp16, T*K elements  the gathered outlier values in 16-column
//                              chunks: X[t, idx[i]] at ((i/16)*T + t)*16 + i%16
//                              for i < nO, zero to the next multiple of 16
//                              (a chunk of a row block is contiguous)
//   WO   : int8, N*K elements  likewise Wq[n, idx[i]] at ((i/16)*N + n)*16 +
//                              i%16.  In the fp16-weight variant the same
//                              region holds fp16 W[n, idx[i]] (2*N*K bytes)
// total_i8 ends the layout after an int8 WO (the int8 and SmoothQuant-style
// paths); total after an fp16 one (every entry point).
struct WsLayout {
    size_t part, bits, meta, idx, wpre, sX, Xq, XO, WO, total_i8, total;
};

inline WsLayout ws_layout(int64_t T, int64_t K, int64_t N)
{
    const size_t A = 256;
    WsLayout L;
    size_t off = 0;
    size_t nwords = (size_t)((K + 31) / 32);
    L.part = off; off = align_up(off + 4 * kDetectParts * (nwords ? nwords : 1), A);
    L.bits = off; off = align_up(off + 4 * (nwords ? nwords : 1), A);
    L.meta = off; off = align_up(off + 256, A);
    L.idx = off;  off = align_up(off + 4 * (size_t)(K ? K : 1), A);
    L.wpre = off; off = align_up(off + 4 * (nwords + 1), A);
    L.sX = off;   off = align_up(off + 4 * (size_t)(T ? T : 1), A);
    L.Xq = off;   off = align_up(off + (size_t)T * (size_t)K + 16, A);
    L.XO = off;   off = align_up(off + 2 * (size_t)T * (size_t)K + 16, A);
    L.WO = off;
    L.total_i8 = align_up(off + (size_t)N * (size_t)K + 16, A);
    L.total = align_up(off + 2 * (size_t)N * (size_t)K + 16, A);
    return L;
}

// Outlier-column cache, owned by the caller and bound to one Wq:
//   hdr  : int32[64]  hdr[0] = 1 when it holds a set, [1] its nO,
//                     [2] hits, [3] misses (calls that gathered)
//   bits : uint32[ceil(K/32)]  the cached outlier bit set
//   WO   : int8, N*K elements, the workspace WO layout (16-column chunks)
struct CacheLayout {
    size_t hdr, bits, WO, total;
};

inline CacheLayout cache_layout(int64_t K, int64_t N)
{
    const size_t A = 256;
    CacheLayout C;
    size_t off = 0;
    size_t nwords = (size_t)((K + 31) / 32);
    C.hdr = off;  off = align_up(off + 256, A);
    C.bits = off; off = align_up(off + 4 * (nwords ? nwords : 1), A);
    C.WO = off;   off = align_up(off + (size_t)N * (size_t)K + 16, A);
    C.total = off;
    return C;
}

// Launchers (quant.hip).  All asynchronous on `s`; return hipGetLastError().
hipError_t launch_quantize_weight(const uint16_t *W, int64_t N, int64_t K,
                                  int8_t *Wq, float *sW, hipStream_t s);
// W16: null, or the fp16 weight [N,K] whose outlier columns are gathered
// instead of those of Wq (the fp16-weight variant).  cache: null, or an
// outlier-column cache (int8 path only) whose WO receives the gathered
// columns, the gather being skipped when it already holds this call's set.
// The weight's outlier columns are left ungathered when skip.lo < nO <=
// skip.hi: the tiled GEMM's fold range, or every count for the few-token
// kernels, which gather by index themselves.
struct GatherSkip {
    int lo, hi;
};
hipError_t launch_prepare(const uint16_t *X, const int8_t *Wq, const uint16_t *W16,
                          uint16_t thr_mag, int64_t T, int64_t K, int64_t N, char *ws,
                          const WsLayout &L, hipStream_t s, char *cache = nullptr,
                          GatherSkip skip = GatherSkip{0, 0});
hipError_t launch_cache_reset(char *cache, hipStream_t s);

// Tile shape of the tiled GEMM for a call of this shape (gemm.hip), and
// fold: the most outlier columns whose weight columns its int8 variant
// copies out of the weight stages it multiplies (0: none).  A call with
// kFoldMin < nO <= fold needs no gathered WO; with fewer the prepare
// kernel's gather is the cheaper (measured on 128-wide tiles at 512 x 5120 x
// 13824 and fewer tokens: 45.7 against 49.4 us per call at 36 outlier
// columns, even at 78, 56.0 against 59.5 at 133), and the plain main loop
// is kept.
constexpr int kFoldMin = 64;
constexpr int64_t kFoldMaxK = 8192;
struct GemmPlan {
    int bm, bn, fold;
};
GemmPlan gemm_plan(int64_t T, int64_t K, int64_t N);

// Launcher (gemm.hip).
// fp16w: the outlier product uses the fp16 weight columns that the prepare
// call gathered from W16 (and the result is added after the scale sW).
// WO: null (the workspace's gathered weight columns) or the cache's.
hipError_t launch_gemm(const int8_t *Wq, const float *sW, int64_t T, int64_t K,
                       int64_t N, uint16_t *Y, int32_t *acc, const char *ws,
                       const WsLayout &L, bool fp16w, hipStream_t s,
                       const int8_t *WO = nullptr);

// Few-token path (decode.hip).  decode_shape(T, K) says whether both
// entry points use it for this shape; the fused launch does the whole
// layer from X, the other reads what launch_prepare left in the workspace.
bool decode_shape(int64_t T, int64_t K);
// W16 non-null selects the fp16-weight variant.
hipError_t launch_decode_fused(const uint16_t *X, const int8_t *Wq, const float *sW,
                               const uint16_t *W16, uint16_t thr_mag, int64_t T, int64_t K,
                               int64_t N, uint16_t *Y, hipStream_t s);
hipError_t launch_decode_gemm(const int8_t *Wq, const float *sW, const uint16_t *W16, int64_t T,
                              int64_t K, int64_t N, uint16_t *Y, int32_t *acc, const char *ws,
                              const WsLayout &L, hipStream_t s);

// Few tokens with K past kDecodeMaxK (decode_split.hip): K split into KS
// slices of KSL columns (a multiple of 512, at most kSplitMaxSlice) over
// KS x NRGC workgroups, each taking row groups rgc, rgc + NRGC, ...
constexpr int kSplitMaxSlice = 8192;
struct SplitPlan {
    int KS, KSL, NRGC;
};
bool split_shape(int64_t T, int64_t K);
SplitPlan split_plan(int64_t T, int64_t K, int64_t N);
// Workspace of the one-call route: the prepared stages in the tiled
// layout's forms (bit set, meta, ascending outlier list, token scales,
// gathered outlier values of X), the scan's per-strip outlier counts and
// token maxima, and the partial sums.
struct SplitLayout {
    size_t bits, meta, idx, sX, XO, ocnt, pmax, part, total;
};
SplitLayout split_layout(int64_t T, int64_t K, int64_t N);
hipError_t launch_split_fused(const uint16_t *X, const int8_t *Wq, const float *sW,
                              const uint16_t *W16, uint16_t thr_mag, int64_t T, int64_t K,
                              int64_t N, uint16_t *Y, char *ws, hipStream_t s);
// The workspace route: codes, scales and outlier stages from launch_prepare,
// the partial sums in the WO region (the few-token kernels never read it).
hipError_t launch_split_gemm(const int8_t *Wq, const float *sW, const uint16_t *W16, int64_t T,
                             int64_t K, int64_t N, uint16_t *Y, int32_t *acc, const char *ws,
                             const WsLayout &L, hipStream_t s);

// SmoothQuant-style W8A8 (smoothquant.hip).  Column absmax of fp16 A
// [rows,K] as fp32; factors s and fl32(1/s); smoothed weight quantization;
// the per-call token side, which leaves codes, scales and nO = 0 in the
// workspace for launch_gemm / launch_decode_gemm.
hipError_t launch_column_absmax(const uint16_t *A, int64_t rows, int64_t K, float *out,
                                hipStream_t s);
hipError_t launch_sq_factors(const float *ax, const float *aw, double alpha, int64_t K, float *sf,
                             float *r, hipStream_t s);
hipError_t launch_sq_quantize_weight(const uint16_t *W, const float *sf, int64_t N, int64_t K,
                                     int8_t *Wq, float *sW, hipStream_t s);
hipError_t launch_sq_prepare(const uint16_t *X, const float *r, int64_t T, int64_t K, char *ws,
                             const WsLayout &L, hipStream_t s);

} // namespace li8
