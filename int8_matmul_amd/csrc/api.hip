// Host side of the C ABI declared in include/llm_int8.h: argument checks,
// workspace carving and kernel launches.  No allocation, no host sync.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "li8_internal.h"
#include "llm_int8.h"

using namespace li8;

// Workspace of llm_int8_linear_noalloc: one fixed array per GPU, held for
// the life of the process.  In host code `scratch` is only a handle: its
// device address, per device, comes from hipGetSymbolAddress and is the
// only form in which it is passed on.
static __device__ __align__(256) char scratch[LI8_NOALLOC_SCRATCH_BYTES];

namespace {

bool misaligned(const void *p) { return ((uintptr_t)p & 15u) != 0; }

// The stage export's conversions: the bit set to one byte per column, and
// the gathered outlier values from their 16-column chunks (rank i of row t
// at ((i / 16) * T + t) * 16 + i % 16) to rows of stride K.
__global__ void k_stage_flags_xo(const uint32_t *__restrict__ bits, const int32_t *__restrict__ meta,
                                 const uint16_t *__restrict__ XO, int T, int K,
                                 uint8_t *__restrict__ flags, uint16_t *__restrict__ xo_rows)
{
    const int nO = min(max(meta[0], 0), K);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t first = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (flags)
        for (int64_t j = first; j < K; j += stride)
            flags[j] = (uint8_t)((bits[j >> 5] >> (j & 31)) & 1u);
    if (xo_rows)
        for (int64_t e = first; e < (int64_t)T * nO; e += stride) {
            const int64_t t = e / nO, i = e - t * nO;
            xo_rows[t * K + i] = XO[((i >> 4) * T + t) * 16 + (i & 15)];
        }
}

li8_status check_shape(int64_t T, int64_t K, int64_t N)
{
    if (T < 0 || K < 0 || N < 0)
        return LI8_ERR_SHAPE;
    if (K % 16 != 0 || K > kMaxK)
        return LI8_ERR_SHAPE;
    // kernels index rows and columns with int; byte offsets are int64
    const int64_t lim = (int64_t)1 << 31;
    if (T >= lim || N >= lim)
        return LI8_ERR_SHAPE;
    // the GEMM addresses the int8 operands with 32-bit buffer offsets
    if (T * K > kMaxOperandBytes || N * K > kMaxOperandBytes)
        return LI8_ERR_SHAPE;
    // T*N*4 (acc) must fit comfortably in int64
    if ((double)T * (double)N * 4.0 > 9.0e18)
        return LI8_ERR_SHAPE;
    return LI8_OK;
}

// Exact value of a binary16 magnitude pattern (0 <= m <= 0x7c00).
double half_mag_value(uint32_t m)
{
    const uint32_t e = m >> 10, f = m & 0x3ffu;
    if (e == 0)
        return ldexp((double)f, -24);
    if (e == 31)
        return INFINITY;
    return ldexp((double)(f | 0x400u), (int)e - 25);
}

// Largest binary16 magnitude pattern H whose value is <= thr (thr >= 0),
// so that |x| > thr  <=>  (bits(x) & 0x7fff) > H for finite x.
uint16_t threshold_magnitude(float thr)
{
    uint32_t lo = 0, hi = 0x7c00;   // value(lo) = 0 <= thr always
    if (half_mag_value(hi) <= (double)thr)
        return (uint16_t)hi;        // thr = +inf: nothing finite exceeds it
    while (hi - lo > 1) {           // invariant: value(lo) <= thr < value(hi)
        const uint32_t mid = (lo + hi) / 2;
        if (half_mag_value(mid) <= (double)thr)
            lo = mid;
        else
            hi = mid;
    }
    return (uint16_t)lo;
}

li8_status from_hip(hipError_t e) { return e == hipSuccess ? LI8_OK : LI8_ERR_HIP; }

// Which outlier counts the prepare kernel may leave ungathered (see
// launch_prepare): all for the few-token kernels, which gather the weight's
// outlier columns by index themselves (K); kFoldMin < nO <= fold for the
// tiled int8 GEMM, which copies them out of its own weight fragments; none
// for the fp16-weight variant and for calls with an outlier-column cache
// (the cache must hold what it records).
GatherSkip gather_above(int64_t T, int64_t K, int64_t N, bool fp16w, bool cached)
{
    if (decode_shape(T, K) || split_shape(T, K))
        return GatherSkip{-1, (int)K};
    if (fp16w || cached)
        return GatherSkip{0, 0};
    return GatherSkip{kFoldMin, gemm_plan(T, K, N).fold};
}

// Workspace bytes an entry point needs: WIDE for the fp16-weight variant
// (fp16 outlier weight columns), else the int8 layout.
enum WsKind { WS_I8, WS_WIDE };

size_t ws_need(int64_t T, int64_t K, int64_t N, WsKind kind)
{
    const WsLayout L = ws_layout(T, K, N);
    return kind == WS_WIDE ? L.total : L.total_i8;
}

// Workspace the one-call entry points need: none for the fused few-token
// kernel, the split layout for few tokens with a long K, else the prepared
// layout.
size_t linear_need(int64_t T, int64_t K, int64_t N, WsKind kind)
{
    if (decode_shape(T, K))
        return 0;
    if (split_shape(T, K))
        return split_layout(T, K, N).total;
    return ws_need(T, K, N, kind);
}

li8_status check_ws(const void *ws, size_t ws_bytes, size_t need)
{
    if (ws && misaligned(ws))
        return LI8_ERR_ALIGN;
    if (need == 0)   // (none used: a null workspace is accepted)
        return LI8_OK;
    if (!ws || ws_bytes < need)
        return LI8_ERR_WORKSPACE;
    return LI8_OK;
}

// ONE_CALL: the one-call entry points (llm_int8_linear and its variants),
// whose workspace need depends on the path (linear_need); the two-call
// route always needs the prepared layout.
enum Route { TWO_CALL, ONE_CALL };

li8_status check_route_ws(int64_t T, int64_t K, int64_t N, const void *ws, size_t ws_bytes,
                          WsKind kind, Route route)
{
    return check_ws(ws, ws_bytes, route == ONE_CALL ? linear_need(T, K, N, kind)
                                                    : ws_need(T, K, N, kind));
}

li8_status check_linear_args(const void *X, const int8_t *Wq, float threshold, int64_t T,
                             int64_t K, int64_t N, const void *ws, size_t ws_bytes,
                             WsKind kind, Route route = TWO_CALL)
{
    li8_status st = check_shape(T, K, N);
    if (st != LI8_OK)
        return st;
    if (isnan(threshold) || threshold < 0.0f)
        return LI8_ERR_INVALID_ARG;
    if (T == 0 || N == 0)
        return LI8_OK;
    if (K > 0 && (!X || !Wq))   // with K == 0, X and Wq hold no element
        return LI8_ERR_INVALID_ARG;
    if (misaligned(X) || misaligned(Wq))
        return LI8_ERR_ALIGN;
    return check_route_ws(T, K, N, ws, ws_bytes, kind, route);
}

li8_status check_gemm_args(const int8_t *Wq, const float *sW, int64_t T, int64_t K, int64_t N,
                           const void *Y, const int32_t *acc, const void *ws, size_t ws_bytes,
                           WsKind kind, Route route = TWO_CALL)
{
    li8_status st = check_shape(T, K, N);
    if (st != LI8_OK)
        return st;
    if (T == 0 || N == 0)
        return LI8_OK;
    if ((K > 0 && !Wq) || !sW || !Y)
        return LI8_ERR_INVALID_ARG;
    if (misaligned(Wq) || misaligned(sW) || misaligned(Y) || (acc && misaligned(acc)))
        return LI8_ERR_ALIGN;
    return check_route_ws(T, K, N, ws, ws_bytes, kind, route);
}

// W16 null: the int8 path; else the fp16-weight variant.  cache: null, or
// the outlier-column cache whose gathered columns the tiled GEMM reads.
li8_status gemm_common(const int8_t *Wq, const float *sW, const uint16_t *W16, int64_t T,
                       int64_t K, int64_t N, void *Y, int32_t *acc, const void *workspace,
                       hipStream_t stream, const void *cache = nullptr)
{
    const WsLayout L = ws_layout(T, K, N);
    if (decode_shape(T, K))
        return from_hip(launch_decode_gemm(Wq, sW, W16, T, K, N, static_cast<uint16_t *>(Y), acc,
                                           static_cast<const char *>(workspace), L, stream));
    if (split_shape(T, K))
        return from_hip(launch_split_gemm(Wq, sW, W16, T, K, N, static_cast<uint16_t *>(Y), acc,
                                          static_cast<const char *>(workspace), L, stream));
    const int8_t *WO =
        cache ? static_cast<const int8_t *>(cache) + cache_layout(K, N).WO : nullptr;
    return from_hip(launch_gemm(Wq, sW, T, K, N, static_cast<uint16_t *>(Y), acc,
                                static_cast<const char *>(workspace), L, W16 != nullptr, stream,
                                WO));
}

li8_status check_cache(const void *cache, size_t cache_bytes, int64_t K, int64_t N)
{
    if (!cache)
        return LI8_ERR_INVALID_ARG;
    if (misaligned(cache))
        return LI8_ERR_ALIGN;
    if (cache_bytes < cache_layout(K, N).total)
        return LI8_ERR_WORKSPACE;
    return LI8_OK;
}

// W16 null: the int8 path; else the fp16-weight variant.
li8_status linear_common(const void *X, const int8_t *Wq, const float *sW, const uint16_t *W16,
                         float threshold, int64_t T, int64_t K, int64_t N, void *Y,
                         void *workspace, hipStream_t stream)
{
    // few tokens: one kernel, bit-identical to the prepare + gemm pair
    if (decode_shape(T, K))
        return from_hip(launch_decode_fused(static_cast<const uint16_t *>(X), Wq, sW, W16,
                                            threshold_magnitude(threshold), T, K, N,
                                            static_cast<uint16_t *>(Y), stream));
    if (split_shape(T, K))
        return from_hip(launch_split_fused(static_cast<const uint16_t *>(X), Wq, sW, W16,
                                           threshold_magnitude(threshold), T, K, N,
                                           static_cast<uint16_t *>(Y), static_cast<char *>(workspace),
                                           stream));
    const WsLayout L = ws_layout(T, K, N);
    hipError_t e = launch_prepare(static_cast<const uint16_t *>(X), Wq, W16,
                                  threshold_magnitude(threshold), T, K, N,
                                  static_cast<char *>(workspace), L, stream, nullptr,
                                  gather_above(T, K, N, W16 != nullptr, false));
    if (e != hipSuccess)
        return LI8_ERR_HIP;
    return from_hip(launch_gemm(Wq, sW, T, K, N, static_cast<uint16_t *>(Y), nullptr,
                                static_cast<const char *>(workspace), L, W16 != nullptr, stream));
}

// Device address of `scratch` on the device that runs `stream`, looked up
// once per device with that device current.
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
char *g_scratch_ptr[kMaxDevices];

li8_status scratch_for(hipStream_t stream, char **out)
{
    int cur = 0;
    hipDevice_t dev = 0;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(stream, &dev) != hipSuccess)
        return LI8_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices)
        return LI8_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess)
            return LI8_ERR_HIP;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess)
            return LI8_ERR_HIP;
        if (e != hipSuccess || !p)
            return LI8_ERR_HIP;
        g_scratch_ptr[dev] = static_cast<char *>(p);
    }
    *out = g_scratch_ptr[dev];
    return LI8_OK;
}

} // namespace

extern "C" {

const char *li8_status_str(li8_status s)
{
    switch (s) {
    case LI8_OK: return "LI8_OK";
    case LI8_ERR_INVALID_ARG: return "LI8_ERR_INVALID_ARG";
    case LI8_ERR_SHAPE: return "LI8_ERR_SHAPE";
    case LI8_ERR_ALIGN: return "LI8_ERR_ALIGN";
    case LI8_ERR_WORKSPACE: return "LI8_ERR_WORKSPACE";
    case LI8_ERR_HIP: return "LI8_ERR_HIP";
    case LI8_ERR_SCRATCH: return "LI8_ERR_SCRATCH";
    }
    return "LI8_UNKNOWN_STATUS";
}

li8_status int8_quantize_weight(const void *W, int64_t N, int64_t K, int8_t *Wq, float *sW,
                                hipStream_t stream)
{
    li8_status st = check_shape(1, K, N);
    if (st != LI8_OK)
        return st;
    if (N == 0)
        return LI8_OK;
    if (!W || !Wq || !sW)
        return LI8_ERR_INVALID_ARG;
    if (misaligned(W) || misaligned(Wq) || misaligned(sW))
        return LI8_ERR_ALIGN;
    return from_hip(launch_quantize_weight(static_cast<const uint16_t *>(W), N, K, Wq, sW,
                                           stream));
}

size_t llm_int8_workspace_bytes(int64_t T, int64_t K, int64_t N)
{
    if (check_shape(T, K, N) != LI8_OK)
        return 0;
    const size_t a = ws_need(T, K, N, WS_WIDE), b = linear_need(T, K, N, WS_WIDE);
    return a > b ? a : b;
}

size_t llm_int8_linear_workspace_bytes(int64_t T, int64_t K, int64_t N)
{
    if (check_shape(T, K, N) != LI8_OK || T == 0 || N == 0)
        return 0;
    return linear_need(T, K, N, WS_I8);
}

li8_status llm_int8_plan(int64_t T, int64_t K, int64_t N, int32_t *path, int32_t *tile_m,
                         int32_t *tile_n, int32_t *fold_lo, int32_t *fold_hi)
{
    li8_status st = check_shape(T, K, N);
    if (st != LI8_OK)
        return st;
    if (!path || !tile_m || !tile_n || !fold_lo || !fold_hi)
        return LI8_ERR_INVALID_ARG;
    *fold_lo = *fold_hi = 0;
    if (T == 0 || N == 0) {
        *path = LI8_PATH_EMPTY;
        *tile_m = *tile_n = 0;
    } else if (decode_shape(T, K)) {
        *path = LI8_PATH_FEW_TOKENS;
        *tile_m = (int32_t)T;
        *tile_n = 16;
    } else if (split_shape(T, K)) {
        *path = LI8_PATH_FEW_TOKENS_SPLIT;
        *tile_m = (int32_t)T;
        *tile_n = 16;
    } else {
        const GemmPlan p = gemm_plan(T, K, N);
        const GatherSkip g = gather_above(T, K, N, false, false);
        *path = LI8_PATH_TILED;
        *tile_m = p.bm;
        *tile_n = p.bn;
        if (g.hi > g.lo) {
            *fold_lo = g.lo;
            *fold_hi = g.hi;
        }
    }
    return LI8_OK;
}

li8_status llm_int8_prepare(const void *X, const int8_t *Wq, float threshold, int64_t T,
                            int64_t K, int64_t N, void *workspace, size_t workspace_bytes,
                            hipStream_t stream)
{
    li8_status st =
        check_linear_args(X, Wq, threshold, T, K, N, workspace, workspace_bytes, WS_I8);
    if (st != LI8_OK || T == 0 || N == 0)
        return st;
    const WsLayout L = ws_layout(T, K, N);
    return from_hip(launch_prepare(static_cast<const uint16_t *>(X), Wq, nullptr,
                                   threshold_magnitude(threshold), T, K, N,
                                   static_cast<char *>(workspace), L, stream, nullptr,
                                   gather_above(T, K, N, false, false)));
}

li8_status llm_int8_prepare_fp16w(const void *X, const void *W, float threshold, int64_t T,
                                  int64_t K, int64_t N, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream)
{
    li8_status st = check_linear_args(X, static_cast<const int8_t *>(W), threshold, T, K, N,
                                      workspace, workspace_bytes, WS_WIDE);
    if (st != LI8_OK || T == 0 || N == 0)
        return st;
    const WsLayout L = ws_layout(T, K, N);
    return from_hip(launch_prepare(static_cast<const uint16_t *>(X), nullptr,
                                   static_cast<const uint16_t *>(W), threshold_magnitude(threshold),
                                   T, K, N, static_cast<char *>(workspace), L, stream, nullptr,
                                   gather_above(T, K, N, true, false)));
}

li8_status llm_int8_gemm(const int8_t *Wq, const float *sW, int64_t T, int64_t K, int64_t N,
                         void *Y, int32_t *acc, const void *workspace, size_t workspace_bytes,
                         hipStream_t stream)
{
    li8_status st = check_gemm_args(Wq, sW, T, K, N, Y, acc, workspace, workspace_bytes, WS_I8);
    if (st != LI8_OK || T == 0 || N == 0)
        return st;
    return gemm_common(Wq, sW, nullptr, T, K, N, Y, acc, workspace, stream);
}

li8_status llm_int8_gemm_fp16w(const int8_t *Wq, const float *sW, const void *W, int64_t T,
                               int64_t K, int64_t N, void *Y, int32_t *acc, const void *workspace,
                               size_t workspace_bytes, hipStream_t stream)
{
    li8_status st =
        check_gemm_args(Wq, sW, T, K, N, Y, acc, workspace, workspace_bytes, WS_WIDE);
    if (st == LI8_OK && T > 0 && N > 0 && K > 0) {
        if (!W)
            st = LI8_ERR_INVALID_ARG;
        else if (misaligned(W))
            st = LI8_ERR_ALIGN;
    }
    if (st != LI8_OK || T == 0 || N == 0)
        return st;
    return gemm_common(Wq, sW, static_cast<const uint16_t *>(W), T, K, N, Y, acc, workspace,
                       stream);
}

li8_status llm_int8_linear(const void *X, const int8_t *Wq, const float *sW, float threshold,
                           int64_t T, int64_t K, int64_t N, void *Y, void *workspace,
                           size_t workspace_bytes, hipStream_t stream)
{
    li8_status st = check_linear_args(X, Wq, threshold, T, K, N, workspace, workspace_bytes,
                                      WS_I8, ONE_CALL);
    if (st == LI8_OK)
        st = check_gemm_args(Wq, sW, T, K, N, Y, nullptr, workspace, workspace_bytes, WS_I8,
                             ONE_CALL);
    if (st != LI8_OK || T == 0 || N == 0)
        return st;
    return linear_common(X, Wq, sW, nullptr, threshold, T, K, N, Y, workspace, stream);
}

li8_status llm_int8_linear_noalloc(const void *X, const int8_t *Wq, const float *sW,
                                   float threshold, int64_t T, int64_t K, int64_t N, void *Y,
                                   hipStream_t stream)
{
    // (the workspace is the scratch array, checked below)
    li8_status st = check_linear_args(X, Wq, threshold, T, K, N, nullptr, 0, WS_I8, ONE_CALL);
    if (st == LI8_ERR_WORKSPACE)
        st = LI8_OK;
    if (st == LI8_OK)
        st = check_gemm_args(Wq, sW, T, K, N, Y, nullptr, nullptr, 0, WS_I8, ONE_CALL);
    if (st == LI8_ERR_WORKSPACE)
        st = LI8_OK;
    if (st != LI8_OK || T == 0 || N == 0)
        return st;
    char *ws = nullptr;
    const size_t need = linear_need(T, K, N, WS_I8);
    if (need > 0) {
        if (need > (size_t)LI8_NOALLOC_SCRATCH_BYTES)
            return LI8_ERR_SCRATCH;
        st = scratch_for(stream, &ws);
        if (st != LI8_OK)
            return st;
    }
    return linear_common(X, Wq, sW, nullptr, threshold, T, K, N, Y, ws, stream);
}

li8_status llm_int8_linear_fp16w(const void *X, const int8_t *Wq, const float *sW, const void *W,
                                 float threshold, int64_t T, int64_t K, int64_t N, void *Y,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    li8_status st = check_linear_args(X, Wq, threshold, T, K, N, workspace, workspace_bytes,
                                      WS_WIDE, ONE_CALL);
    if (st == LI8_OK)
        st = check_gemm_args(Wq, sW, T, K, N, Y, nullptr, workspace, workspace_bytes, WS_WIDE,
                             ONE_CALL);
    if (st == LI8_OK && T > 0 && N > 0 && K > 0) {
        if (!W)
            st = LI8_ERR_INVALID_ARG;
        else if (misaligned(W))
            st = LI8_ERR_ALIGN;
    }
    if (st != LI8_OK || T == 0 || N == 0)
        return st;
    return linear_common(X, Wq, sW, static_cast<const uint16_t *>(W), threshold, T, K, N, Y,
                         workspace, stream);
}

li8_status smoothquant_column_absmax(const void *A, int64_t rows, int64_t K, float *absmax,
                                     hipStream_t stream)
{
    li8_status st = check_shape(1, K, 1);
    if (st != LI8_OK)
        return st;
    if (rows < 0 || rows >= ((int64_t)1 << 31))
        return LI8_ERR_SHAPE;
    if (K == 0)
        return LI8_OK;
    if ((rows > 0 && !A) || !absmax)
        return LI8_ERR_INVALID_ARG;
    if (misaligned(A) || misaligned(absmax))
        return LI8_ERR_ALIGN;
    return from_hip(
        launch_column_absmax(static_cast<const uint16_t *>(A), rows, K, absmax, stream));
}

li8_status smoothquant_factors(const float *ax, const float *aw, double alpha, int64_t K,
                               float *s, float *s_inv, hipStream_t stream)
{
    li8_status st = check_shape(1, K, 1);
    if (st != LI8_OK)
        return st;
    if (!(alpha >= 0.0 && alpha <= 1.0))
        return LI8_ERR_INVALID_ARG;
    if (K == 0)
        return LI8_OK;
    if (!ax || !aw || !s || !s_inv)
        return LI8_ERR_INVALID_ARG;
    if (misaligned(ax) || misaligned(aw) || misaligned(s) || misaligned(s_inv))
        return LI8_ERR_ALIGN;
    return from_hip(launch_sq_factors(ax, aw, alpha, K, s, s_inv, stream));
}

li8_status smoothquant_quantize_weight(const void *W, const float *s, int64_t N, int64_t K,
                                       int8_t *Wq, float *sW, hipStream_t stream)
{
    li8_status st = check_shape(1, K, N);
    if (st != LI8_OK)
        return st;
    if (N == 0)
        return LI8_OK;
    if ((K > 0 && (!W || !s || !Wq)) || !sW)
        return LI8_ERR_INVALID_ARG;
    if (misaligned(W) || misaligned(s) || misaligned(Wq) || misaligned(sW))
        return LI8_ERR_ALIGN;
    return from_hip(
        launch_sq_quantize_weight(static_cast<const uint16_t *>(W), s, N, K, Wq, sW, stream));
}

li8_status smoothquant_prepare(const void *X, const float *s_inv, int64_t T, int64_t K,
                               int64_t N, void *workspace, size_t workspace_bytes,
                               hipStream_t stream)
{
    // the threshold is unused here; 0 passes the check
    li8_status st = check_linear_args(X, reinterpret_cast<const int8_t *>(s_inv), 0.0f, T, K, N,
                                      workspace, workspace_bytes, WS_I8);
    if (st != LI8_OK || T == 0 || N == 0)
        return st;
    return from_hip(launch_sq_prepare(static_cast<const uint16_t *>(X), s_inv, T, K,
                                      static_cast<char *>(workspace), ws_layout(T, K, N), stream));
}

li8_status smoothquant_linear(const void *X, const float *s_inv, const int8_t *Wq,
                              const float *sW, int64_t T, int64_t K, int64_t N, void *Y,
                              void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    li8_status st = check_linear_args(X, reinterpret_cast<const int8_t *>(s_inv), 0.0f, T, K, N,
                                      workspace, workspace_bytes, WS_I8);
    if (st == LI8_OK)
        st = check_gemm_args(Wq, sW, T, K, N, Y, nullptr, workspace, workspace_bytes, WS_I8);
    if (st != LI8_OK || T == 0 || N == 0)
        return st;
    hipError_t e = launch_sq_prepare(static_cast<const uint16_t *>(X), s_inv, T, K,
                                     static_cast<char *>(workspace), ws_layout(T, K, N), stream);
    if (e != hipSuccess)
        return LI8_ERR_HIP;
    return gemm_common(Wq, sW, nullptr, T, K, N, Y, nullptr, workspace, stream);
}

size_t llm_int8_cache_bytes(int64_t K, int64_t N)
{
    if (check_shape(1, K, N) != LI8_OK)
        return 0;
    return cache_layout(K, N).total;
}

li8_status llm_int8_cache_reset(void *cache, size_t cache_bytes, int64_t K, int64_t N,
                                hipStream_t stream)
{
    li8_status st = check_shape(1, K, N);
    if (st == LI8_OK)
        st = check_cache(cache, cache_bytes, K, N);
    if (st != LI8_OK)
        return st;
    return from_hip(launch_cache_reset(static_cast<char *>(cache), stream));
}

li8_status llm_int8_prepare_cached(const void *X, const int8_t *Wq, float threshold, int64_t T,
                                   int64_t K, int64_t N, void *workspace, size_t workspace_bytes,
                                   void *cache, size_t cache_bytes, hipStream_t stream)
{
    li8_status st =
        check_linear_args(X, Wq, threshold, T, K, N, workspace, workspace_bytes, WS_I8);
    if (st == LI8_OK && T > 0 && N > 0)
        st = check_cache(cache, cache_bytes, K, N);
    if (st != LI8_OK || T == 0 || N == 0)
        return st;
    // few tokens: the workspace GEMM gathers the outlier weights by index
    // itself; the cache is neither read nor written
    const bool use = !decode_shape(T, K) && !split_shape(T, K);
    return from_hip(launch_prepare(static_cast<const uint16_t *>(X), Wq, nullptr,
                                   threshold_magnitude(threshold), T, K, N,
                                   static_cast<char *>(workspace), ws_layout(T, K, N), stream,
                                   use ? static_cast<char *>(cache) : nullptr,
                                   gather_above(T, K, N, false, use)));
}

li8_status llm_int8_gemm_cached(const int8_t *Wq, const float *sW, int64_t T, int64_t K, int64_t N,
                                void *Y, int32_t *acc, const void *workspace,
                                size_t workspace_bytes, const void *cache, size_t cache_bytes,
                                hipStream_t stream)
{
    li8_status st = check_gemm_args(Wq, sW, T, K, N, Y, acc, workspace, workspace_bytes, WS_I8);
    if (st == LI8_OK && T > 0 && N > 0)
        st = check_cache(cache, cache_bytes, K, N);
    if (st != LI8_OK || T == 0 || N == 0)
        return st;
    return gemm_common(Wq, sW, nullptr, T, K, N, Y, acc, workspace, stream, cache);
}

li8_status llm_int8_linear_cached(const void *X, const int8_t *Wq, const float *sW,
                                  float threshold, int64_t T, int64_t K, int64_t N, void *Y,
                                  void *workspace, size_t workspace_bytes, void *cache,
                                  size_t cache_bytes, hipStream_t stream)
{
    li8_status st = check_linear_args(X, Wq, threshold, T, K, N, workspace, workspace_bytes,
                                      WS_I8, ONE_CALL);
    if (st == LI8_OK)
        st = check_gemm_args(Wq, sW, T, K, N, Y, nullptr, workspace, workspace_bytes, WS_I8,
                             ONE_CALL);
    if (st == LI8_OK && T > 0 && N > 0)
        st = check_cache(cache, cache_bytes, K, N);
    if (st != LI8_OK || T == 0 || N == 0)
        return st;
    if (decode_shape(T, K) || split_shape(T, K))   // few tokens: the cache is not used
        return linear_common(X, Wq, sW, nullptr, threshold, T, K, N, Y, workspace, stream);
    const WsLayout L = ws_layout(T, K, N);
    hipError_t e = launch_prepare(static_cast<const uint16_t *>(X), Wq, nullptr,
                                  threshold_magnitude(threshold), T, K, N,
                                  static_cast<char *>(workspace), L, stream,
                                  static_cast<char *>(cache), gather_above(T, K, N, false, true));
    if (e != hipSuccess)
        return LI8_ERR_HIP;
    return gemm_common(Wq, sW, nullptr, T, K, N, Y, nullptr, workspace, stream, cache);
}

li8_status llm_int8_export_stages(const void *workspace, size_t workspace_bytes, int64_t T,
                                  int64_t K, int64_t N, uint32_t *outlier_bits,
                                  int32_t *n_outliers, int32_t *outlier_idx, int8_t *Xq,
                                  float *sX, void *X_out, hipStream_t stream)
{
    li8_status st = check_shape(T, K, N);
    if (st != LI8_OK)
        return st;
    const WsLayout L = ws_layout(T, K, N);
    if (!workspace || workspace_bytes < L.WO)   // (the stages end where WO starts)
        return LI8_ERR_WORKSPACE;
    const char *ws = static_cast<const char *>(workspace);
    struct {
        void *dst;
        size_t off, bytes;
    } cp[] = {
        {outlier_bits, L.bits, 4 * (size_t)((K + 31) / 32)},
        {n_outliers, L.meta, 4},
        {outlier_idx, L.idx, 4 * (size_t)K},
        {Xq, L.Xq, (size_t)T * (size_t)K},
        {sX, L.sX, 4 * (size_t)T},
        {X_out, L.XO, 2 * (size_t)T * (size_t)K},
    };
    for (auto &c : cp) {
        if (!c.dst || c.bytes == 0)
            continue;
        hipError_t e = hipMemcpyAsync(c.dst, ws + c.off, c.bytes, hipMemcpyDeviceToDevice, stream);
        if (e != hipSuccess)
            return LI8_ERR_HIP;
    }
    return LI8_OK;
}

li8_status llm_int8_stages(const void *X, const int8_t *Wq, const float *sW, float threshold,
                           int64_t T, int64_t K, int64_t N, void *Y, void *workspace,
                           size_t workspace_bytes, uint8_t *flags, int32_t *n_outliers,
                           int32_t *outlier_idx, int8_t *Xq, float *sX, void *X_out, int32_t *acc,
                           hipStream_t stream)
{
    // every check before anything is enqueued
    li8_status st =
        check_linear_args(X, Wq, threshold, T, K, N, workspace, workspace_bytes, WS_I8);
    if (st == LI8_OK)
        st = check_gemm_args(Wq, sW, T, K, N, Y, acc, workspace, workspace_bytes, WS_I8);
    if (st == LI8_OK && (misaligned(Xq) || misaligned(sX) || misaligned(X_out)))
        st = LI8_ERR_ALIGN;
    if (st != LI8_OK || T == 0 || N == 0)
        return st;
    st = llm_int8_prepare(X, Wq, threshold, T, K, N, workspace, workspace_bytes, stream);
    if (st == LI8_OK)
        st = llm_int8_gemm(Wq, sW, T, K, N, Y, acc, workspace, workspace_bytes, stream);
    if (st == LI8_OK)
        st = llm_int8_export_stages(workspace, workspace_bytes, T, K, N, nullptr, n_outliers,
                                    outlier_idx, Xq, sX, nullptr, stream);
    if (st != LI8_OK || K == 0 || (!flags && !X_out))
        return st;
    const WsLayout L = ws_layout(T, K, N);
    const char *ws = static_cast<const char *>(workspace);
    const int64_t work = std::max<int64_t>(K, T * K);
    const unsigned blocks = (unsigned)std::min<int64_t>((work + 255) / 256, 4096);
    hipLaunchKernelGGL(k_stage_flags_xo, dim3(blocks), dim3(256), 0, stream,
                       reinterpret_cast<const uint32_t *>(ws + L.bits),
                       reinterpret_cast<const int32_t *>(ws + L.meta),
                       reinterpret_cast<const uint16_t *>(ws + L.XO), (int)T, (int)K, flags,
                       static_cast<uint16_t *>(X_out));
    return from_hip(hipGetLastError());
}

} // extern "C"
