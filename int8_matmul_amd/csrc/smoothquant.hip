// SmoothQuant-style W8A8 on the same int8 GEMM, for gfx950 (lowentro.cn
// "model quantization" notes, Q9: the rewrite; Q10: the factor, whose
// printed product form is garbled and is read as the quotient below, the
// form under which alpha = 0.5 balances the two smoothed ranges and
// alpha = 0 flattens the weight's; hncyxsy.com/news/230290, section 5.1).
//
// The rewrite x . W^T = (x / s) . (W * s)^T with one factor s_j per input
// channel moves quantization difficulty from the activation to the weight;
// both sides are then quantized with the absmax int8 scheme and multiplied
// with no outlier decomposition:
//   s_j  = ax_j^alpha / aw_j^(1-alpha)   (fp64, rounded to fp32; 1 when ax_j
//          or aw_j is 0), r_j = fl32(1 / s_j)
//   W'   = fl32(W * s_j),      sW = fl32(max_j |W'| / 127), codes rne(fl32(W'/sW))
//   X'   = fl32(X * r_j),      sX = fl32(max_j |X'| / 127), codes rne(fl32(X'/sX))
//   Y    = fp16(fl32(fl32(acc * sX) * sW))        (the GEMM with nO = 0)
// ax_j is the channel's absmax over a calibration batch of activations and
// aw_j the column absmax of W; the factors are computed once per layer.
// The smoothed values are fp32, so the codes use IEEE division (the
// reciprocal shortcut of the fp16 path was checked for fp16 inputs only).
#include "li8_internal.h"

namespace li8 {
namespace {

constexpr int kSThreads = 256;

__device__ __forceinline__ float h2f_sq(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// absmax code of an fp32 value for a scale s > 0, clamped to [-127, 127]
__device__ __forceinline__ int sq_code(float v, float s)
{
    const float q = fminf(fmaxf(rintf(v / s), -127.0f), 127.0f);
    return (int)q;
}

__device__ __forceinline__ float block_max_f(float v, float *red)
{
    for (int o = 32; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, 64));
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    if (lane == 0)
        red[wid] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < kSThreads / 64; i++)
        r = fmaxf(r, red[i]);
    __syncthreads();
    return r;
}

// ---- column absmax: out[j] = max_r |A[r,j]| (out pre-filled with 0) ----
__global__ __launch_bounds__(kSThreads) void k_fill0(uint32_t *out, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * kSThreads + threadIdx.x;
    if (i < n)
        out[i] = 0u;
}

// Block (x, y): columns 8*(x*256 + tid) .. +7 over rows [y*R, y*R + R).
// Non-negative floats order like their bit patterns, so an integer atomic
// max on the fp32 bits of |a| is the float max.
__global__ __launch_bounds__(kSThreads) void k_colmax(const uint16_t *__restrict__ A, int64_t rows,
                                                      int K, int R, uint32_t *__restrict__ out)
{
    const int c = blockIdx.x * kSThreads + threadIdx.x;   // 8-column chunk
    if (c >= K / 8)
        return;
    const int64_t r0 = (int64_t)blockIdx.y * R, r1 = min<int64_t>(rows, r0 + R);
    uint32_t m[8] = {0, 0, 0, 0, 0, 0, 0, 0};   // fp16 magnitude patterns
    for (int64_t r = r0; r < r1; r++) {
        const uint4 v = reinterpret_cast<const uint4 *>(A + r * K)[c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; e++)
            m[e] = max(m[e], (w[e >> 1] >> (16 * (e & 1))) & 0x7fffu);
    }
#pragma unroll
    for (int e = 0; e < 8; e++)
        if (m[e])
            atomicMax(out + 8 * c + e, __builtin_bit_cast(uint32_t, h2f_sq(m[e])));
}

// ---- factors ----
__global__ __launch_bounds__(kSThreads) void k_sq_factors(const float *__restrict__ ax,
                                                          const float *__restrict__ aw,
                                                          double alpha, int K,
                                                          float *__restrict__ s,
                                                          float *__restrict__ r)
{
    const int j = blockIdx.x * kSThreads + threadIdx.x;
    if (j >= K)
        return;
    float f = 1.0f;
    if (ax[j] != 0.0f && aw[j] != 0.0f)
        f = (float)(pow((double)ax[j], alpha) / pow((double)aw[j], 1.0 - alpha));
    s[j] = f;
    r[j] = 1.0f / f;
}

// ---- smoothed weight quantization: one block per weight row ----
__global__ __launch_bounds__(kSThreads) void k_sq_quantize_weight(
    const uint16_t *__restrict__ W, const float *__restrict__ s, int K, int8_t *__restrict__ Wq,
    float *__restrict__ sW)
{
    __shared__ float red[kSThreads / 64];
    const int64_t n = blockIdx.x;
    const uint16_t *w = W + n * K;
    float a = 0.0f;
    for (int j = threadIdx.x; j < K; j += kSThreads)
        a = fmaxf(a, fabsf(h2f_sq(w[j]) * s[j]));
    a = block_max_f(a, red);
    const float sc = a / 127.0f;
    if (threadIdx.x == 0)
        sW[n] = sc;
    for (int j = threadIdx.x; j < K; j += kSThreads)
        Wq[n * K + j] = sc > 0.0f ? (int8_t)sq_code(h2f_sq(w[j]) * s[j], sc) : (int8_t)0;
}

// ---- the per-call activation side: one block per token row ----
// Writes Xq (codes of X * r), sX, and meta[0] = 0 outlier columns (block 0)
// for the GEMM.  The smoothed row is kept in registers between the absmax
// pass and the code pass for K <= 8 * 256 * kSq; longer rows are re-read.
// kSq (8-column chunks per thread held in registers) is chosen from K at
// launch, so that no thread issues loads for chunks past the row.
template <int kSq>
__global__ __launch_bounds__(kSThreads) void k_sq_rows(const uint16_t *__restrict__ X,
                                                       const float *__restrict__ r, int K,
                                                       int8_t *__restrict__ Xq,
                                                       float *__restrict__ sX,
                                                       int32_t *__restrict__ meta)
{
    __shared__ float red[kSThreads / 64];
    const int64_t t = blockIdx.x;
    const int nchunk = K / 8;
    const uint4 *xr = reinterpret_cast<const uint4 *>(X + t * K);
    const float4 *r4 = reinterpret_cast<const float4 *>(r);
    if (t == 0 && threadIdx.x == 0)
        meta[0] = 0;
    if (nchunk == 0) {   // K = 0: an empty row
        if (threadIdx.x == 0)
            sX[t] = 0.0f;
        return;
    }
    auto smooth = [&](int c, float v[8]) {
        const uint4 x = xr[c];
        const float4 ra = r4[2 * c], rb = r4[2 * c + 1];
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
        const float rr[8] = {ra.x, ra.y, ra.z, ra.w, rb.x, rb.y, rb.z, rb.w};
#pragma unroll
        for (int e = 0; e < 8; e++)
            v[e] = h2f_sq((w[e >> 1] >> (16 * (e & 1))) & 0xffffu) * rr[e];
    };
    // the register-held chunks are loaded unconditionally (a chunk past
    // the row re-reads the last one and is not used), so that all loads are
    // in flight together: loads behind branches make the compiler wait for
    // each before the next
    float v[kSq][8];
    float a = 0.0f;
#pragma unroll
    for (int u = 0; u < kSq; u++)
        smooth(min((int)threadIdx.x + u * kSThreads, nchunk - 1), v[u]);
#pragma unroll
    for (int u = 0; u < kSq; u++)
        if ((int)threadIdx.x + u * kSThreads < nchunk)
#pragma unroll
            for (int e = 0; e < 8; e++)
                a = fmaxf(a, fabsf(v[u][e]));
    for (int c = threadIdx.x + kSq * kSThreads; c < nchunk; c += kSThreads) {
        float w8[8];
        smooth(c, w8);
#pragma unroll
        for (int e = 0; e < 8; e++)
            a = fmaxf(a, fabsf(w8[e]));
    }
    a = block_max_f(a, red);
    const float sc = a / 127.0f;
    if (threadIdx.x == 0)
        sX[t] = sc;
    uint2 *q = reinterpret_cast<uint2 *>(Xq + t * K);
    auto emit = [&](int c, const float w8[8]) {
        uint32_t lo = 0, hi = 0;
        if (sc > 0.0f) {
#pragma unroll
            for (int e = 0; e < 4; e++)
                lo |= ((uint32_t)sq_code(w8[e], sc) & 0xffu) << (8 * e);
#pragma unroll
            for (int e = 0; e < 4; e++)
                hi |= ((uint32_t)sq_code(w8[4 + e], sc) & 0xffu) << (8 * e);
        }
        q[c] = make_uint2(lo, hi);
    };
#pragma unroll
    for (int u = 0; u < kSq; u++) {
        const int c = threadIdx.x + u * kSThreads;
        if (c < nchunk)
            emit(c, v[u]);
    }
    for (int c = threadIdx.x + kSq * kSThreads; c < nchunk; c += kSThreads) {
        float w8[8];
        smooth(c, w8);
        emit(c, w8);
    }
}

} // namespace

hipError_t launch_column_absmax(const uint16_t *A, int64_t rows, int64_t K, float *out,
                                hipStream_t s)
{
    if (K == 0)
        return hipSuccess;
    uint32_t *o = reinterpret_cast<uint32_t *>(out);
    hipLaunchKernelGGL(k_fill0, dim3((unsigned)((K + kSThreads - 1) / kSThreads)), dim3(kSThreads),
                       0, s, o, K);
    if (rows > 0) {
        const int gx = (int)((K / 8 + kSThreads - 1) / kSThreads);
        const int gy = (int)std::min<int64_t>(rows, 1024);
        const int R = (int)((rows + gy - 1) / gy);
        hipLaunchKernelGGL(k_colmax, dim3(gx, (unsigned)((rows + R - 1) / R)), dim3(kSThreads), 0, s,
                           A, rows, (int)K, R, o);
    }
    return hipGetLastError();
}

hipError_t launch_sq_factors(const float *ax, const float *aw, double alpha, int64_t K, float *sf,
                             float *r, hipStream_t s)
{
    hipLaunchKernelGGL(k_sq_factors, dim3((unsigned)((K + kSThreads - 1) / kSThreads)),
                       dim3(kSThreads), 0, s, ax, aw, alpha, (int)K, sf, r);
    return hipGetLastError();
}

hipError_t launch_sq_quantize_weight(const uint16_t *W, const float *sf, int64_t N, int64_t K,
                                     int8_t *Wq, float *sW, hipStream_t s)
{
    hipLaunchKernelGGL(k_sq_quantize_weight, dim3((unsigned)N), dim3(kSThreads), 0, s, W, sf, (int)K,
                       Wq, sW);
    return hipGetLastError();
}

hipError_t launch_sq_prepare(const uint16_t *X, const float *r, int64_t T, int64_t K, char *ws,
                             const WsLayout &L, hipStream_t s)
{
    const int64_t need = (K / 8 + kSThreads - 1) / kSThreads;   // chunks per thread
    auto kern = need <= 1 ? k_sq_rows<1> : need <= 2 ? k_sq_rows<2> : k_sq_rows<4>;
    hipLaunchKernelGGL(kern, dim3((unsigned)T), dim3(kSThreads), 0, s, X, r, (int)K,
                       reinterpret_cast<int8_t *>(ws + L.Xq), reinterpret_cast<float *>(ws + L.sX),
                       reinterpret_cast<int32_t *>(ws + L.meta));
    return hipGetLastError();
}

} // namespace li8
