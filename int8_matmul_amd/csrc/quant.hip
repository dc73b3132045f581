// Outlier detection and vector-wise int8 quantization kernels for gfx950.
//
// The method (hncyxsy.com/news/230290 "LLM quantization, part 2", section
// 2.1; lowentro.cn "model quantization" notes, Q2-Q4, Q11; tqpw.cn/news/5683,
// section 2.1):
//   outlier columns  O = { j : some |X[t,j]| > threshold }
//   token scale      sX[t] = max_{j not in O} |X[t,j]| / 127
//   token codes      Xq[t,j] = round(X[t,j] / sX[t]) clipped to [-127,127],
//                    0 for j in O
//   weight scale     sW[n] = max_k |W[n,k]| / 127, codes likewise.
// Scales are fp32 (IEEE division), codes round half to even.
//
// All three kernels are HBM-bound streaming passes: 16-byte coalesced
// loads, the row or column-strip reduction kept in registers, wave-level
// reductions, and a single atomic per 32 columns for the outlier bit set.
//
// Magnitudes are compared as integers: for a finite binary16 value h,
// |h| is monotone in (h & 0x7fff), so |x| > thr  <=>  (h & 0x7fff) > H,
// with H the largest binary16 magnitude pattern whose value is <= thr
// (computed on the host).  The same ordering gives the exact absmax.
#include <algorithm>

#include "li8_internal.h"
#include "quant_math.h"

namespace li8 {
namespace {

constexpr int kThreads = 256;
constexpr int kPrepRows = 2;   // token rows per quantization workgroup

// Block-wide max of a uint32 (all threads get the result).
__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t *red)
{
    v = wave_max(v);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    if (lane == 0)
        red[wid] = v;
    __syncthreads();
    uint32_t r = red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; i++)
        r = max(r, red[i]);
    __syncthreads();
    return r;
}

// Codes of 8 values packed little-endian into two words; positions whose
// bit in `skip` is set get code 0, and so does everything when s == 0 (an
// all-zero vector).
__device__ __forceinline__ uint2 codes8(uint4 v, uint32_t skip, float s, float r)
{
    if (s == 0.0f)
        return make_uint2(0u, 0u);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; e++) {
        const uint32_t h = (w[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        const int q = ((skip >> e) & 1u) ? 0 : code_of(h, s, r);
        out[e >> 2] |= ((uint32_t)q & 0xffu) << (8 * (e & 3));
    }
    return make_uint2(out[0], out[1]);
}

// ---------------------------------------------------------------------------
// Weight quantization: one block per output feature n.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_quantize_weight(
    const uint16_t *__restrict__ W, int K, int8_t *__restrict__ Wq, float *__restrict__ sW)
{
    __shared__ uint32_t red[kThreads / 64];
    const int64_t n = blockIdx.x;
    const uint4 *w = reinterpret_cast<const uint4 *>(W + n * (int64_t)K);
    const int nchunk = K / 8;
    uint32_t m = 0;
    for (int c = threadIdx.x; c < nchunk; c += kThreads)
        m = max(m, masked_max8(w[c], 0u));
    m = block_max(m, red);
    const float s = h2f(m) / 127.0f;
    const float r = 1.0f / s;
    if (threadIdx.x == 0)
        sW[n] = s;
    uint2 *q = reinterpret_cast<uint2 *>(Wq + n * (int64_t)K);
    for (int c = threadIdx.x; c < nchunk; c += kThreads)
        q[c] = codes8(w[c], 0u, s, r);
}

// ---------------------------------------------------------------------------
// Clear the outlier bit set and the meta words (a kernel rather than a
// memset so that the sequence stays capturable in a HIP graph).
// ---------------------------------------------------------------------------
__global__ void k_clear(uint32_t *__restrict__ bits, int nwords, int32_t *__restrict__ meta)
{
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < nwords)
        bits[i] = 0u;
    if (i < 64)
        meta[i] = 0;
}

// ---------------------------------------------------------------------------
// Outlier detection.  Block (x, y) covers 2048 columns (8 per thread) of
// rows [y*R, y*R+R).  Rows are read in batches of kDetectRows with every load of a
// batch issued before any is used (these short streaming kernels are
// latency-bound otherwise); rows past the end re-read the last row, which
// leaves the maximum unchanged.  The per-column magnitude max is kept
// packed in registers; one compare per column at the end; four lanes
// combine their 8-bit masks into one 32-bit word, and non-zero words are
// OR-ed into the bit set.
// ---------------------------------------------------------------------------
typedef li8_us2 us2;

constexpr int kDetectRows = 16;   // rows per load batch

__global__ __launch_bounds__(kThreads) void k_detect(
    const uint16_t *__restrict__ X, int T, int K, int R, uint32_t thr_mag,
    uint32_t *__restrict__ bits)
{
    const int nchunk = K / 8;
    const int c = blockIdx.x * kThreads + threadIdx.x;
    const int t0 = blockIdx.y * R;
    const int t1 = min(T, t0 + R);
    us2 mx[4] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
    if (c < nchunk) {
        const uint4 *p = reinterpret_cast<const uint4 *>(X) + c;
        const int64_t stride = K / 8;
        for (int tb = t0; tb < t1; tb += kDetectRows) {
            uint4 v[kDetectRows];
#pragma unroll
            for (int u = 0; u < kDetectRows; u++)
                v[u] = p[(int64_t)min(tb + u, t1 - 1) * stride];
#pragma unroll
            for (int u = 0; u < kDetectRows; u++)
                column_max8(mx, v[u]);
        }
    }
    const uint32_t m8 = outlier_flags8(mx, thr_mag);
    // chunk c holds columns 8c..8c+7 = bits 8*(c%4).. of word c/4
    uint32_t word = m8 << (8 * (c & 3));
    word |= (uint32_t)__shfl_xor((int)word, 1, 64);
    word |= (uint32_t)__shfl_xor((int)word, 2, 64);
    if ((c & 3) == 0 && c < nchunk && word != 0u)
        atomicOr(bits + (c >> 2), word);
}

// Bit-set words held in registers per thread by k_prepare (nw <= 256,
// i.e. K <= 8192); longer bit sets are read from global memory.
constexpr int kBitsPerThread = 1;

// Load the bit set into LDS and write the exclusive prefix of the
// popcounts per word; returns nO (the total) to every thread.  Thread tid
// owns words [tid*per, tid*per + per); with REG, bw already holds them
// (nw <= kBitsPerThread * kThreads).
template <bool REG>
__device__ int load_bits_and_scan(const uint32_t *__restrict__ bits_g, int nw,
                                  uint32_t *bits, int32_t *pre, int32_t *scan,
                                  const uint32_t (&bw)[kBitsPerThread])
{
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int per = (nw + kThreads - 1) / kThreads;
    const int w0 = min(nw, tid * per), w1 = min(nw, w0 + per);
    int s = 0;
    if constexpr (REG) {
        // (a select, not a branch, consumes bw: a load whose only use sits
        // in a branch is moved into it, behind the row loads)
#pragma unroll
        for (int i = 0; i < kBitsPerThread; i++) {
            const uint32_t b = (w0 + i < w1) ? bw[i] : 0u;
            s += __popc(b);
            if (w0 + i < w1)
                bits[w0 + i] = b;
        }
    } else {
        for (int w = w0; w < w1; w++) {
            uint32_t b = bits_g[w];
            bits[w] = b;
            s += __popc(b);
        }
    }
    // inclusive scan within the wave
    int v = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int u = __shfl_up(v, o, 64);
        if (lane >= o)
            v += u;
    }
    if (lane == 63)
        scan[wid] = v;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int i = 0; i < kThreads / 64; i++) {
        if (i < wid)
            base += scan[i];
        total += scan[i];
    }
    int p = base + v - s;   // exclusive prefix of this thread's first word
    for (int w = w0; w < w1; w++) {
        pre[w] = p;
        p += __popc(bits[w]);
    }
    __syncthreads();
    return total;
}

// ---------------------------------------------------------------------------
// Token quantization + outlier gathers.  Blocks [0, xblocks) each quantize
// kPrepRows token rows; the remaining blocks gather the outlier columns of
// wrows rows of Wq (or of the fp16 weight W16, in the fp16-weight variant)
// each.  Every block rebuilds the prefix counts of the bit set in LDS, which
// gives each outlier column its compact index.
// ---------------------------------------------------------------------------

// REG: the bit set fits in kBitsPerThread words per thread (K <= 8192).
// RREG: 16-byte chunks per thread and row kept in registers (2 when K <=
// 4096, else 4; columns past RREG * 8 * 256 are read again from memory).
template <int ROWS, bool REG, int RREG>
__global__ __launch_bounds__(kThreads) void k_prepare(
    const uint16_t *__restrict__ X, const int8_t *__restrict__ Wq,
    const uint16_t *__restrict__ W16, int T, int K, int N,
    int wrows, const uint32_t *__restrict__ bits_g, int32_t *__restrict__ meta,
    int32_t *__restrict__ idx_g, float *__restrict__ sX, int8_t *__restrict__ Xq,
    uint16_t *__restrict__ XO, int8_t *__restrict__ WO, int32_t *__restrict__ cache_hdr,
    uint32_t *__restrict__ cache_bits)
{
    extern __shared__ uint32_t smem[];
    __shared__ int32_t scan[kThreads / 64];
    __shared__ uint32_t redr[ROWS][kThreads / 64];
    __shared__ int nnz_s, miss_s;
    const int nw = (K + 31) / 32;
    uint32_t *bits = smem;
    int32_t *pre = reinterpret_cast<int32_t *>(smem + nw);
    const int tid = threadIdx.x;
    const int nchunk = K / 8;
    const int xblocks = (T + ROWS - 1) / ROWS;
    const bool xblock = (int)blockIdx.x < xblocks;
    const int t0 = blockIdx.x * ROWS;

    // Loads first, all unconditional: this thread's bit-set words, then the
    // token rows (buffer loads; chunks past the row and the lanes of
    // weight-gather blocks use offset 2^31, past the buffer whenever X is
    // under 2 GiB, else a valid address whose value is not used).  Loads behind branches would make the compiler wait for all
    // of them at the first use; this way the bit-set scan waits only for
    // the bit-set words (loads complete in order) while the rows arrive.
    uint32_t bw[kBitsPerThread] = {};
    if constexpr (REG) {
        const int per = (nw + kThreads - 1) / kThreads;
        const int w0 = tid * per, wl = nw > 0 ? nw - 1 : 0;   // (the region has >= 1 word)
#pragma unroll
        for (int i = 0; i < kBitsPerThread; i++)
            bw[i] = bits_g[min(w0 + i, wl)];
    }
    __builtin_amdgcn_sched_barrier(0);   // (keep the row loads after them)
    uint4 v[ROWS][RREG];
    {
        const __amdgpu_buffer_rsrc_t rX =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(X), (short)0,
                                              (int)(2u * (unsigned)T * (unsigned)K), 0x00020000);
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            const unsigned row = (unsigned)min(t0 + r, T - 1);
#pragma unroll
            for (int s = 0; s < RREG; s++) {
                const int c = tid + s * kThreads;
                const int off = (xblock & (c < nchunk)) ? (int)(16u * (row * (unsigned)nchunk + (unsigned)c))
                                                        : (int)0x80000000;
                v[r][s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rX, off, 0, 0));
            }
        }
    }
    const int nO = load_bits_and_scan<REG>(bits_g, nw, bits, pre, scan, bw);
    const int nO16 = (nO + 15) & ~15;   // <= K since K % 16 == 0

    if (xblock) {
        // this thread's bit-set words, skip masks and word ranks, read once
        // for all its rows and unconditionally (a clamped index; chunks
        // past K hold zeros and store nothing): a read under the lane test
        // would be a branch per read
        uint32_t wbits[RREG], skipm[RREG];
        int wpre[RREG];
#pragma unroll
        for (int s = 0; s < RREG; s++) {
            const int c = tid + s * kThreads, wi = min(c, nchunk - 1) >> 2;
            wbits[s] = bits[wi];
            wpre[s] = pre[wi];
            skipm[s] = (wbits[s] >> (8 * (c & 3))) & 0xffu;
        }
        uint32_t m[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            m[r] = 0;
#pragma unroll
            for (int s = 0; s < RREG; s++)
                m[r] = max(m[r], chunk_max(v[r][s], skipm[s]));
            const uint4 *xr = reinterpret_cast<const uint4 *>(X + (int64_t)min(t0 + r, T - 1) * K);
            for (int c = tid + RREG * kThreads; c < nchunk; c += kThreads)
                m[r] = max(m[r], chunk_max(xr[c], (bits[c >> 2] >> (8 * (c & 3))) & 0xffu));
        }
        // block-wide max of each row's value
        {
            const int lane = tid & 63, wid = tid >> 6;
#pragma unroll
            for (int r = 0; r < ROWS; r++) {
                const uint32_t wmax = wave_max(m[r]);
                if (lane == 0)
                    redr[r][wid] = wmax;
            }
            __syncthreads();
#pragma unroll
            for (int r = 0; r < ROWS; r++) {
                uint32_t x = redr[r][0];
#pragma unroll
                for (int i = 1; i < kThreads / 64; i++)
                    x = max(x, redr[r][i]);
                m[r] = x;
            }
        }
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            const int64_t t = t0 + r;
            if (t >= T)
                break;
            const float sc = h2f(m[r]) / 127.0f;
            const float rc = 1.0f / sc;
            if (tid == 0)
                sX[t] = sc;
            uint2 *q = reinterpret_cast<uint2 *>(Xq + t * K);
            // outlier values in 16-column chunks: rank i of row t at
            // ((i / 16) * T + t) * 16 + i % 16
            auto xo = [&](int i) -> uint16_t & { return XO[((int64_t)(i >> 4) * T + t) * 16 + (i & 15)]; };
            auto emit = [&](int c, uint4 x, uint32_t wb, uint32_t skip, int wp) {
                q[c] = (sc == 0.0f) ? make_uint2(0u, 0u) : token_codes8(x, skip, sc, rc);
                if (skip) {
                    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
                    const int b0 = 8 * (c & 3);
                    int i = wp + __popc(wb & ((1u << b0) - 1u));
#pragma unroll
                    for (int e = 0; e < 8; e++)
                        if ((skip >> e) & 1u)
                            xo(i++) = (uint16_t)((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
                }
            };
#pragma unroll
            for (int s2 = 0; s2 < RREG; s2++) {
                const int c = tid + s2 * kThreads;
                if (c < nchunk)
                    emit(c, v[r][s2], wbits[s2], skipm[s2], wpre[s2]);
            }
            const uint4 *xr = reinterpret_cast<const uint4 *>(X + t * K);
            for (int c = tid + RREG * kThreads; c < nchunk; c += kThreads) {
                const uint32_t wb = bits[c >> 2];
                emit(c, xr[c], wb, (wb >> (8 * (c & 3))) & 0xffu, pre[c >> 2]);
            }
            if (tid < nO16 - nO)
                xo(nO + tid) = 0;
        }
        return;
    }

    // ---- outlier columns of wrows weight rows ----
    const int wb = blockIdx.x - xblocks;
    const int n0 = wb * wrows;
    const int n1 = min(N, n0 + wrows);
    if (wb == 0) {
        for (int w = tid; w < nw; w += kThreads) {
            uint32_t b = bits[w];
            int p = pre[w];
            while (b) {
                idx_g[p++] = 32 * w + __ffs(b) - 1;
                b &= b - 1u;
            }
        }
        if (tid == 0)
            meta[0] = nO;
    }
    // Outlier-column cache (cache_hdr non-null): WO is the cache's copy of
    // the gathered columns.  If the cache holds this call's exact set, the
    // gather is skipped.  Every gather block decides alike (nothing writes
    // the cached set during this kernel); k_cache_commit, the next kernel,
    // records the set.
    bool miss = true;
    if (cache_hdr) {
        if (tid == 0)
            miss_s = cache_hdr[0] != 1;
        __syncthreads();
        bool diff = false;
        for (int w = tid; w < nw; w += kThreads)
            diff |= bits[w] != cache_bits[w];
        if (diff)
            atomicOr(&miss_s, 1);
        __syncthreads();
        miss = miss_s != 0;
    }
    if (!miss || nO == 0)   // nothing to gather
        return;
    // list the non-zero words once (one wave, ballot compaction), then
    // visit (row, non-zero word) pairs only
    int *nzw = reinterpret_cast<int *>(pre + nw);
    if (tid < 64) {
        int cnt = 0;
        for (int base = 0; base < nw; base += 64) {
            const int w = base + tid;
            const bool nz = w < nw && bits[w] != 0u;
            const uint64_t mask = __ballot(nz);
            if (nz)
                nzw[cnt + __popcll(mask & ((1ull << tid) - 1ull))] = w;
            cnt += __popcll(mask);
        }
        if (tid == 0)
            nnz_s = cnt;
    }
    __syncthreads();
    const int nnz = nnz_s;
    const int pairs = (n1 - n0) * nnz;
    if (W16) {   // fp16-weight variant: the outlier columns of W, as fp16
        uint16_t *WO16 = reinterpret_cast<uint16_t *>(WO);
        for (int p = tid; p < pairs; p += kThreads) {
            const int n = n0 + p / nnz;
            const int w = nzw[p - (p / nnz) * nnz];
            uint32_t b = bits[w];
            const uint16_t *src = W16 + (int64_t)n * K + 32 * w;
            uint32_t hw[16];   // the word's 32 columns, two per register
#pragma unroll
            for (int q = 0; q < 4; q++) {
                uint4 v = make_uint4(0, 0, 0, 0);
                if (32 * w + 8 * q < K)
                    v = *reinterpret_cast<const uint4 *>(src + 8 * q);
                hw[4 * q] = v.x;
                hw[4 * q + 1] = v.y;
                hw[4 * q + 2] = v.z;
                hw[4 * q + 3] = v.w;
            }
            // (16-column chunks: rank i of row n at ((i / 16) * N + n) * 16 + i % 16)
            int i = pre[w];
            while (b) {
                const int j = __ffs(b) - 1;
                WO16[((int64_t)(i >> 4) * N + n) * 16 + (i & 15)] = (uint16_t)((hw[j >> 1] >> (16 * (j & 1))) & 0xffffu);
                i++;
                b &= b - 1u;
            }
        }
        for (int p = tid; p < (n1 - n0) * 16; p += kThreads) {
            const int n = n0 + p / 16, e = p % 16;
            if (nO + e < nO16)
                WO16[((int64_t)((nO + e) >> 4) * N + n) * 16 + ((nO + e) & 15)] = 0;
        }
        return;
    }
    for (int p = tid; p < pairs; p += kThreads) {
        const int n = n0 + p / nnz;
        const int w = nzw[p - (p / nnz) * nnz];
        uint32_t b = bits[w];
        const int8_t *src = Wq + (int64_t)n * K + 32 * w;
        uint4 lo = *reinterpret_cast<const uint4 *>(src);
        uint4 hi = make_uint4(0, 0, 0, 0);
        if (32 * w + 16 < K)
            hi = *reinterpret_cast<const uint4 *>(src + 16);
        const uint32_t by[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        // (16-column chunks: rank i of row n at ((i / 16) * N + n) * 16 + i % 16)
        int i = pre[w];
        while (b) {
            const int j = __ffs(b) - 1;
            WO[((int64_t)(i >> 4) * N + n) * 16 + (i & 15)] = (int8_t)((by[j >> 2] >> (8 * (j & 3))) & 0xffu);
            i++;
            b &= b - 1u;
        }
    }
    for (int p = tid; p < (n1 - n0) * 16; p += kThreads) {
        const int n = n0 + p / 16, e = p % 16;
        if (nO + e < nO16)
            WO[((int64_t)((nO + e) >> 4) * N + n) * 16 + ((nO + e) & 15)] = 0;
    }
}

// After k_prepare on a cache: the same comparison as its gather blocks
// (this call's bit set against the cached one), then the set is recorded
// on a miss and the hit or miss counted.  One workgroup.
__global__ __launch_bounds__(kThreads) void k_cache_commit(const uint32_t *__restrict__ bits,
                                                           const int32_t *__restrict__ meta,
                                                           int nw, int32_t *__restrict__ hdr,
                                                           uint32_t *__restrict__ cbits)
{
    __shared__ int miss_s;
    const int tid = threadIdx.x;
    if (tid == 0)
        miss_s = hdr[0] != 1;
    __syncthreads();
    bool diff = false;
    for (int w = tid; w < nw; w += kThreads)
        diff |= bits[w] != cbits[w];
    if (diff)
        atomicOr(&miss_s, 1);
    __syncthreads();
    const bool miss = miss_s != 0;
    if (miss)
        for (int w = tid; w < nw; w += kThreads)
            cbits[w] = bits[w];
    if (tid == 0) {
        if (miss) {
            hdr[1] = meta[0];
            hdr[3] += 1;
            hdr[0] = 1;
        } else {
            hdr[2] += 1;
        }
    }
}

// Marks an outlier-column cache empty (valid flag and counters zeroed).
__global__ void k_cache_reset(int32_t *__restrict__ hdr)
{
    if (threadIdx.x < 64)
        hdr[threadIdx.x] = 0;
}

} // namespace

hipError_t launch_quantize_weight(const uint16_t *W, int64_t N, int64_t K, int8_t *Wq,
                                  float *sW, hipStream_t s)
{
    hipLaunchKernelGGL(k_quantize_weight, dim3((unsigned)N), dim3(kThreads), 0, s, W,
                       (int)K, Wq, sW);
    return hipGetLastError();
}

hipError_t launch_cache_reset(char *cache, hipStream_t s)
{
    hipLaunchKernelGGL(k_cache_reset, dim3(1), dim3(64), 0, s,
                       reinterpret_cast<int32_t *>(cache + cache_layout(0, 0).hdr));
    return hipGetLastError();
}

hipError_t launch_prepare(const uint16_t *X, const int8_t *Wq, const uint16_t *W16,
                          uint16_t thr_mag, int64_t T, int64_t K, int64_t N, char *ws,
                          const WsLayout &L, hipStream_t s, char *cache)
{
    const CacheLayout C = cache_layout(K, N);
    uint32_t *bits = reinterpret_cast<uint32_t *>(ws + L.bits);
    int32_t *meta = reinterpret_cast<int32_t *>(ws + L.meta);
    const int nw = (int)((K + 31) / 32);
    hipLaunchKernelGGL(k_clear, dim3((unsigned)((max(nw, 64) + 255) / 256)), dim3(256), 0, s,
                       bits, nw, meta);
    const int nchunk = (int)(K / 8);
    if (nchunk > 0) {
        const int gx = (nchunk + kThreads - 1) / kThreads;
        // rows per block: a multiple of the load batch.  Two batches per
        // block when that still gives at least 256 workgroups (measured
        // fastest at 4096 x 4096 and 4096 x 8192), else about 256
        // workgroups of one batch; grid.y <= 65535
        const int64_t gy2 = (T + 2 * kDetectRows - 1) / (2 * kDetectRows);
        int gy = gx * gy2 >= 256
                     ? (int)std::min<int64_t>(gy2, 65535)
                     : (int)std::min<int64_t>((T + kDetectRows - 1) / kDetectRows, std::max(1, 256 / gx));
        int R = (int)((T + gy - 1) / gy);
        R = (R + kDetectRows - 1) / kDetectRows * kDetectRows;
        while ((T + R - 1) / R > 65535)
            R *= 2;
        gy = (int)((T + R - 1) / R);
        hipLaunchKernelGGL(k_detect, dim3(gx, gy), dim3(kThreads), 0, s, X, (int)T, (int)K,
                           R, (uint32_t)thr_mag, bits);
    }
    const int wrows = 32;
    const int64_t wblocks = (N + wrows - 1) / wrows;
    const size_t lds = 12 * (size_t)(nw > 0 ? nw : 1);   // bits, prefix, non-zero words
    const int64_t xblocks = (T + kPrepRows - 1) / kPrepRows;
    const bool reg = nw <= kBitsPerThread * kThreads, narrow = K / 8 <= 2 * kThreads;
    auto kp = reg ? (narrow ? k_prepare<kPrepRows, true, 2> : k_prepare<kPrepRows, true, 4>)
                  : (narrow ? k_prepare<kPrepRows, false, 2> : k_prepare<kPrepRows, false, 4>);
    auto launch = [&](auto KP) {
    hipLaunchKernelGGL(KP, dim3((unsigned)(xblocks + wblocks)), dim3(kThreads), lds, s, X, Wq,
                       W16, (int)T, (int)K, (int)N, wrows, bits, meta,
                       reinterpret_cast<int32_t *>(ws + L.idx),
                       reinterpret_cast<float *>(ws + L.sX),
                       reinterpret_cast<int8_t *>(ws + L.Xq),
                       reinterpret_cast<uint16_t *>(ws + L.XO),
                       reinterpret_cast<int8_t *>(cache ? cache + C.WO : ws + L.WO),
                       cache ? reinterpret_cast<int32_t *>(cache + C.hdr) : nullptr,
                       cache ? reinterpret_cast<uint32_t *>(cache + C.bits) : nullptr);
    };
    launch(kp);
    if (cache)
        hipLaunchKernelGGL(k_cache_commit, dim3(1), dim3(kThreads), 0, s, bits, meta, nw,
                           reinterpret_cast<int32_t *>(cache + C.hdr),
                           reinterpret_cast<uint32_t *>(cache + C.bits));
    return hipGetLastError();
}

} // namespace li8
