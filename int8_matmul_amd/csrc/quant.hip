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
// The weight quantization, the detection and the token quantization
// kernels are HBM-bound streaming passes: 16-byte coalesced loads, the row
// or column-strip reduction kept in registers, wave-level reductions, and
// the outlier bit set written as per-strip partial words with plain stores
// (no atomics on global memory).
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
// Token rows per quantization workgroup: 1 up to 1024 rows, else 2.  Every
// workgroup merges the detection strips' bit sets itself; fewer rows per
// workgroup mean more workgroups in flight.  Measured prepare stage: 13B
// (512 rows) 11.0 us with 2 rows, 9.05 with 1; at 2048 and 4096 rows 2 rows
// beat 1 (12.6 against 13.5 us, 21.0 against 22.0) and 4 (13.2, 22.2).
constexpr int kPrepRowsMax = 2;
inline int prep_rows(int64_t T) { return T <= 1024 ? 1 : kPrepRowsMax; }
// One wave per token row (k_prepare_rows) instead of k_prepare: from 2048
// rows (below that k_prepare's one row per workgroup keeps more of the chip
// busy), for K <= 4096 (8 chunks per lane) and X under 2 GiB (buffer
// offsets).
inline bool prep_wave_rows(int64_t T, int64_t K)
{
    return T >= 2048 && K >= 16 && K <= 4096 && 2 * T * K < ((int64_t)1 << 31);
}

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
// Outlier detection.  Block (x, y) covers CPB 8-column chunks (CPB/4
// bit-set words) of the row strip [y*R, y*R+R): thread (rl, cl) reads
// chunk x*CPB + cl of rows t0+rl, t0+rl+RL, ... (RL = 256/CPB row lanes),
// in batches of kDetectRows loads issued before any is used (these short
// streaming kernels are latency-bound otherwise); rows past the strip
// re-read its last row, which leaves the maximum unchanged.  The per-column
// magnitude max is kept packed in registers, one compare per column at the
// end, and the row lanes' flags are OR-ed through LDS.  Each block stores
// its words of strip y's partial bit set with plain stores: every word of
// every strip is written by exactly one block, so nothing is cleared
// first and no atomics are needed; k_prepare ORs the strips.
// ---------------------------------------------------------------------------
typedef li8_us2 us2;

constexpr int kDetectRows = 16;   // rows per load batch

template <int CPB>
__global__ __launch_bounds__(kThreads) void k_detect(
    const uint16_t *__restrict__ X, int T, int K, int R, uint32_t thr_mag,
    uint32_t *__restrict__ part)
{
    static_assert(CPB % 4 == 0 && CPB <= kThreads && kThreads % CPB == 0, "chunks per block");
    constexpr int RL = kThreads / CPB;
    __shared__ uint32_t fl[RL][CPB];
    const int nchunk = K / 8, nw = (K + 31) / 32;
    const int cl = threadIdx.x % CPB, rl = threadIdx.x / CPB;
    const int c = blockIdx.x * CPB + cl;
    const int t0 = blockIdx.y * R;
    const int t1 = min(T, t0 + R);
    us2 mx[4] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
    if (c < nchunk) {
        const uint4 *p = reinterpret_cast<const uint4 *>(X) + c;
        const int64_t stride = K / 8;
        for (int tb = t0 + rl; tb < t1; tb += RL * kDetectRows) {
            uint4 v[kDetectRows];
#pragma unroll
            for (int u = 0; u < kDetectRows; u++)
                v[u] = p[(int64_t)min(tb + u * RL, t1 - 1) * stride];
#pragma unroll
            for (int u = 0; u < kDetectRows; u++)
                column_max8(mx, v[u]);
        }
    }
    fl[rl][cl] = outlier_flags8(mx, thr_mag);
    __syncthreads();
    if ((int)threadIdx.x < CPB) {
        uint32_t f = 0;
#pragma unroll
        for (int r = 0; r < RL; r++)
            f |= fl[r][threadIdx.x];
        // chunk c holds columns 8c..8c+7 = bits 8*(c%4).. of word c/4; the
        // four chunks of a word sit in four consecutive lanes
        uint32_t word = f << (8 * (threadIdx.x & 3));
        word |= (uint32_t)__shfl_xor((int)word, 1, 64);
        word |= (uint32_t)__shfl_xor((int)word, 2, 64);
        const int w = (blockIdx.x * CPB + threadIdx.x) >> 2;
        if ((threadIdx.x & 3) == 0 && w < nw)
            part[(int64_t)blockIdx.y * nw + w] = word;
    }
}

// Bit-set words held in registers per thread by k_prepare (nw <= 256,
// i.e. K <= 8192); longer bit sets are read from global memory.
constexpr int kBitsPerThread = 1;

// Load the bit set into LDS (the OR of the nparts row strips' partial
// sets) and write the exclusive prefix of the popcounts per word; returns
// nO (the total) to every thread.  Thread tid owns words [tid*per,
// tid*per + per); with REG, bw already holds them (nw <= kBitsPerThread *
// kThreads).
template <bool REG>
__device__ int load_bits_and_scan(const uint32_t *__restrict__ parts, int nparts, int nw,
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
            uint32_t b = 0u;
            for (int y = 0; y < nparts; y++)
                b |= parts[(int64_t)y * nw + w];
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
// ROWS token rows; the remaining blocks gather the outlier columns of
// wrows rows of Wq (or of the fp16 weight W16, in the fp16-weight variant)
// each.  Every block rebuilds the prefix counts of the bit set in LDS, which
// gives each outlier column its compact index.
// ---------------------------------------------------------------------------

// The weight-gather part of the prepare kernels: block wb (of the blocks
// past the token blocks) copies the outlier columns of weight rows
// [wb*wrows, wb*wrows + wrows) into WO, and block 0 of them writes the
// outlier list, the count, the prefix counts per bit-set word and the
// merged bit set.  bits/pre: the merged bit set and its exclusive prefix
// counts in LDS (nw words each, followed by nw words of scratch).
template <int NT>
__device__ __forceinline__ void gather_block(
    int wb, const int8_t *__restrict__ Wq, const uint16_t *__restrict__ W16, int K, int N,
    int wrows, int fold_lo, int fold_hi, int nO, const uint32_t *bits, int32_t *pre,
    uint32_t *__restrict__ bits_g, int32_t *__restrict__ meta, int32_t *__restrict__ idx_g,
    int32_t *__restrict__ wpre, int8_t *__restrict__ WO, int32_t *__restrict__ cache_hdr,
    uint32_t *__restrict__ cache_bits, int *nnz_s_p, int *miss_s_p)
{
    const int tid = threadIdx.x;
    const int nw = (K + 31) / 32;
    const int nO16 = (nO + 15) & ~15;
    int &nnz_s = *nnz_s_p, &miss_s = *miss_s_p;
    const int n0 = wb * wrows;
    const int n1 = min(N, n0 + wrows);
    if (wb == 0) {
        for (int w = tid; w < nw; w += NT) {
            uint32_t b = bits[w];
            int p = pre[w];
            while (b) {
                idx_g[p++] = 32 * w + __ffs(b) - 1;
                b &= b - 1u;
            }
        }
        if (tid == 0)
            meta[0] = nO;
        // outlier columns before each bit-set word (the tiled GEMM's fold),
        // and the merged bit set (for the cache's record and the stage export)
        for (int w = tid; w <= nw; w += NT) {
            wpre[w] = w < nw ? pre[w] : nO;
            if (w < nw)
                bits_g[w] = bits[w];
        }
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
        for (int w = tid; w < nw; w += NT)
            diff |= bits[w] != cache_bits[w];
        if (diff)
            atomicOr(&miss_s, 1);
        __syncthreads();
        miss = miss_s != 0;
    }
    // (the tiled GEMM copies the weight's outlier columns itself when
    // fold_lo < nO <= fold_hi)
    if (!miss || nO == 0 || (nO > fold_lo && nO <= fold_hi))   // nothing to gather, or the GEMM takes them
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
        for (int p = tid; p < pairs; p += NT) {
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
        for (int p = tid; p < (n1 - n0) * 16; p += NT) {
            const int n = n0 + p / 16, e = p % 16;
            if (nO + e < nO16)
                WO16[((int64_t)((nO + e) >> 4) * N + n) * 16 + ((nO + e) & 15)] = 0;
        }
        return;
    }
    for (int p = tid; p < pairs; p += NT) {
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
    for (int p = tid; p < (n1 - n0) * 16; p += NT) {
        const int n = n0 + p / 16, e = p % 16;
        if (nO + e < nO16)
            WO[((int64_t)((nO + e) >> 4) * N + n) * 16 + ((nO + e) & 15)] = 0;
    }
}

// REG: the bit set fits in kBitsPerThread words per thread (K <= 8192).
// RREG: 16-byte chunks per thread and row kept in registers (2 when K <=
// 4096, else 4; columns past RREG * 8 * 256 are read again from memory).
template <int ROWS, bool REG, int RREG>
__global__ __launch_bounds__(kThreads) void k_prepare(
    const uint16_t *__restrict__ X, const int8_t *__restrict__ Wq,
    const uint16_t *__restrict__ W16, int T, int K, int N,
    int wrows, int fold_lo, int fold_hi, const uint32_t *__restrict__ parts, int nparts,
    uint32_t *__restrict__ bits_g, int32_t *__restrict__ meta, int32_t *__restrict__ idx_g, int32_t *__restrict__ wpre,
    float *__restrict__ sX,
    int8_t *__restrict__ Xq,
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

    // Loads first, all unconditional: this thread's bit-set words in every
    // row strip's partial set, then the token rows (buffer loads; chunks
    // past the row and the lanes of weight-gather blocks use offset 2^31,
    // past the buffer whenever X is under 2 GiB, else a valid address whose
    // value is not used).  Loads behind branches would make the compiler
    // wait for all of them at the first use; this way the bit-set scan
    // waits only for the bit-set words (loads complete in order) while the
    // rows arrive.  Strips past nparts re-read the last one (an OR of the
    // same word twice), so their count is no branch either.
    uint32_t bw[kBitsPerThread] = {};
    if constexpr (REG) {
        const int per = (nw + kThreads - 1) / kThreads;
        const int w0 = tid * per, wl = nw > 0 ? nw - 1 : 0;   // (the region has >= 1 word)
#pragma unroll
        for (int i = 0; i < kBitsPerThread; i++) {
            const int w = min(w0 + i, wl);
            uint32_t b = 0u;
#pragma unroll
            for (int y = 0; y < kDetectParts; y++)
                b |= parts[min(y, nparts - 1) * nw + w];
            bw[i] = b;
        }
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
    const int nO = load_bits_and_scan<REG>(parts, nparts, nw, bits, pre, scan, bw);
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
    gather_block<kThreads>(blockIdx.x - xblocks, Wq, W16, K, N, wrows, fold_lo, fold_hi, nO, bits, pre,
                           bits_g, meta, idx_g, wpre, WO, cache_hdr, cache_bits, &nnz_s, &miss_s);
}

// v with the binary16 values whose bit in skip is set replaced by +0.
__device__ __forceinline__ uint4 clear_halves8(uint4 v, uint32_t skip)
{
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t b = ((skip >> (2 * i)) & 1u) | (((skip >> (2 * i + 1)) & 1u) << 16);
        w[i] &= ~(b * 0xffffu);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// ---------------------------------------------------------------------------
// Token quantization with one wave per token row (long prompts, K <= 4096).
// Lane l holds the 16-byte chunks c = l + 64*s (s < CH) of the wave's row,
// so the masked row maximum is a wave reduction with no LDS round trip and
// no barrier, and the wave stores the row's codes, scale and outlier values
// itself.  A workgroup of 4 waves (4 rows) merges the detection strips' bit
// sets and builds their prefix counts once, with barriers that wait for LDS
// only, so the rows keep arriving meanwhile.  The blocks past the token
// blocks gather the weight's outlier columns as in k_prepare.
// (Measured against k_prepare's two rows per 256-thread workgroup: prepare
// stage 21.0 -> 19.3 us at 4096 x 4096, 12.3 -> 11.6 us at 2048 x 4096.
// Several rows per wave with their loads in flight together, 8 or 16 waves
// per workgroup, and two threads per bit-set word were all slower or the
// same; at K = 8192 this layout was slower, 35 -> 37 us.)
// ---------------------------------------------------------------------------
template <int CH>
__global__ __launch_bounds__(kThreads) void k_prepare_rows(
    const uint16_t *__restrict__ X, const int8_t *__restrict__ Wq,
    const uint16_t *__restrict__ W16, int T, int K, int N,
    int wrows, int fold_lo, int fold_hi, const uint32_t *__restrict__ parts, int nparts,
    uint32_t *__restrict__ bits_g, int32_t *__restrict__ meta, int32_t *__restrict__ idx_g, int32_t *__restrict__ wpre,
    float *__restrict__ sX,
    int8_t *__restrict__ Xq,
    uint16_t *__restrict__ XO, int8_t *__restrict__ WO, int32_t *__restrict__ cache_hdr,
    uint32_t *__restrict__ cache_bits, int xblocks)
{
    typedef unsigned int v2u_t __attribute__((ext_vector_type(2)));
    constexpr int NWV = kThreads / 64;
    static_assert(CH * 8 * 64 / 32 <= kThreads, "one bit-set word per thread");
    extern __shared__ uint32_t smem[];
    __shared__ int32_t scan[NWV];
    __shared__ int nnz_s, miss_s;
    const int nw = (K + 31) / 32;
    uint32_t *bits = smem;
    int32_t *pre = reinterpret_cast<int32_t *>(smem + nw);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nchunk = K / 8;
    const bool xblock = (int)blockIdx.x < xblocks;
    const int t = (int)blockIdx.x * NWV + wid;   // this wave's row (< T unless past the end)

    // Loads first, all unconditional: this thread's bit-set word in every
    // row strip's partial set (strips past nparts re-read the last one),
    // then the row (buffer loads, the row's offset in the scalar operand;
    // chunks past K, and every lane of a weight-gather block, use offset
    // 2^31, past X, which is under 2 GiB on this path).
    uint32_t bw = 0u;
    {
        // (the strip's offset in the scalar operand)
        const __amdgpu_buffer_rsrc_t rP = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint32_t *>(parts), (short)0, 4 * nparts * nw, 0x00020000);
        const int vo = 4 * min(tid, nw - 1);
#pragma unroll
        for (int y = 0; y < kDetectParts; y++)
            bw |= __builtin_amdgcn_raw_buffer_load_b32(rP, vo, 4 * min(y, nparts - 1) * nw, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    uint4 v[CH];
    {
        const __amdgpu_buffer_rsrc_t rX = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(X), (short)0, (int)(2u * (unsigned)T * (unsigned)K), 0x00020000);
        const int so = __builtin_amdgcn_readfirstlane((int)(2u * (unsigned)min(t, T - 1) * (unsigned)K));
#pragma unroll
        for (int s = 0; s < CH; s++) {
            const int c = lane + 64 * s;
            v[s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rX, (xblock & (c < nchunk)) ? 16 * c : (int)0x80000000, so, 0));
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // merged bit set and its exclusive prefix counts in LDS
    int nO;
    {
        const uint32_t b = tid < nw ? bw : 0u;
        if (tid < nw)
            bits[tid] = b;
        const int s = __popc(b);
        int x = s;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(x, o, 64);
            if (lane >= o)
                x += u;
        }
        if (lane == 63)
            scan[wid] = x;
        lds_barrier();
        int base = 0, total = 0;
#pragma unroll
        for (int i = 0; i < NWV; i++) {
            base += i < wid ? scan[i] : 0;
            total += scan[i];
        }
        if (tid < nw)
            pre[tid] = base + x - s;
        nO = total;
        lds_barrier();
    }

    if (xblock) {
        const int nO16 = (nO + 15) & ~15;
        const bool live = t < T;   // (uniform)
        // skip masks of this lane's chunks, and which chunk positions hold
        // an outlier column in any lane (a wave-uniform bit per position:
        // the masking is a uniform branch with no memory access)
        uint32_t skipm[CH];
        uint32_t anym = 0;
#pragma unroll
        for (int s = 0; s < CH; s++) {
            const int c = lane + 64 * s, cc = min(c, nchunk - 1);   // (a read inside the bit set either way)
            skipm[s] = c < nchunk ? (bits[cc >> 2] >> (8 * (c & 3))) & 0xffu : 0u;
            anym |= (__ballot(skipm[s] != 0u) != 0ull ? 1u : 0u) << s;
        }
        anym = __builtin_amdgcn_readfirstlane(anym);
        // outlier values (rank r of row t at ((r / 16) * T + t) * 16 + r % 16),
        // from the lanes that hold them, then the zero pad
        if (live) {
#pragma unroll
            for (int s = 0; s < CH; s++) {
                uint32_t sk = skipm[s];
                if (((anym >> s) & 1u) && sk) {
                    const int c = lane + 64 * s;
                    const uint4 x = v[s];
                    int r = pre[c >> 2] + __popc(bits[c >> 2] & ((1u << (8 * (c & 3))) - 1u));
#pragma unroll 1
                    while (sk) {
                        const int e = __builtin_ctz(sk);
                        sk &= sk - 1u;
                        const uint32_t w = e < 4 ? (e < 2 ? x.x : x.y) : (e < 6 ? x.z : x.w);
                        XO[((int64_t)(r >> 4) * T + t) * 16 + (r & 15)] = (uint16_t)((w >> (16 * (e & 1))) & 0xffffu);
                        r++;
                    }
                }
            }
            if (lane < nO16 - nO)
                XO[((int64_t)((nO + lane) >> 4) * T + t) * 16 + ((nO + lane) & 15)] = 0;
        }
        // then the outlier values are cleared in registers: the row maximum
        // over the rest is the plain maximum, and a cleared value gets code
        // 0, the code of an outlier column
#pragma unroll
        for (int s = 0; s < CH; s++)
            if ((anym >> s) & 1u)
                v[s] = clear_halves8(v[s], skipm[s]);
        uint32_t m = 0;
#pragma unroll
        for (int s = 0; s < CH; s++)
            m = max(m, chunk_max(v[s], 0u));
        m = wave_max(m);
        const float sc = h2f(m) / 127.0f;
        const float rc = 1.0f / sc;
        // a zero scale (every normal value of the row is 0) quantizes with
        // (1, 1), which gives those zeros their code 0
        const float su = sc == 0.0f ? 1.0f : sc, ru = sc == 0.0f ? 1.0f : rc;
        // stores: the row's offset in the scalar operand; a row past T puts
        // every lane out of range
        const __amdgpu_buffer_rsrc_t rQ = __builtin_amdgcn_make_buffer_rsrc(Xq, (short)0, T * K, 0x00020000);
        const __amdgpu_buffer_rsrc_t rS = __builtin_amdgcn_make_buffer_rsrc(sX, (short)0, 4 * T, 0x00020000);
        const int so = __builtin_amdgcn_readfirstlane(live ? t * K : 0);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sc), rS,
                                              (live & (lane == 0)) ? 4 * t : (int)0x80000000, 0, 0);
#pragma unroll
        for (int s = 0; s < CH; s++) {
            const uint2 q = token_codes8(v[s], 0u, su, ru);
            const int c = lane + 64 * s;
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u_t, q), rQ,
                                                  (live & (c < nchunk)) ? 8 * c : (int)0x80000000, so, 0);
        }
        return;
    }

    // ---- outlier columns of wrows weight rows ----
    gather_block<kThreads>(blockIdx.x - xblocks, Wq, W16, K, N, wrows, fold_lo, fold_hi, nO, bits, pre,
                           bits_g, meta, idx_g, wpre, WO, cache_hdr, cache_bits, &nnz_s, &miss_s);
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

// The detection grid: CPB chunks per block (of 16..256) and gy <= 16 row
// strips.  The first (rows per thread, CPB) pair, in that order of
// preference, that gives at least 256 workgroups with at most that many
// rows per thread (two load batches, then one, then half of one); else the
// most workgroups the shape allows.  (Two batches per workgroup measured
// fastest at 4096 x 4096 and 4096 x 8192.)
struct DetectGrid {
    int cpb, gx, gy, R;
};

DetectGrid detect_grid(int64_t T, int64_t K)
{
    const int64_t nchunk = K / 8;
    if (nchunk == 0 || T == 0)
        return {16, 0, 0, 0};
    auto make = [&](int cpb, int64_t rpt) {
        const int64_t rl = kThreads / cpb;
        const int64_t gy = std::min<int64_t>(kDetectParts, (T + rl * rpt - 1) / (rl * rpt));
        const int64_t R = (T + gy - 1) / gy;
        return DetectGrid{cpb, (int)((nchunk + cpb - 1) / cpb), (int)gy, (int)R};
    };
    for (int64_t rpt : {2 * kDetectRows, kDetectRows, kDetectRows / 2}) {
        for (int cpb : {256, 128, 64, 32, 16}) {
            const DetectGrid g = make(cpb, rpt);
            const int64_t rows = ((int64_t)g.R + kThreads / cpb - 1) / (kThreads / cpb);
            if ((int64_t)g.gx * g.gy >= 256 && rows <= rpt)
                return g;
        }
    }
    return make(16, kDetectRows / 2);
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
                          const WsLayout &L, hipStream_t s, char *cache, GatherSkip skip)
{
    const CacheLayout C = cache_layout(K, N);
    uint32_t *bits = reinterpret_cast<uint32_t *>(ws + L.bits);
    uint32_t *part = reinterpret_cast<uint32_t *>(ws + L.part);
    int32_t *meta = reinterpret_cast<int32_t *>(ws + L.meta);
    const int nw = (int)((K + 31) / 32);
    const DetectGrid dg = detect_grid(T, K);
    if (dg.gy > 0) {
        auto launch_detect = [&](auto KD) {
            hipLaunchKernelGGL(KD, dim3((unsigned)dg.gx, (unsigned)dg.gy), dim3(kThreads), 0, s, X,
                               (int)T, (int)K, dg.R, (uint32_t)thr_mag, part);
        };
        switch (dg.cpb) {
        case 256: launch_detect(k_detect<256>); break;
        case 128: launch_detect(k_detect<128>); break;
        case 64: launch_detect(k_detect<64>); break;
        case 32: launch_detect(k_detect<32>); break;
        default: launch_detect(k_detect<16>); break;
        }
    }
    // weight rows per gather block: 16 (8 for the fp16 weight, twice the
    // bytes per column).  Measured against 32: 13B fp16-weight call 80.5 ->
    // 77.1 us (16) and 76.0 us (8); 8 costs 0.5 us elsewhere, 64 and 128
    // were slower everywhere.
    const int wrows = W16 ? 8 : 16;
    const int64_t wblocks = (N + wrows - 1) / wrows;
    const size_t lds = 12 * (size_t)(nw > 0 ? nw : 1);   // bits, prefix, non-zero words
    const int rows = prep_rows(T);
    const int64_t xblocks = (T + rows - 1) / rows;
    const bool reg = nw <= kBitsPerThread * kThreads, narrow = K / 8 <= 2 * kThreads;
    if (prep_wave_rows(T, K)) {   // one wave per token row
        const int64_t xb = (T + 3) / 4;
        hipLaunchKernelGGL(k_prepare_rows<8>, dim3((unsigned)(xb + wblocks)), dim3(kThreads), lds, s, X,
                           Wq, W16, (int)T, (int)K, (int)N, wrows, skip.lo, skip.hi, part,
                           std::max(dg.gy, 1), bits, meta, reinterpret_cast<int32_t *>(ws + L.idx),
                           reinterpret_cast<int32_t *>(ws + L.wpre),
                           reinterpret_cast<float *>(ws + L.sX),
                           reinterpret_cast<int8_t *>(ws + L.Xq),
                           reinterpret_cast<uint16_t *>(ws + L.XO),
                           reinterpret_cast<int8_t *>(cache ? cache + C.WO : ws + L.WO),
                           cache ? reinterpret_cast<int32_t *>(cache + C.hdr) : nullptr,
                           cache ? reinterpret_cast<uint32_t *>(cache + C.bits) : nullptr, (int)xb);
        if (cache)
            hipLaunchKernelGGL(k_cache_commit, dim3(1), dim3(kThreads), 0, s, bits, meta, nw,
                               reinterpret_cast<int32_t *>(cache + C.hdr),
                               reinterpret_cast<uint32_t *>(cache + C.bits));
        return hipGetLastError();
    }
    auto kp = rows == 1
                  ? (reg ? (narrow ? k_prepare<1, true, 2> : k_prepare<1, true, 4>)
                         : (narrow ? k_prepare<1, false, 2> : k_prepare<1, false, 4>))
                  : (reg ? (narrow ? k_prepare<kPrepRowsMax, true, 2> : k_prepare<kPrepRowsMax, true, 4>)
                         : (narrow ? k_prepare<kPrepRowsMax, false, 2> : k_prepare<kPrepRowsMax, false, 4>));
    auto launch = [&](auto KP) {
    hipLaunchKernelGGL(KP, dim3((unsigned)(xblocks + wblocks)), dim3(kThreads), lds, s, X, Wq,
                       W16, (int)T, (int)K, (int)N, wrows, skip.lo, skip.hi, part,
                       std::max(dg.gy, 1), bits, meta, reinterpret_cast<int32_t *>(ws + L.idx),
                       reinterpret_cast<int32_t *>(ws + L.wpre),
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
