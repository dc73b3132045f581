// The LLM.int8() layer for few tokens and a long K (decode-time FFN
// down-projections: T <= 16, K past what one workgroup's LDS holds codes
// for), for gfx950.  Same arithmetic as the prepare kernels and the tiled
// GEMM:
//   O      = { j : some |X[t,j]| > threshold }                  (union over t)
//   sX[t]  = fl32(max_{j not in O} |X[t,j]| / 127), Xq codes rne, 0 on O
//   acc    = sum_j Xq[t,j] Wq[n,j]                              (exact int32)
//   D      = fl32(acc * sX[t]) + sum_{j in O} X[t,j] Wq[n,j]    (fp16 MFMA, fp32)
//   Y[t,n] = fp16(fl32(D * sW[n]))
// (hncyxsy.com/news/230290, section 2.1; tqpw.cn/news/5683, section 2.1.)
//
// The layer is bound by one read of Wq (N*K bytes).  K is split into KS
// slices across workgroups, so that each workgroup quantizes only its
// slice of X (the codes of a slice live in LDS) and a grid of 256
// workgroups streams Wq however few output features there are:
//  1. k_dscan: one wave per 512 columns over all T <= 16 rows finds the
//     outlier columns of its strip exactly (every row is in the strip),
//     counts them, and takes the per-token maxima over its normal columns.
//     No cross-workgroup reduction, so nothing has to be cleared first.
//  2. k_dsplit: workgroup (slice ks, row-group class rgc) derives the token
//     scales from the strips' maxima, quantizes its slice of X into LDS,
//     and for row groups rg = rgc, rgc + NRGC, ... multiplies 16 weight rows
//     of its slice by the codes (v_mfma_i32_16x16x64_i8, the 8 waves
//     splitting the slice), adding the waves' int32 sums in LDS and storing
//     one partial sum per (slice, row group).  The workgroups of class 0
//     also write the outlier list, the gathered outlier values of X, the
//     token scales and nO in the prepared-workspace layout.  Variant
//     FUSED = false reads codes from a workspace that the prepare kernels
//     filled instead.
//  3. k_dfinish: one wave per row group adds the KS partial sums (exact),
//     dequantizes, adds the outlier product over chunks of 32 outlier
//     columns (v_mfma_f32_16x16x32_f16), scales by sW and stores fp16.
//     Both routes end in this kernel on the same inputs, so they give
//     bit-identical outputs.
// F16W: the outlier columns multiply the fp16 weight W16, and
// D = fl32(fl32(acc * sX) * sW) + sum_O X * W16.
#include <algorithm>

#include "li8_internal.h"
#include "quant_math.h"

namespace li8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kScanCols = 512;          // columns per k_dscan wave
constexpr int kSThreads = 512;          // k_dsplit: 8 waves
constexpr int kSWaves = kSThreads / 64;
constexpr int kFThreads = 256;          // k_dfinish: 4 waves, one row group each
constexpr int kOutOfRange = (int)0x80000000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ v4i load16(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Exclusive prefix over the wave's lanes of a count 0..8, and the total.
__device__ __forceinline__ int wave_prefix8(int cnt, int lane, int &total)
{
    const uint64_t below = (1ull << lane) - 1ull;
    int p = 0, tot = 0;
#pragma unroll
    for (int bit = 0; bit < 4; bit++) {
        const uint64_t m = __ballot((cnt >> bit) & 1);
        p += __popcll(m & below) << bit;
        tot += __popcll(m) << bit;
    }
    total = tot;
    return p;
}

// ---------------------------------------------------------------------------
// 1. Scan: wave b covers columns [512 b, 512 b + 512), 8 per lane, all rows.
//   bits   : the outlier bit set (this strip's 16 words)
//   ocnt[b]: outlier columns in the strip
//   pmax[b][16]: per-token max magnitude pattern over the strip's normal
//                columns (0 for token slots past T)
// ---------------------------------------------------------------------------
template <int TB>
__global__ __launch_bounds__(64) void k_dscan(const uint16_t *__restrict__ X, int T, int K,
                                              uint32_t thr_mag, uint32_t *__restrict__ bits,
                                              int32_t *__restrict__ ocnt, uint32_t *__restrict__ pmax)
{
    const int lane = threadIdx.x, b = blockIdx.x;
    const int nchunk = K / 8;
    const int c = b * 64 + lane;
    const __amdgpu_buffer_rsrc_t rX = make_rsrc(X, 2 * T * K);
    uint4 xv[TB];
#pragma unroll
    for (int t = 0; t < TB; t++) {   // rows past T and chunks past K read zeros
        const bool ok = (t < T) & (c < nchunk);
        xv[t] = __builtin_bit_cast(uint4, load16(rX, ok ? 16 * (t * nchunk + c) : kOutOfRange));
    }
    li8_us2 mx[4] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
#pragma unroll
    for (int t = 0; t < TB; t++)
        column_max8(mx, xv[t]);
    const uint32_t fl = outlier_flags8(mx, thr_mag);
    uint32_t word = fl << (8 * (c & 3));
    word |= (uint32_t)__shfl_xor((int)word, 1, 64);
    word |= (uint32_t)__shfl_xor((int)word, 2, 64);
    if ((c & 3) == 0 && c < nchunk)
        bits[c >> 2] = word;
    int total;
    (void)wave_prefix8(__popc(fl), lane, total);
    if (lane == 0)
        ocnt[b] = total;
    uint32_t wm[TB];
#pragma unroll
    for (int t = 0; t < TB; t++)
        wm[t] = wave_max(chunk_max(xv[t], fl));
    if (lane < 16) {
        uint32_t m = 0;
#pragma unroll
        for (int t = 0; t < TB; t++)
            m = (lane == t) ? wm[t] : m;
        pmax[b * 16 + lane] = m;
    }
}

// ---------------------------------------------------------------------------
// 2. Split GEMV.  Workgroup blockIdx.x = ks * NRGC + rgc: slice ks covers
// columns [ks * KSL, min(K, ks * KSL + KSL)), KSL a multiple of 512 and at
// most 512 * KB; the 8 waves split its 64-column k-steps.  Partial sums go
// to part[((ks * NRG + rg) * 64 + lane)] as 4 int32 per lane, lane holding
// token (lane & 15) and features rg * 16 + 4 * (lane >> 4) + 0..3.
// ---------------------------------------------------------------------------
struct SplitOut {   // FUSED: where class-0 workgroups write the prepared stages
    int32_t *meta, *idx;
    float *sX;
    uint16_t *XO;
};

template <bool FUSED, int KB, int TB>
__global__ __launch_bounds__(kSThreads) void k_dsplit(
    const uint16_t *__restrict__ X, const int8_t *__restrict__ Wq, int T, int K, int N, int KSL,
    int NRGC, const uint32_t *__restrict__ bits, const int32_t *__restrict__ ocnt,
    const uint32_t *__restrict__ pmax, SplitOut out, const int8_t *__restrict__ Xq_g,
    int32_t *__restrict__ part)
{
    static_assert(KB % 8 == 0, "weight loads per lane come in groups of 8");
    constexpr int CPT = KB / 8;                       // 8-column chunks per thread: KSL <= 512 * KB
    constexpr int kXq = KB * 32 * (16 * TB + 16);     // codes: KSL/16 blocks of 16T + 16 bytes
    __shared__ __attribute__((aligned(16))) int8_t xq[kXq];
    __shared__ __attribute__((aligned(16))) v4i red[2][kSWaves][64];
    __shared__ float sxl[16], rxl[16];
    __shared__ __attribute__((aligned(16))) uint32_t zero16[4];
    __shared__ int wtot[kSWaves];
    static_assert(sizeof(xq) + sizeof(red) + 160 <= 160 * 1024, "LDS of one workgroup");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int NRG = (N + 15) / 16;
    const int ks = blockIdx.x / NRGC, rgc = blockIdx.x - ks * NRGC;
    const int k0 = ks * KSL, kw = min(K - k0, KSL);   // the slice; kw % 16 == 0
    const int QS = 16 * T + 16;
    const int S = (kw + 63) / 64;                     // k-steps of the slice
    const int s0 = wid * S / kSWaves, s1 = (wid + 1) * S / kSWaves;
    const int kg = lane >> 4, tok = lane & 15;
    const int kend = k0 + min(s1 * 64, kw);           // end of this wave's share
    const __amdgpu_buffer_rsrc_t rW = make_rsrc(Wq, N * K);
    if (tid < 4)
        zero16[tid] = 0u;

    v4i wbuf[2][KB];
    auto wload = [&](int set, int rg) {   // (rg >= NRG reads zeros)
        const int n = min(rg * 16 + (lane & 15), N - 1);
        const int kl = rg < NRG ? kend : 0;
#pragma unroll
        for (int j = 0; j < KB; j++) {
            const int k = k0 + (s0 + j) * 64 + 16 * kg;
            wbuf[set][j] = load16(rW, k < kl ? n * K + k : kOutOfRange);
        }
    };
    const int rg0 = rgc;
    // The fused variant with two chunks of X per thread for 16 token slots
    // has no registers to spare for a weight batch during the activation
    // work: it requests the first batch after it.
    constexpr bool kEarly = !(FUSED && KB > 8 && TB > 8);

    if constexpr (FUSED) {
        // this thread's chunks of the slice (all token rows), the flags of
        // their columns, the strips' maxima and outlier counts: every load
        // issued first and unconditionally (out-of-range offsets read zeros)
        const int nchunk = K / 8, c0 = k0 / 8;
        const int nb1 = (K + kScanCols - 1) / kScanCols;
        const int sbeg = k0 / kScanCols, nsb = (kw + kScanCols - 1) / kScanCols;   // the slice's strips
        const __amdgpu_buffer_rsrc_t rX = make_rsrc(X, 2 * T * K);
        const __amdgpu_buffer_rsrc_t rC = make_rsrc(ocnt, 4 * nb1);
        const __amdgpu_buffer_rsrc_t rP = make_rsrc(pmax, 64 * nb1);
        uint4 xv[CPT][TB];
        uint32_t bw[CPT];
#pragma unroll
        for (int u = 0; u < CPT; u++) {
            const int cl = tid + u * kSThreads;
            const bool in = 8 * cl < kw;
#pragma unroll
            for (int t = 0; t < TB; t++)
                xv[u][t] = __builtin_bit_cast(
                    uint4, load16(rX, (in & (t < T)) ? 16 * (t * nchunk + c0 + cl) : kOutOfRange));
            bw[u] = bits[min(c0 + cl, nchunk - 1) >> 2];
        }
        // strip maxima: thread (t = tid & 15, p = tid >> 4) takes strips p, p + 32, ...
        constexpr int kMaxStrips = (int)((kMaxK + kScanCols - 1) / kScanCols);
        uint32_t pmv[(kMaxStrips + 31) / 32];
#pragma unroll
        for (int i = 0; i < (kMaxStrips + 31) / 32; i++) {
            const int sb = (tid >> 4) + 32 * i;
            pmv[i] = __builtin_amdgcn_raw_buffer_load_b32(rP, sb < nb1 ? 4 * (sb * 16 + (tid & 15)) : kOutOfRange,
                                                          0, 0);
        }
        // outlier counts: the strips before the slice (thread sb), and the
        // slice's own strips (lane i of every wave holds strip sbeg + i)
        const int cbefore = (int)__builtin_amdgcn_raw_buffer_load_b32(rC, tid < sbeg ? 4 * tid : kOutOfRange, 0, 0);
        const int ocs = (int)__builtin_amdgcn_raw_buffer_load_b32(rC, lane < nsb ? 4 * (sbeg + lane) : kOutOfRange,
                                                                  0, 0);
        if constexpr (kEarly)
            wload(0, rg0);
        // token scales: max over the strips, then fl32(max / 127) and its
        // reciprocal (IEEE divisions), through LDS
        uint32_t pm = 0;
#pragma unroll
        for (int i = 0; i < (kMaxStrips + 31) / 32; i++)
            pm = max(pm, pmv[i]);
        uint32_t *pml = reinterpret_cast<uint32_t *>(&red[0][0][0]);   // [32][16], free until the MFMAs
        pml[tid] = pm;
        {   // block sum of the counts before the slice
            int v = cbefore;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1)
                v += __shfl_xor(v, o, 64);
            if (lane == 0)
                wtot[wid] = v;
        }
        lds_barrier();
        if (tid < 16) {
            uint32_t m = 0;
#pragma unroll 8
            for (int p = 0; p < 32; p++)
                m = max(m, pml[p * 16 + tid]);
            m = tid < T ? m : 0u;
            const float sc = h2f(m) / 127.0f;
            sxl[tid] = sc;
            rxl[tid] = 1.0f / sc;
        }
        int base = 0;   // rank of the slice's first outlier column
#pragma unroll
        for (int w = 0; w < kSWaves; w++)
            base += wtot[w];
        lds_barrier();
        float sx[TB], rx[TB];
#pragma unroll
        for (int t = 0; t < TB; t++) {
            sx[t] = sxl[t];
            rx[t] = rxl[t];
        }
        // codes of the slice into LDS (block q of 16 columns, token t at q*QS + 16t)
        uint32_t fl[CPT];
#pragma unroll
        for (int u = 0; u < CPT; u++) {
            const int cl = tid + u * kSThreads;
            fl[u] = (8 * cl < kw) ? (bw[u] >> (8 * (cl & 3))) & 0xffu : 0u;   // (c0 % 64 == 0)
            const uint2 keep = keep_bytes8(fl[u]);
            if (8 * cl < kw) {
#pragma unroll
                for (int t = 0; t < TB; t++)
                    if (t < T) {
                        const uint2 q = (sx[t] == 0.0f) ? make_uint2(0u, 0u)
                                                        : token_codes8_keep(xv[u][t], keep, sx[t], rx[t]);
                        *reinterpret_cast<uint2 *>(xq + (cl >> 1) * QS + 16 * t + 8 * (cl & 1)) = q;
                    }
            }
        }
        if (rgc == 0) {
            // Class 0 writes the prepared stages for its slice: the ascending
            // outlier list, the outlier values of X in 16-column chunks (rank
            // i of token t at ((i/16)*T + t)*16 + i%16) and, for the last
            // slice, the zero pad and nO; slice 0 writes the token scales.
            // Chunk cl of wave w in pass u lies in strip sbeg + 8u + w, in
            // lane order, so a ballot prefix within the wave ranks it there.
#pragma unroll
            for (int u = 0; u < CPT; u++) {
                int wsum;
                const int p = wave_prefix8(__popc(fl[u]), lane, wsum);
                int before = 0, pass = 0;   // this pass: strips of waves before this one, all
#pragma unroll
                for (int w = 0; w < kSWaves; w++) {
                    const int v = __shfl(ocs, u * kSWaves + w, 64);   // (0 past the slice)
                    before += (w < wid) ? v : 0;
                    pass += v;
                }
                int i = base + before + p;
                const int cl = tid + u * kSThreads;
                for (uint32_t f = fl[u]; f; f &= f - 1u, i++) {
                    const int e = __ffs(f) - 1;
                    out.idx[i] = k0 + 8 * cl + e;
#pragma unroll
                    for (int t = 0; t < TB; t++)
                        if (t < T) {
                            const uint32_t wd[4] = {xv[u][t].x, xv[u][t].y, xv[u][t].z, xv[u][t].w};
                            out.XO[((int64_t)(i >> 4) * T + t) * 16 + (i & 15)] =
                                (uint16_t)(wd[e >> 1] >> (16 * (e & 1)));
                        }
                }
                base += pass;
            }
            if (k0 + kw == K) {   // last slice: nO is known; pad to a multiple of 16
                const int nO = base;
                const int pad = ((nO + 15) & ~15) - nO;
                for (int j = tid; j < pad * T; j += kSThreads) {
                    const int i = nO + j / T, t = j % T;
                    out.XO[((int64_t)(i >> 4) * T + t) * 16 + (i & 15)] = 0;
                }
                if (tid == 0)
                    out.meta[0] = nO;
            }
            if (ks == 0 && tid < T)
                out.sX[tid] = sxl[tid];
        }
        if constexpr (!kEarly)
            wload(0, rg0);
        lds_barrier();
    } else {
        // codes of the slice from the prepared workspace (row-major [T,K])
        constexpr int CPTW = TB * KB / 16;   // 16-byte chunks per thread: T * KSL/16 <= 512 * CPTW
        const int nq = kw / 16, tot = T * nq;
        const __amdgpu_buffer_rsrc_t rQ = make_rsrc(Xq_g, T * K);
        uint4 st[CPTW];
#pragma unroll
        for (int j = 0; j < CPTW; j++) {
            const int i = tid + j * kSThreads;
            const int t = i / max(nq, 1), q = i - t * nq;
            st[j] = __builtin_bit_cast(uint4, load16(rQ, i < tot ? t * K + k0 + 16 * q : kOutOfRange));
        }
        wload(0, rg0);
#pragma unroll
        for (int j = 0; j < CPTW; j++) {
            const int i = tid + j * kSThreads;
            if (i < tot) {
                const int t = i / nq, q = i - t * nq;
                *reinterpret_cast<uint4 *>(xq + q * QS + 16 * t) = st[j];
            }
        }
        lds_barrier();
    }

    // ---- row groups: int8 MFMAs over this wave's share of the slice ----
    auto process = [&](int set, int rg, int par) {
        v4i acc = {0, 0, 0, 0}, acc2 = {0, 0, 0, 0};
#pragma unroll
        for (int h = 0; h < KB; h += 8) {
            v4i xf[8];
#pragma unroll
            for (int j = 0; j < 8; j++) {   // (no token or no column: the zero bytes)
                const int q = (s0 + h + j) * 4 + kg;
                const bool ok = tok < T && s0 + h + j < s1 && 16 * q < kw;
                xf[j] = *reinterpret_cast<const v4i *>(ok ? xq + q * QS + 16 * tok
                                                          : reinterpret_cast<const int8_t *>(zero16));
            }
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wbuf[set][h + j], xf[j], acc, 0, 0, 0);
                acc2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(wbuf[set][h + j + 1], xf[j + 1], acc2, 0, 0, 0);
            }
        }
        acc += acc2;
        red[par][wid][lane] = acc;
        lds_barrier();
        if (wid == 0) {
            v4i tot = red[par][0][lane];
#pragma unroll
            for (int w = 1; w < kSWaves; w++)
                tot += red[par][w][lane];
            *reinterpret_cast<v4i *>(part + ((int64_t)(ks * NRG + rg) * 64 + lane) * 4) = tot;
        }
    };

    int rg = rg0;
    if (NRG <= NRGC) {   // one row group per workgroup
        process(0, rg, 0);
        return;
    }
    while (rg < NRG) {   // two per iteration: the next group's loads ahead of this one's MFMAs
        const int rg1 = rg + NRGC;
        wload(1, rg1);
        process(0, rg, 0);
        if (rg1 >= NRG)
            break;
        const int rg2 = rg1 + NRGC;
        wload(0, rg2);
        process(1, rg1, 1);
        rg = rg2;
    }
}

// ---------------------------------------------------------------------------
// 3. Finish: wave w of workgroup g handles row group rg = 4 g + w.
// ---------------------------------------------------------------------------
template <bool F16W, bool STORE_ACC>
__global__ __launch_bounds__(kFThreads) void k_dfinish(
    const int8_t *__restrict__ Wq, const float *__restrict__ sW, const uint16_t *__restrict__ W16,
    int T, int K, int N, int KS, const int32_t *__restrict__ part, const int32_t *__restrict__ meta,
    const int32_t *__restrict__ idx_g, const float *__restrict__ sX_g,
    const uint16_t *__restrict__ XO_g, uint16_t *__restrict__ Y, int32_t *__restrict__ acc_out)
{
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int NRG = (N + 15) / 16;
    const int rg = blockIdx.x * (kFThreads / 64) + wid;
    if (rg >= NRG)
        return;
    const int kg = lane >> 4, tok = lane & 15;
    const int ttok = min(tok, T - 1);
    const int nO = min(max(meta[0], 0), K);   // (a bad workspace cannot lengthen the loop)
    const int nb = rg * 16 + 4 * kg;          // this lane's first feature
    // every independent load first: the partial sums, the token scale, the
    // column scales, the first chunk's indices and outlier values
    v4i tot = {0, 0, 0, 0};
    for (int s = 0; s < KS; s++)
        tot += *reinterpret_cast<const v4i *>(part + ((int64_t)(s * NRG + rg) * 64 + lane) * 4);
    const float sx = tok < T ? sX_g[ttok] : 0.0f;
    float swv[4];
#pragma unroll
    for (int r = 0; r < 4; r++)
        swv[r] = sW[min(nb + r, N - 1)];
    if constexpr (STORE_ACC) {
        if (tok < T)
#pragma unroll
            for (int r = 0; r < 4; r++)
                if (nb + r < N)
                    acc_out[(int64_t)tok * N + nb + r] = tot[r];
    }
    v4f d;
#pragma unroll
    for (int r = 0; r < 4; r++)
        d[r] = (float)tot[r] * sx;
    if constexpr (F16W)   // the fp16 outlier product is then in output units
#pragma unroll
        for (int r = 0; r < 4; r++)
            d[r] *= swv[r];
    // D += X[:, O] . W[:, O]^T, 32 outlier columns per MFMA: lane supplies
    // weight row (lane & 15) and token tok at ranks 32c + 8 kg .. +7
    const int rows = min(16, N - rg * 16);
    const int wl = min(lane & 15, rows - 1);   // local weight row
    const __amdgpu_buffer_rsrc_t rWg = F16W ? make_rsrc(W16 + (int64_t)rg * 16 * K, 2 * rows * K)
                                            : make_rsrc(Wq + (int64_t)rg * 16 * K, rows * K);
    const __amdgpu_buffer_rsrc_t rI = make_rsrc(idx_g, 4 * K);
    const __amdgpu_buffer_rsrc_t rXO = make_rsrc(XO_g, 2 * T * K);
    for (int c = 0; c < (nO + 31) / 32; c++) {
        const int i0 = 32 * c + 8 * kg;
        int col[8];
        uint32_t xr[8];
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const int i = i0 + e;
            const bool ok = i < nO;
            col[e] = (int)__builtin_amdgcn_raw_buffer_load_b32(rI, ok ? 4 * i : kOutOfRange, 0, 0);
            xr[e] = __builtin_amdgcn_raw_buffer_load_b16(
                rXO, ok ? 2 * (((i >> 4) * T + ttok) * 16 + (i & 15)) : kOutOfRange, 0, 0);
        }
        int wr[8];
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const bool ok = i0 + e < nO;
            const int wo = wl * K + min(max(col[e], 0), K - 1);
            if constexpr (F16W)
                wr[e] = __builtin_amdgcn_raw_buffer_load_b16(rWg, ok ? 2 * wo : kOutOfRange, 0, 0);
            else
                wr[e] = (int8_t)__builtin_amdgcn_raw_buffer_load_b8(rWg, ok ? wo : kOutOfRange, 0, 0);
        }
        v8h a, b;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const bool ok = i0 + e < nO;
            if constexpr (F16W)
                a[e] = ok ? __builtin_bit_cast(_Float16, (uint16_t)wr[e]) : (_Float16)0.0f;
            else
                a[e] = ok ? (_Float16)(float)wr[e] : (_Float16)0.0f;
            b[e] = (ok && tok < T) ? __builtin_bit_cast(_Float16, (uint16_t)xr[e]) : (_Float16)0.0f;
        }
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, d, 0, 0, 0);
    }
    if (tok >= T)
        return;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
        // fl32(D * sW) first, then one rounding to fp16 (the empty asm
        // keeps the product and the conversion from being fused)
        p[r] = d[r];
        if constexpr (!F16W)
            p[r] *= swv[r];
        asm("" : "+v"(p[r]));
    }
    const uint32_t h01 = pack_f16x2(p[0], p[1]), h23 = pack_f16x2(p[2], p[3]);
    uint16_t *y = Y + (int64_t)tok * N + nb;
    if ((N & 3) == 0 && nb + 3 < N) {
        *reinterpret_cast<uint2 *>(y) = make_uint2(h01, h23);
    } else {
        const uint32_t hw[2] = {h01, h23};
#pragma unroll
        for (int r = 0; r < 4; r++)
            if (nb + r < N)
                y[r] = (uint16_t)(hw[r >> 1] >> (16 * (r & 1)));
    }
}

template <bool FUSED, int KB, int TB>
void launch_split_kb(const uint16_t *X, const int8_t *Wq, int64_t T, int64_t K, int64_t N,
                     const SplitPlan &p, const uint32_t *bits, const int32_t *ocnt,
                     const uint32_t *pmax, SplitOut out, const int8_t *Xq, int32_t *part,
                     hipStream_t s)
{
    hipLaunchKernelGGL((k_dsplit<FUSED, KB, TB>), dim3((unsigned)(p.KS * p.NRGC)), dim3(kSThreads), 0,
                       s, X, Wq, (int)T, (int)K, (int)N, p.KSL, p.NRGC, bits, ocnt, pmax, out, Xq,
                       part);
}

template <bool FUSED>
void launch_split(const uint16_t *X, const int8_t *Wq, int64_t T, int64_t K, int64_t N,
                  const SplitPlan &p, const uint32_t *bits, const int32_t *ocnt, const uint32_t *pmax,
                  SplitOut out, const int8_t *Xq, int32_t *part, hipStream_t s)
{
    if (p.KSL <= 8 * 512)
        return T <= 8 ? launch_split_kb<FUSED, 8, 8>(X, Wq, T, K, N, p, bits, ocnt, pmax, out, Xq, part, s)
                      : launch_split_kb<FUSED, 8, 16>(X, Wq, T, K, N, p, bits, ocnt, pmax, out, Xq, part, s);
    return T <= 8 ? launch_split_kb<FUSED, 16, 8>(X, Wq, T, K, N, p, bits, ocnt, pmax, out, Xq, part, s)
                  : launch_split_kb<FUSED, 16, 16>(X, Wq, T, K, N, p, bits, ocnt, pmax, out, Xq, part, s);
}

void launch_finish(const int8_t *Wq, const float *sW, const uint16_t *W16, int64_t T, int64_t K,
                   int64_t N, int KS, const int32_t *part, const int32_t *meta, const int32_t *idx,
                   const float *sX, const uint16_t *XO, uint16_t *Y, int32_t *acc, hipStream_t s)
{
    const int NRG = (int)((N + 15) / 16);
    const dim3 grid((unsigned)((NRG + 3) / 4)), block(kFThreads);
    if (W16) {
        if (acc)
            hipLaunchKernelGGL((k_dfinish<true, true>), grid, block, 0, s, Wq, sW, W16, (int)T, (int)K,
                               (int)N, KS, part, meta, idx, sX, XO, Y, acc);
        else
            hipLaunchKernelGGL((k_dfinish<true, false>), grid, block, 0, s, Wq, sW, W16, (int)T, (int)K,
                               (int)N, KS, part, meta, idx, sX, XO, Y, acc);
    } else {
        if (acc)
            hipLaunchKernelGGL((k_dfinish<false, true>), grid, block, 0, s, Wq, sW, W16, (int)T, (int)K,
                               (int)N, KS, part, meta, idx, sX, XO, Y, acc);
        else
            hipLaunchKernelGGL((k_dfinish<false, false>), grid, block, 0, s, Wq, sW, W16, (int)T, (int)K,
                               (int)N, KS, part, meta, idx, sX, XO, Y, acc);
    }
}

} // namespace

bool split_shape(int64_t T, int64_t K)
{
    return T >= 1 && T <= kDecodeMaxT && K > kDecodeMaxK;
}

// Slices of K and row-group classes: the grid is at most 256 workgroups
// (one per CU); per workgroup the cost is its row groups times the slice's
// weight bytes, plus its slice's codes and a fixed cost per row group.
SplitPlan split_plan(int64_t T, int64_t K, int64_t N)
{
    const int64_t NRG = (N + 15) / 16;
    const int64_t ks_lo = (K + kSplitMaxSlice - 1) / kSplitMaxSlice, ks_hi = (K + 511) / 512;
    // the fewest slices always fit (slices of at most 8192 columns; their
    // partial sums take at most 1024 * ceil(K/8192) * ceil(N/16) <= N*K bytes)
    const int64_t ksl0 = ((K + ks_lo - 1) / ks_lo + 511) / 512 * 512;
    SplitPlan best{(int)((K + ksl0 - 1) / ksl0), (int)ksl0,
                   (int)std::min<int64_t>(NRG, std::max<int64_t>(1, kDecodeMaxBlocks / ks_lo))};
    double best_cost = 1e300;
    for (int64_t ks = ks_lo; ks <= ks_hi && ks <= kDecodeMaxBlocks; ks++) {
        const int64_t ksl = ((K + ks - 1) / ks + 511) / 512 * 512;
        const int64_t ksr = (K + ksl - 1) / ksl;
        if (ksr != ks)
            continue;
        if (ks * NRG * 1024 > N * K)   // the partial sums must fit where the workspace route keeps them
            continue;
        const int64_t nrgc = std::min<int64_t>(NRG, std::max<int64_t>(1, kDecodeMaxBlocks / ks));
        const int64_t rpw = (NRG + nrgc - 1) / nrgc;
        const double cost = (double)rpw * 16.0 * (double)ksl + (double)T * (double)ksl + 4096.0 * (double)rpw;
        if (cost < best_cost) {
            best_cost = cost;
            best = SplitPlan{(int)ks, (int)ksl, (int)nrgc};
        }
    }
    return best;
}

SplitLayout split_layout(int64_t T, int64_t K, int64_t N)
{
    const size_t A = 256;
    const int64_t nb1 = (K + kScanCols - 1) / kScanCols;
    const SplitPlan p = split_plan(T, K, N);
    const int64_t NRG = (N + 15) / 16;
    SplitLayout L;
    size_t off = 0;
    L.bits = off; off = align_up(off + 4 * (size_t)((K + 31) / 32 + 1), A);
    L.meta = off; off = align_up(off + 256, A);
    L.idx = off;  off = align_up(off + 4 * (size_t)(K + 1), A);
    L.sX = off;   off = align_up(off + 4 * 16, A);
    L.XO = off;   off = align_up(off + 2 * (size_t)T * (size_t)K + 16, A);
    L.ocnt = off; off = align_up(off + 4 * (size_t)nb1, A);
    L.pmax = off; off = align_up(off + 4 * 16 * (size_t)nb1, A);
    L.part = off; off = align_up(off + 1024 * (size_t)p.KS * (size_t)NRG, A);
    L.total = off;
    return L;
}

size_t split_part_bytes(int64_t T, int64_t K, int64_t N)
{
    return 1024 * (size_t)split_plan(T, K, N).KS * (size_t)((N + 15) / 16);
}

hipError_t launch_split_fused(const uint16_t *X, const int8_t *Wq, const float *sW,
                              const uint16_t *W16, uint16_t thr_mag, int64_t T, int64_t K,
                              int64_t N, uint16_t *Y, char *ws, hipStream_t s)
{
    const SplitLayout L = split_layout(T, K, N);
    const SplitPlan p = split_plan(T, K, N);
    const int nb1 = (int)((K + kScanCols - 1) / kScanCols);
    uint32_t *bits = reinterpret_cast<uint32_t *>(ws + L.bits);
    int32_t *ocnt = reinterpret_cast<int32_t *>(ws + L.ocnt);
    uint32_t *pmax = reinterpret_cast<uint32_t *>(ws + L.pmax);
    int32_t *part = reinterpret_cast<int32_t *>(ws + L.part);
    SplitOut out{reinterpret_cast<int32_t *>(ws + L.meta), reinterpret_cast<int32_t *>(ws + L.idx),
                 reinterpret_cast<float *>(ws + L.sX), reinterpret_cast<uint16_t *>(ws + L.XO)};
    if (T <= 8)
        hipLaunchKernelGGL((k_dscan<8>), dim3((unsigned)nb1), dim3(64), 0, s, X, (int)T, (int)K,
                           (uint32_t)thr_mag, bits, ocnt, pmax);
    else
        hipLaunchKernelGGL((k_dscan<16>), dim3((unsigned)nb1), dim3(64), 0, s, X, (int)T, (int)K,
                           (uint32_t)thr_mag, bits, ocnt, pmax);
    launch_split<true>(X, Wq, T, K, N, p, bits, ocnt, pmax, out, nullptr, part, s);
    launch_finish(Wq, sW, W16, T, K, N, p.KS, part, out.meta, out.idx, out.sX, out.XO, Y, nullptr, s);
    return hipGetLastError();
}

hipError_t launch_split_gemm(const int8_t *Wq, const float *sW, const uint16_t *W16, int64_t T,
                             int64_t K, int64_t N, uint16_t *Y, int32_t *acc, const char *ws,
                             const WsLayout &L, hipStream_t s)
{
    const SplitPlan p = split_plan(T, K, N);
    // the partial sums go to the WO region, which the few-token kernels do
    // not read (they gather the outlier weights by index)
    int32_t *part = reinterpret_cast<int32_t *>(const_cast<char *>(ws) + L.WO);
    const int32_t *meta = reinterpret_cast<const int32_t *>(ws + L.meta);
    launch_split<false>(nullptr, Wq, T, K, N, p, nullptr, nullptr, nullptr, SplitOut{},
                        reinterpret_cast<const int8_t *>(ws + L.Xq), part, s);
    launch_finish(Wq, sW, W16, T, K, N, p.KS, part, meta, reinterpret_cast<const int32_t *>(ws + L.idx),
                  reinterpret_cast<const float *>(ws + L.sX), reinterpret_cast<const uint16_t *>(ws + L.XO),
                  Y, acc, s);
    return hipGetLastError();
}

} // namespace li8
