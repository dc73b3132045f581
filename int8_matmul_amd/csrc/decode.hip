// The LLM.int8() layer for few tokens (decode: T <= 16), for gfx950.
//
// Same arithmetic as the prepare kernels followed by the tiled GEMM:
//   O       = { j : some |X[t,j]| > threshold }                (union over t)
//   sX[t]   = fl32(max_{j not in O} |X[t,j]| / 127), Xq codes rne, 0 on O
//   acc     = sum_j Xq[t,j] Wq[n,j]                            (exact int32)
//   D       = fl32(acc * sX[t]) + sum_{j in O} X[t,j] Wq[n,j]  (fp16 MFMA, fp32)
//   Y[t,n]  = fp16(fl32(D * sW[n]))
// (hncyxsy.com/news/230290, section 2.1: outlier columns in fp16, the rest
// in int8 with row and column scales, the two products added in fp16;
// tqpw.cn/news/5683, section 2.1: absmax scales and codes.)
//
// With T <= 16 the layer is bound by reading Wq (N*K bytes) from HBM once;
// every other operand is a few KB.  So the whole call is one kernel:
//  - Each workgroup handles 16-feature row groups (a grid-stride loop).
//    Its first batch of Wq loads is issued at entry, so that the HBM
//    latency overlaps the activation work below.
//  - The activation work: every workgroup reads the T rows of X (L2
//    resident after the first), finds the outlier columns, the row scales
//    and the codes itself, and keeps the codes in LDS.  This is redundant
//    across workgroups, and it avoids three dependent launches.
//  - Per row group, the 8 waves split K; each wave multiplies 16 weight
//    rows (MFMA A operand, straight from global memory) by the token codes
//    (B operand, 16 token slots, from LDS) with v_mfma_i32_16x16x64_i8.
//    The int32 partial sums are added across waves in LDS (exact, so the
//    order does not matter).
//  - Wave 0 finishes the row group: dequantization, the outlier product as
//    v_mfma_f32_16x16x32_f16 over chunks of 32 outlier columns (gathered
//    from X and Wq by column index: the first chunk and the column scales
//    by all threads before the MFMAs, through LDS), the column scale and
//    the fp16 store.
// MW (MFMA waves, the fused variant for K <= 4096): the workgroup gets MW
// more waves that request the weights into their registers and run the int8
// MFMAs once the codes are in LDS; waves 0-7 do the activation work, and
// wave 0 the epilogue.  A wave that issues its share of the weight loads
// stalls at issue while the memory pipeline drains; in waves of their own
// those stalls no longer hold up the activation work.
//  - MW = 4 (one row group per workgroup): each MFMA wave covers the K
//    shares of two activation waves; 12 waves.
//  - MW = 8 (more row groups than workgroups, T <= 8): MFMA wave m covers
//    share m of every row group of the workgroup, with the weights of two
//    row groups in flight and the epilogue operands gathered a group ahead;
//    16 waves of at most 128 registers.
// The variant FUSED = false reads the token codes, scales and outlier
// columns that the prepare kernels left in the workspace instead of
// deriving them; everything after that is the same code, so the two
// variants give bit-identical results.  F16W: the outlier columns multiply
// the original fp16 weight W16 (the fp16-weight variant), and the sum is
// D = fl32(fl32(acc * sX) * sW) + sum_O X * W16.
#include <type_traits>

#include "li8_internal.h"
#include "quant_math.h"

namespace li8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kDThreads = 512;   // 8 waves, two per SIMD
constexpr int kDWaves = kDThreads / 64;
constexpr int kDRows = 16;       // output features per row group
constexpr int kDMaxT = kDecodeMaxT;
constexpr int kDMaxK = kDecodeMaxK;
constexpr int kOutOfRange = (int)0x80000000;   // buffer offset past any operand

// LDS carve-up (bytes).  Token codes: block q (columns 16q..16q+15) holds
// the 16 codes of token t at q*QS + 16t, QS = 16T + 16 (the 16-byte pad
// spreads the writes of consecutive blocks over the banks).
constexpr int kXqMax = kDMaxK / 16 * (16 * kDMaxT + 16);
constexpr int kOffBits = kXqMax;                          // uint32[K/32]
constexpr int kOffPre = kOffBits + 4 * (kDMaxK / 32);     // int32[K/32]
constexpr int kOffRmax = kOffPre + 4 * (kDMaxK / 32);     // uint32[16][8]: token-major wave maxima
constexpr int kOffSx = kOffRmax + 4 * kDWaves * kDMaxT;   // float[16] token scales
constexpr int kOffRed = kOffSx + 4 * kDMaxT;              // v4i[2][8][64]
constexpr int kIdxCap = 256;                              // outlier columns listed in LDS
constexpr int kOffIdx = kOffRed + 2 * kDWaves * 64 * 16;  // int32[kIdxCap]
constexpr int kMaxCpt = kDMaxK / (8 * kDThreads);         // 8-column chunks per thread
constexpr int kOffOcnt = kOffIdx + 4 * kIdxCap;           // int32[kMaxCpt][8] outlier columns per wave
// the first 32 outlier columns of the row group's 16 weight rows and of the
// 16 token slots, and the group's 16 column scales, gathered by all threads;
// two copies, alternating between row groups like the partial sums, since
// the other waves write the next group's copy while wave 0 may still read
// this one
constexpr int kOffGw = kOffOcnt + 4 * kMaxCpt * kDWaves;  // uint16[2][16][32] code bytes (or fp16 weights)
constexpr int kOffGx = kOffGw + 2 * 2 * 16 * 32;          // uint16[2][16][32] fp16 activations
constexpr int kOffGs = kOffGx + 2 * 2 * 16 * 32;          // float[2][16]
constexpr int kLds = kOffGs + 2 * 4 * kDRows;
static_assert(kLds <= 160 * 1024, "LDS of one workgroup");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, 0x00020000);
}

// 16 bytes of Wq at byte offset `off` (kOutOfRange reads zeros).
__device__ __forceinline__ v4i load_w16(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Columns of the outlier set with ranks i0 .. i0+7 (ascending), from the
// bit set and the exclusive prefix counts of its words; -1 past nO.
__device__ void outlier_columns8(const uint32_t *bits, const int32_t *pre, int nw, int nO, int i0,
                                 int col[8])
{
#pragma unroll
    for (int e = 0; e < 8; e++)
        col[e] = -1;
    if (i0 >= nO)
        return;
    // the word holding rank i0: the last word whose prefix is <= i0
    int lo = 0, hi = nw - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= i0)
            lo = mid;
        else
            hi = mid - 1;
    }
    int w = lo;
    uint32_t b = bits[w];
    for (int s = i0 - pre[w]; s > 0; s--)
        b &= b - 1u;
#pragma unroll
    for (int e = 0; e < 8; e++) {
        if (i0 + e >= nO)
            break;
        col[e] = 32 * w + __ffs(b) - 1;
        b &= b - 1u;
        while (b == 0u && w + 1 < nw)
            b = bits[++w];
    }
}

// Magnitude masks for the 8 binary16 values of a chunk (dword i holds
// columns 2i and 2i+1): halfword e is 0x7fff where bit e of `skip` is clear
// and 0 where it is set, so that one AND gives the magnitude of a column
// outside the outlier set and 0 for one inside it.
__device__ __forceinline__ uint4 keep_mag_halves8(uint32_t skip)
{
    const uint2 kb = keep_bytes8(skip);   // byte e: 0xff kept, 0 skipped
    // bytes (e, e, e+1, e+1) of the byte masks (v_perm_b32 selects)
    return make_uint4(__builtin_amdgcn_perm(kb.x, kb.x, 0x01010000u) & 0x7fff7fffu,
                      __builtin_amdgcn_perm(kb.x, kb.x, 0x03030202u) & 0x7fff7fffu,
                      __builtin_amdgcn_perm(kb.y, kb.y, 0x01010000u) & 0x7fff7fffu,
                      __builtin_amdgcn_perm(kb.y, kb.y, 0x03030202u) & 0x7fff7fffu);
}

// Max magnitude of a chunk's values under the masks of keep_mag_halves8.
__device__ __forceinline__ uint32_t chunk_max_keep(uint4 v, uint4 km)
{
    li8_us2 m = __builtin_elementwise_max(__builtin_bit_cast(li8_us2, v.x & km.x),
                                          __builtin_bit_cast(li8_us2, v.y & km.y));
    m = __builtin_elementwise_max(m, __builtin_bit_cast(li8_us2, v.z & km.z));
    m = __builtin_elementwise_max(m, __builtin_bit_cast(li8_us2, v.w & km.w));
    return max((uint32_t)m.x, (uint32_t)m.y);
}

// Lane exchange within rows of 16 (DPP control code) folded into a max.
template <int CTRL>
__device__ __forceinline__ uint32_t max_dpp(uint32_t keep, uint32_t send)
{
    return max(keep, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, CTRL, 0xF, 0xF, false));
}

// Maxima over the 64 lanes of a wave of TB values per lane (TB = 8 or 16),
// all at once.  A step at lane distance d takes the n values still held
// and pairs value i with value i + n/2: lanes whose index has bit d clear
// keep token i, the others token i + n/2, and each combines its own value
// with its partner's (a lane whose bit d differs), so every step halves
// the values held.  After the steps for d = 32 .. 64/TB lane l holds part
// of the maximum of token l / (64/TB), and the last steps reduce within
// those groups of 64/TB lanes.  Exchanges: the gfx950 lane swaps for
// d = 32 and 16 (the swap itself places the two tokens), DPP within rows
// for the rest (rotate by 8; the half-row mirror, which pairs each lane
// with one whose bit 2 differs; quad permutations).  Returns the token's
// maximum in every lane of its group.
template <int TB>
__device__ __forceinline__ uint32_t wave_max_tokens(const uint32_t (&v)[TB], int lane)
{
    static_assert(TB == 8 || TB == 16, "token slots");
    uint32_t a[TB / 2], b[TB / 4], c[TB / 8];
#pragma unroll
    for (int i = 0; i < TB / 2; i++) {   // lanes 0-31: token i, 32-63: token i + TB/2
        const auto r = __builtin_amdgcn_permlane32_swap(v[i], v[i + TB / 2], false, false);
        a[i] = max((uint32_t)r[0], (uint32_t)r[1]);
    }
#pragma unroll
    for (int i = 0; i < TB / 4; i++) {   // rows 0, 2: the first value's token, rows 1, 3: the second's
        const auto r = __builtin_amdgcn_permlane16_swap(a[i], a[i + TB / 4], false, false);
        b[i] = max((uint32_t)r[0], (uint32_t)r[1]);
    }
    const bool s8 = (lane & 8) != 0;
#pragma unroll
    for (int i = 0; i < TB / 8; i++)
        c[i] = max_dpp<0x128>(s8 ? b[i + TB / 8] : b[i], s8 ? b[i] : b[i + TB / 8]);   // row_ror:8
    uint32_t m;
    if constexpr (TB == 16) {
        const bool s4 = (lane & 4) != 0;
        m = max_dpp<0x141>(s4 ? c[1] : c[0], s4 ? c[0] : c[1]);   // row_half_mirror
    } else {
        m = max_dpp<0x141>(c[0], c[0]);
    }
    m = max_dpp<0x4E>(m, m);   // quad_perm [2,3,0,1]
    return max_dpp<0xB1>(m, m);   // quad_perm [1,0,3,2]
}

// The MFMA waves of the MW = 4 variant (wave mw = 0..3 of them): the weight
// rows of the workgroup's row group over the K shares of activation waves
// 2mw and 2mw+1, 16 loads of 16 bytes per lane, then the int8 MFMAs with the
// token codes from LDS, the partial sums to red[mw].  The barriers pair with
// the activation waves' (issue, row maxima, outlier list, codes, reduction):
// 12 of the weight loads before the row-maxima barrier and the other 4 before
// the next, a split at which these waves reach each barrier about when the
// activation waves do.
template <int KB>
__device__ __forceinline__ void mfma_wave(const int8_t *__restrict__ Wq, int T, int K, int N,
                                          const int8_t *lds, v4i *red, int mw, int lane)
{
    static_assert(KB == 8, "two shares of 8 k-steps");
    constexpr int NL = 2 * KB;
    const int S = (K + 63) / 64;
    const int QS = 16 * T + 16;
    const int kg = lane >> 4, tok = lane & 15;
    const int n = min((int)blockIdx.x * kDRows + (lane & 15), N - 1);
    const __amdgpu_buffer_rsrc_t rW = make_rsrc(Wq, N * K);
    v4i wr[NL];
    // load i: share w = 2mw + i / KB, its k-step j = i % KB (zeros past the
    // share's end, so that a k-step is counted by exactly one share)
    auto wl = [&](int i) {
        const int w = 2 * mw + i / KB, j = i % KB;
        const int s0 = w * S / kDWaves, s1 = (w + 1) * S / kDWaves;
        const int k = (s0 + j) * 64 + 16 * kg;
        wr[i] = load_w16(rW, k < min(s1 * 64, K) ? n * K + k : kOutOfRange);
    };
    __builtin_amdgcn_s_barrier();   // issue barrier: the activation loads go first
#pragma unroll
    for (int i = 0; i < 12; i++)
        wl(i);
    lds_barrier();   // row maxima
#pragma unroll
    for (int i = 12; i < NL; i++)
        wl(i);
    lds_barrier();   // outlier list
    lds_barrier();   // codes in LDS
    // every code fragment first (all reads in flight), then the MFMAs.  No
    // masks: a token slot past T only feeds outputs that are never stored,
    // and a k-step past a share's end meets zero weights; the addresses stay
    // inside the code region (k-step < 64, QS <= 272)
    v4i xf[NL];
#pragma unroll
    for (int i = 0; i < NL; i++) {
        const int w = 2 * mw + i / KB, j = i % KB;
        const int q = (w * S / kDWaves + j) * 4 + kg;
        xf[i] = *reinterpret_cast<const v4i *>(lds + q * QS + 16 * tok);
    }
    __builtin_amdgcn_sched_barrier(0);
    v4i acc = {0, 0, 0, 0}, acc2 = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < NL; i += 2) {
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wr[i], xf[i], acc, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(wr[i + 1], xf[i + 1], acc2, 0, 0, 0);
    }
    red[mw * 64 + lane] = acc + acc2;   // (copy 0)
    lds_barrier();   // reduction
}

// TB: a compile-time bound on T (8 or 16), so that the per-token loops of
// the activation work run over T <= 8 slots when that suffices.  MW: see the
// file comment (launched with 8 + MW waves).
template <bool FUSED, int KB, int TB, bool F16W, bool STORE_ACC, int MW>
__global__ __launch_bounds__(kDThreads + 64 * MW) void k_decode(
    const uint16_t *__restrict__ X, const int8_t *__restrict__ Wq, const float *__restrict__ sW,
    const uint16_t *__restrict__ W16,
    uint32_t thr_mag, int T, int K, int N,
    const int32_t *__restrict__ meta, const int32_t *__restrict__ idx_g,
    const float *__restrict__ sX_g, const int8_t *__restrict__ Xq_g,
    const uint16_t *__restrict__ XO_g, uint16_t *__restrict__ Y, int32_t *__restrict__ acc_out)
{
    static_assert(KB % 8 == 0, "weight loads per lane come in groups of 8");
    __shared__ __attribute__((aligned(16))) int8_t lds[kLds];
    int8_t *xq = lds;
    uint32_t *bits = reinterpret_cast<uint32_t *>(lds + kOffBits);
    int32_t *pre = reinterpret_cast<int32_t *>(lds + kOffPre);
    uint32_t *rmax = reinterpret_cast<uint32_t *>(lds + kOffRmax);
    float *sxl = reinterpret_cast<float *>(lds + kOffSx);
    int32_t *idxl = reinterpret_cast<int32_t *>(lds + kOffIdx);
    int32_t *ocnt = reinterpret_cast<int32_t *>(lds + kOffOcnt);
    uint16_t *gwl = reinterpret_cast<uint16_t *>(lds + kOffGw);
    uint16_t *gxl = reinterpret_cast<uint16_t *>(lds + kOffGx);
    float *gsl = reinterpret_cast<float *>(lds + kOffGs);
    v4i *red = reinterpret_cast<v4i *>(lds + kOffRed);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr bool ROLES = MW != 0;   // the MFMA waves hold the products
    static_assert(MW == 0 || (FUSED && KB == 8), "MFMA waves: the fused variant, K <= 4096");
    static_assert(MW != 8 || TB == 8, "8 MFMA waves: 16 waves of at most 128 registers");
    if constexpr (MW == 4) {
        if (wid >= kDWaves) {
            mfma_wave<KB>(Wq, T, K, N, lds, red, wid - kDWaves, lane);
            return;
        }
    }
    const int QS = 16 * T + 16;
    const int NRG = (N + kDRows - 1) / kDRows;
    const int G = gridDim.x;

    // ---- this wave's share of K: MFMA k-steps [s0, s1) of 64 columns ----
    const int S = (K + 63) / 64;
    const int wsh = wid & (kDWaves - 1);   // (an MFMA wave of MW = 8 takes share wid - 8)
    const int s0 = wsh * S / kDWaves, s1 = (wsh + 1) * S / kDWaves;
    const int kg = lane >> 4;     // 16-byte group of the k-step this lane supplies
    const int tok = lane & 15;    // token slot (B column) of this lane
    const __amdgpu_buffer_rsrc_t rW = make_rsrc(Wq, N * K);

    // Every load below is unconditional, with an out-of-range offset (zeros)
    // where a lane has nothing to read, and the test is per lane: loads
    // behind branches leave the compiler unable to count the loads in
    // flight, and it then waits for all of them (weights included) before
    // the first use of any.
    v4i wbuf[2][KB];
    const int kend = min(s1 * 64, K);   // end of this wave's share of K
    // (a row group past the last one, rg >= NRG, reads zeros)
    auto wload = [&](int set, int rg) {
        const int n = min(rg * kDRows + (lane & 15), N - 1);
        const int kl = rg < NRG ? kend : 0;
#pragma unroll
        for (int j = 0; j < KB; j++) {
            const int k = (s0 + j) * 64 + 16 * kg;
            wbuf[set][j] = load_w16(rW, k < kl ? n * K + k : kOutOfRange);
        }
    };
    int rg = blockIdx.x;

    // ---- token codes, scales, outlier set ----
    // The activation loads are issued before the first weight batch: loads
    // complete in order, so this way the activation work waits only for
    // its own data while the weight batch is in flight.  (The fused
    // variant with two chunks of X per thread for 16 token slots has no
    // registers to spare for the weights during that work: it requests
    // them after it.)
    constexpr bool kEarly = !(FUSED && KB > 8 && TB > 8);
    int nO;
    int g_idx = 0;   // workspace path: column of outlier rank tid % 32 (loaded before the weights)
    // The epilogue's small operands for row group rgc, spread over all 512
    // threads: thread (r = tid / 32, e = tid % 32) fetches the weight of row
    // r and the activation of token slot r at outlier rank e, threads 0..15
    // the column scales.  Unconditional buffer loads (zeros past the ends).
    // gather_store puts them in LDS copy `par`.
    const int gt = tid & (kDThreads - 1);   // (MW = 8: the MFMA waves gather as threads 0..511)
    // (the column of rank e is the same for every row group)
    auto gather_col = [&]() -> int {
        const int e = gt & 31;
        int col = 0;
        if constexpr (FUSED) {
            if (nO <= kIdxCap) {
                col = idxl[min(e, kIdxCap - 1)];
            } else {   // more columns than the LDS list holds
                int c8[8];
                outlier_columns8(bits, pre, (K + 31) / 32, nO, e, c8);
                col = max(c8[0], 0);
            }
        } else {
            col = min(max(g_idx, 0), K - 1);
        }
        return col;
    };
    auto gather_at = [&](int rgc, int col, uint32_t &g_w, uint32_t &g_x, uint32_t &g_s) {
        const int e = gt & 31, r = gt >> 5;
        // a row group past the last one gathers nothing: an empty buffer
        // at the last group's rows (every offset out of range, zeros)
        const int rows = rgc < NRG ? min(kDRows, N - rgc * kDRows) : 0;
        const int64_t rbase = (int64_t)min(rgc, NRG - 1) * kDRows * K;
        const __amdgpu_buffer_rsrc_t rWg =
            F16W ? make_rsrc(W16 + rbase, 2 * rows * K) : make_rsrc(Wq + rbase, rows * K);
        const int wo = r * K + col;
        const int woff = (e < nO && r < rows) ? (F16W ? 2 * wo : wo) : kOutOfRange;
        if constexpr (F16W)
            g_w = __builtin_amdgcn_raw_buffer_load_b16(rWg, woff, 0, 0);
        else
            g_w = __builtin_amdgcn_raw_buffer_load_b8(rWg, woff, 0, 0);   // (code byte)
        // 16-column chunks of XO: rank i of token t at ((i / 16) * T + t) * 16 + i % 16
        const int xo = FUSED ? r * K + col : ((e >> 4) * T + r) * 16 + (e & 15);
        const __amdgpu_buffer_rsrc_t rXg = FUSED ? make_rsrc(X, 2 * T * K) : make_rsrc(XO_g, 2 * T * K);
        g_x = __builtin_amdgcn_raw_buffer_load_b16(rXg, (e < nO && r < T) ? 2 * xo : kOutOfRange, 0, 0);
        g_s = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(sW, 4 * N),
                                                   gt < kDRows ? 4 * min(rgc * kDRows + gt, N - 1)
                                                               : kOutOfRange,
                                                   0, 0);
    };
    auto gather_issue = [&](int rgc, uint32_t &g_w, uint32_t &g_x, uint32_t &g_s) {
        gather_at(rgc, gather_col(), g_w, g_x, g_s);
    };
    auto gather_store = [&](int par, uint32_t g_w, uint32_t g_x, uint32_t g_s) {
        gwl[par * 16 * 32 + gt] = (uint16_t)g_w;   // [r][e] = gt
        gxl[par * 16 * 32 + gt] = (uint16_t)g_x;
        if (gt < kDRows)
            gsl[par * kDRows + gt] = __builtin_bit_cast(float, g_s);
    };
    // row groups of this workgroup: rg, rg + G, ... (the grid is at most NRG)
    const int nG = (NRG - (int)blockIdx.x + G - 1) / G;

    if constexpr (MW == 8) {
        if (wid >= kDWaves) {
            // MFMA waves: share wsh of every row group of the workgroup, the
            // weights in registers (two row groups in flight); each row
            // group's partial sums to red[set] and its epilogue operands,
            // gathered one group ahead, to copy `set`.  Barriers pair with the
            // activation waves' (issue, row maxima, outlier list, codes) and
            // then with wave 0's, one per row group.
            __builtin_amdgcn_s_barrier();   // issue barrier: the activation loads go first
            wload(0, rg);
            lds_barrier();   // row maxima
            nO = 0;
#pragma unroll
            for (int w = 0; w < kDWaves; w++)
                nO += ocnt[w];
            wload(1, rg + G);   // (zeros past the last row group)
            lds_barrier();   // outlier list
            const int gcol = gather_col();
            uint32_t c_w, c_x, c_s;
            gather_at(rg, gcol, c_w, c_x, c_s);
            lds_barrier();   // codes in LDS
            // Row group i uses weight set i % 2; two groups per iteration so
            // that the set is fixed at compile time.  The fragments need no
            // masks: a token slot past T only feeds outputs that are never
            // stored, a k-step past the share or past K meets zero weights.
            auto step = [&](auto set_c, int i) {
                constexpr int set = decltype(set_c)::value;
                uint32_t n_w, n_x, n_s;
                gather_at(rg + (i + 1) * G, gcol, n_w, n_x, n_s);   // (zeros past the last group)
                // code fragments in two batches of four, each read ahead of
                // its MFMAs (register budget: 16 waves of at most 128)
                v4i acc = {0, 0, 0, 0};
#pragma unroll
                for (int h = 0; h < KB; h += 4) {
                    v4i xf[4];
#pragma unroll
                    for (int j = 0; j < 4; j++)
                        xf[j] = *reinterpret_cast<const v4i *>(lds + ((s0 + h + j) * 4 + kg) * QS + 16 * tok);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int j = 0; j < 4; j++)
                        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wbuf[set][h + j], xf[j], acc, 0, 0, 0);
                }
                wload(set, rg + (i + 2) * G);   // (zeros past the last group)
                gather_store(set, c_w, c_x, c_s);
                red[(set * kDWaves + wsh) * 64 + lane] = acc;
                lds_barrier();   // this row group's partial sums and operands
                c_w = n_w;
                c_x = n_x;
                c_s = n_s;
            };
            for (int i = 0; i < nG; i += 2) {
                step(std::integral_constant<int, 0>{}, i);
                if (i + 1 >= nG)
                    break;
                step(std::integral_constant<int, 1>{}, i + 1);
            }
            return;
        }
    }


    if constexpr (FUSED) {
        constexpr int CPT = KB / 8;   // 8-column chunks per thread: K <= 4096*CPT
        static_assert(CPT <= kMaxCpt, "chunks per thread");
        const int nchunk = K / 8;
        const __amdgpu_buffer_rsrc_t rX = make_rsrc(X, 2 * T * K);
        uint4 xv[CPT][TB];
#pragma unroll
        for (int u = 0; u < CPT; u++) {
            const int c = tid + u * kDThreads;
#pragma unroll
            for (int t = 0; t < TB; t++) {   // rows past T and chunks past K read zeros
                const bool ok = (t < T) & (c < nchunk);
                xv[u][t] = __builtin_bit_cast(uint4, load_w16(rX, ok ? 16 * (t * (K / 8) + c) : kOutOfRange));
            }
        }
        // every wave's activation loads ahead of any weight load in the
        // memory pipeline (a barrier on issue only: no wait for data)
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kEarly && !ROLES)   // (rg = blockIdx.x < NRG: the grid is at most NRG)
            wload(0, rg);
        uint32_t fl[CPT];
        int orank[CPT];   // outlier columns before this chunk's, within this wave and pass u
        uint32_t rm[TB];
#pragma unroll
        for (int t = 0; t < TB; t++)
            rm[t] = 0;
#pragma unroll
        for (int u = 0; u < CPT; u++) {
            const int c = tid + u * kDThreads;
            li8_us2 mx[4] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
#pragma unroll
            for (int t = 0; t < TB; t++)
                column_max8(mx, xv[u][t]);   // padding rows are zero
            fl[u] = outlier_flags8(mx, thr_mag);
            // chunks 4w..4w+3 sit in four consecutive lanes: one word
            uint32_t word = fl[u] << (8 * (c & 3));
            word |= (uint32_t)__shfl_xor((int)word, 1, 64);
            word |= (uint32_t)__shfl_xor((int)word, 2, 64);
            if ((c & 3) == 0 && c < nchunk)
                bits[c >> 2] = word;
            // ranks of the outlier columns: chunks are ordered by (u, tid),
            // so an exclusive prefix of the per-chunk counts (0..8) over the
            // lanes, bit by bit with ballots, and per-wave totals in LDS
            {
                const int cnt = __popc(fl[u]);
                const uint64_t below = (1ull << lane) - 1ull;
                int p = 0, tot = 0;
#pragma unroll
                for (int bit = 0; bit < 4; bit++) {
                    const uint64_t m = __ballot((cnt >> bit) & 1);
                    p += __popcll(m & below) << bit;
                    tot += __popcll(m) << bit;
                }
                orank[u] = p;
                if (lane == 0)
                    ocnt[u * kDWaves + wid] = tot;
            }
            // row maxima over the chunk's columns outside the outlier set:
            // masks only in a wave where some lane's chunk holds one (a
            // wave-uniform branch, no divergence over the 8 columns)
            if (__ballot(fl[u] != 0u) != 0ull) {
                const uint4 km = keep_mag_halves8(fl[u]);
#pragma unroll
                for (int t = 0; t < TB; t++)
                    rm[t] = max(rm[t], chunk_max_keep(xv[u][t], km));
            } else {
#pragma unroll
                for (int t = 0; t < TB; t++)
                    rm[t] = max(rm[t], chunk_max(xv[u][t], 0u));
            }
        }
        {   // the wave's maxima of all TB tokens at once: token t in lanes
            // t * 64/TB .. (t+1) * 64/TB - 1
            const uint32_t m = wave_max_tokens<TB>(rm, lane);
            if ((lane & (64 / TB - 1)) == 0)
                rmax[(lane / (64 / TB)) * kDWaves + wid] = m;
        }
        lds_barrier();
        // Every wave derives the token scales itself, lane t for token t:
        // the maximum over the waves' partial maxima, the scale and its
        // reciprocal (IEEE divisions), broadcast across the wave; no second
        // barrier.  Wave 0 keeps the scales in LDS for the epilogue.
        float sx[TB], rx[TB];
        {
            // the 8 wave maxima of token min(lane, TB - 1) in two 16-byte
            // reads (unconditional: a masked read is a branch per read)
            const uint4 m0 = *reinterpret_cast<const uint4 *>(rmax + min(lane, TB - 1) * kDWaves);
            const uint4 m1 = *reinterpret_cast<const uint4 *>(rmax + min(lane, TB - 1) * kDWaves + 4);
            uint32_t m = max(max(max(m0.x, m0.y), max(m0.z, m0.w)), max(max(m1.x, m1.y), max(m1.z, m1.w)));
            m = lane < TB ? m : 0u;
            const float sc = h2f(m) / 127.0f;
            const float rc = 1.0f / sc;
            if (wid == 0 && lane < kDMaxT)
                sxl[lane] = sc;
            // A token with sc = 0 has only zeros outside the outlier set,
            // whose codes are 0; the pair (1, 1) gives exactly those codes
            // (and 0 for the masked outlier positions), so the code loop
            // needs no test per token.
            const float sq = sc == 0.0f ? 1.0f : sc, rq = sc == 0.0f ? 1.0f : rc;
#pragma unroll
            for (int t = 0; t < TB; t++) {
                sx[t] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sq), t));
                rx[t] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rq), t));
            }
        }
        // nO and the rank of this thread's first outlier column in each pass
        nO = 0;
#pragma unroll
        for (int u = 0; u < CPT; u++) {
            int before = 0, pass = 0;   // this pass: waves before this one, all waves
#pragma unroll
            for (int w = 0; w < kDWaves; w++) {
                const int v = ocnt[u * kDWaves + w];
                before += (w < wid) ? v : 0;
                pass += v;
            }
            orank[u] += nO + before;
            nO += pass;
        }
        // the ascending list of outlier columns (while it fits in LDS), and
        // the rank of each bit-set word's first column for the rank search
        // past that; each thread writes its own chunks' entries
#pragma unroll
        for (int u = 0; u < CPT; u++) {
            const int c = tid + u * kDThreads;
            if ((c & 3) == 0 && c < nchunk)
                pre[c >> 2] = orank[u];
            if (nO <= kIdxCap) {
                uint32_t b = fl[u];
                int p = orank[u];
                while (b) {
                    idxl[p++] = 8 * c + __ffs(b) - 1;
                    b &= b - 1u;
                }
            }
        }
        // (the list and the prefixes for every thread's rank search)
        lds_barrier();
        // the first row group's epilogue operands, requested now so that
        // their latency passes during the code computation
        uint32_t e_w = 0, e_x = 0, e_s = 0;
        if constexpr (MW != 8)
            gather_issue(rg, e_w, e_x, e_s);
#pragma unroll
        for (int u = 0; u < CPT; u++) {
            const int c = tid + u * kDThreads;
            const uint2 keep = keep_bytes8(fl[u]);   // the chunk's columns are the same for every token
            if (c < nchunk) {
#pragma unroll
                for (int t = 0; t < TB; t++)
                    if (t < T) {
                        const uint2 q = token_codes8_keep(xv[u][t], keep, sx[t], rx[t]);
                        *reinterpret_cast<uint2 *>(xq + (c >> 1) * QS + 16 * t + 8 * (c & 1)) = q;
                    }
            }
        }
        if constexpr (MW != 8)
            gather_store(0, e_w, e_x, e_s);
        lds_barrier();
    } else {
        // token codes of the prepared workspace into the LDS layout: up to
        // 16 chunks of 16 bytes per thread (T*K/16 <= 16*512)
        // clamped, so that a workspace no prepare call wrote (outside the
        // contract) gives wrong values, not reads out of bounds
        nO = min(max(meta[0], 0), K);
        const int nq = K / 16, tot = T * nq;
        const __amdgpu_buffer_rsrc_t rQ = make_rsrc(Xq_g, T * K);
        const __amdgpu_buffer_rsrc_t rS = make_rsrc(sX_g, 4 * T);
        uint4 st[TB];
#pragma unroll
        for (int j = 0; j < TB; j++) {   // (row-major [T,K]: chunk i is at byte 16 i)
            const int i = tid + j * kDThreads;
            st[j] = __builtin_bit_cast(uint4, load_w16(rQ, i < tot ? 16 * i : kOutOfRange));
        }
        // the token scales too before the weights: loads complete in order,
        // so a later load would wait for the whole weight batch
        const float sxg = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rS, tid < T ? 4 * tid : kOutOfRange, 0, 0));
        // and the first 32 outlier columns' indices, which the epilogue
        // gathers are addressed by
        g_idx = (int)__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(idx_g, 4 * K),
                                                          (tid & 31) < nO ? 4 * (tid & 31) : kOutOfRange, 0, 0);
        wload(0, rg);
#pragma unroll
        for (int j = 0; j < TB; j++) {
            const int i = tid + j * kDThreads;
            if (i < tot) {
                const int t = i / nq, q = i - t * nq;
                *reinterpret_cast<uint4 *>(xq + q * QS + 16 * t) = st[j];
            }
        }
        if (tid < kDMaxT)
            sxl[tid] = sxg;
        lds_barrier();
    }

    if constexpr (!kEarly)
        wload(0, rg);

    // ---- row groups: int8 MFMAs over this wave's share of K ----
    // Outlier operands of 8 consecutive ranks from i0 for this lane (wave 0,
    // outlier chunks past the first): the raw values (weight of this lane's
    // row, binary16 of token tok; buffer loads, zeros past the ends), then
    // the MFMA fragments with the ranks past nO (and padding tokens) zeroed.
    auto gather_raw = [&](int rgc, int i0, int (&wr)[8], uint32_t (&xr)[8]) {
        int col[8];
        if constexpr (FUSED) {
            if (nO <= kIdxCap) {
#pragma unroll
                for (int e = 0; e < 8; e++)
                    col[e] = (i0 + e < nO) ? idxl[i0 + e] : 0;
            } else {   // more columns than the LDS list holds
                outlier_columns8(bits, pre, (K + 31) / 32, nO, i0, col);
#pragma unroll
                for (int e = 0; e < 8; e++)
                    col[e] = max(col[e], 0);
            }
        } else {
            const __amdgpu_buffer_rsrc_t rI = make_rsrc(idx_g, 4 * K);
#pragma unroll
            for (int e = 0; e < 8; e++)
                col[e] = min(max((int)__builtin_amdgcn_raw_buffer_load_b32(
                                     rI, i0 + e < nO ? 4 * (i0 + e) : kOutOfRange, 0, 0),
                                 0),
                             K - 1);
        }
        // weight rows of this row group (at most 16 rows of K elements from
        // its first row, so the offsets stay small), token rows of X / XO
        const int rows = min(kDRows, N - rgc * kDRows);
        const int wl = min(rgc * kDRows + (lane & 15), N - 1) - rgc * kDRows;   // local weight row
        const __amdgpu_buffer_rsrc_t rWg =
            F16W ? make_rsrc(W16 + (int64_t)rgc * kDRows * K, 2 * rows * K)
                 : make_rsrc(Wq + (int64_t)rgc * kDRows * K, rows * K);
        const int ttok = min(tok, T - 1);
        const __amdgpu_buffer_rsrc_t rXg = FUSED ? make_rsrc(X, 2 * T * K) : make_rsrc(XO_g, 2 * T * K);
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const bool ok = i0 + e < nO;
            const int wo = wl * K + col[e];
            int xo;
            if constexpr (FUSED) {
                xo = ttok * K + col[e];
            } else {   // 16-column chunks: rank i of token t at ((i / 16) * T + t) * 16 + i % 16
                const int i = i0 + e;
                xo = ((i >> 4) * T + ttok) * 16 + (i & 15);
            }
            const int woff = ok ? (F16W ? 2 * wo : wo) : kOutOfRange;
            const int xoff = ok ? 2 * xo : kOutOfRange;
            if constexpr (F16W)
                wr[e] = __builtin_amdgcn_raw_buffer_load_b16(rWg, woff, 0, 0);
            else
                wr[e] = (int8_t)__builtin_amdgcn_raw_buffer_load_b8(rWg, woff, 0, 0);
            xr[e] = __builtin_amdgcn_raw_buffer_load_b16(rXg, xoff, 0, 0);
        }
    };
    auto fragments = [&](int i0, const int (&wr)[8], const uint32_t (&xr)[8], v8h &a, v8h &b) {
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const bool ok = i0 + e < nO;
            if constexpr (F16W)
                a[e] = ok ? __builtin_bit_cast(_Float16, (uint16_t)wr[e]) : (_Float16)0.0f;
            else
                a[e] = ok ? (_Float16)(float)wr[e] : (_Float16)0.0f;
            b[e] = (ok && tok < T) ? __builtin_bit_cast(_Float16, (uint16_t)xr[e]) : (_Float16)0.0f;
        }
    };

    auto process = [&](int set, int rgc, int par, bool gathered) {
        // The epilogue's small operands (gathered here unless the activation
        // work already did, for the first row group of the fused variant),
        // requested before the MFMAs: loads complete in order, so the MFMAs
        // wait only for the older weight loads.  They go to LDS after the
        // MFMAs, for wave 0 to read after the reduction barrier.
        const int nb = rgc * kDRows + 4 * kg;   // this lane's first feature
        uint32_t g_w = 0, g_x = 0, g_s = 0;
        if (!gathered)
            gather_issue(rgc, g_w, g_x, g_s);
        // fragment reads 8 at a time, all in flight ahead of their MFMAs,
        // which alternate between two accumulators (the int32 sums are
        // exact, so splitting the dependency chain changes nothing).  No
        // masks: a token slot past T only feeds outputs that are never
        // stored, and a k-step past the wave's share or past K meets zero
        // weights.  The reads stay inside the code region: k-steps below
        // 8 * KB and token slots below 16 address at most 32 * KB blocks of
        // at most 272 bytes.
        if constexpr (ROLES) {   // the MFMA waves hold the products
            if (wid != 0)
                return;
            lds_barrier();   // reduction
        } else {
        v4i acc = {0, 0, 0, 0}, acc2 = {0, 0, 0, 0};
#pragma unroll
        for (int h = 0; h < KB; h += 8) {
            v4i xf[8];
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const int q = (s0 + h + j) * 4 + kg;
                xf[j] = *reinterpret_cast<const v4i *>(lds + q * QS + 16 * tok);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wbuf[set][h + j], xf[j], acc, 0, 0, 0);
                acc2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(wbuf[set][h + j + 1], xf[j + 1], acc2, 0, 0, 0);
            }
        }
        // (no scheduling across: the stores below wait for the gathers)
        __builtin_amdgcn_sched_barrier(0);
        acc += acc2;
        if (!gathered)
            gather_store(par, g_w, g_x, g_s);
        red[(par * kDWaves + wid) * 64 + lane] = acc;
        lds_barrier();
        if (wid != 0)
            return;
        }
        const uint16_t *gw = gwl + par * 16 * 32, *gx = gxl + par * 16 * 32;
        const float *gs = gsl + par * kDRows;
        float swv[4];
#pragma unroll
        for (int r = 0; r < 4; r++)
            swv[r] = gs[4 * kg + r];
        // wave 0: lane holds token tok and features nb .. nb+3
        v4i tot = red[par * kDWaves * 64 + lane];
#pragma unroll
        for (int w = 1; w < (MW == 4 ? 4 : kDWaves); w++)
            tot += red[(par * kDWaves + w) * 64 + lane];
        if constexpr (STORE_ACC) {
            if (tok < T)
#pragma unroll
                for (int r = 0; r < 4; r++)
                    if (nb + r < N)
                        acc_out[(int64_t)tok * N + nb + r] = tot[r];
        }
        const float sx = sxl[tok];
        v4f d;
#pragma unroll
        for (int r = 0; r < 4; r++)
            d[r] = (float)tot[r] * sx;
        if constexpr (F16W)   // the fp16 outlier product is then in output units
#pragma unroll
            for (int r = 0; r < 4; r++)
                d[r] *= swv[r];
        // D += X[:, O] . Wq[:, O]^T, 32 outlier columns per MFMA: lane
        // supplies weight row (lane & 15) and token tok at ranks
        // 32c + 8*kg .. +7.  Chunk 0 from the LDS copies, straight-line code
        // for the common case of at most 32 outlier columns; later chunks
        // gathered here.  The copies hold zeros past rank nO and past token
        // T, so chunk 0 needs no masks, and with no outlier columns at all
        // it adds exact zeros (d is never -0: its integer part is not -0 and
        // the scales are not negative).
        {
            const int i0 = 8 * kg;
            const uint4 wv = *reinterpret_cast<const uint4 *>(gw + (lane & 15) * 32 + i0);
            const uint4 xv4 = *reinterpret_cast<const uint4 *>(gx + tok * 32 + i0);
            const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w}, xw[4] = {xv4.x, xv4.y, xv4.z, xv4.w};
            v8h a, b;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const uint16_t w = (uint16_t)(ww[e >> 1] >> (16 * (e & 1)));
                if constexpr (F16W)
                    a[e] = __builtin_bit_cast(_Float16, w);
                else
                    a[e] = (_Float16)(float)(int8_t)(w & 0xffu);
                b[e] = __builtin_bit_cast(_Float16, (uint16_t)(xw[e >> 1] >> (16 * (e & 1))));
            }
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, d, 0, 0, 0);
        }
        for (int c = 1; c < (nO + 31) / 32; c++) {
            const int i0 = 32 * c + 8 * kg;
            int wr[8];
            uint32_t xr[8];
            gather_raw(rgc, i0, wr, xr);
            v8h a, b;
            fragments(i0, wr, xr, a, b);
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
    };

    if constexpr (MW == 8) {   // wave 0: the epilogue of every row group
        if (wid != 0)
            return;
        for (int i = 0; i < nG; i++)
            process(0, rg + i * G, i & 1, true);
        return;
    }
    // One row group per workgroup (N <= 16 x grid): no next group to load.
    if (NRG <= G) {
        process(0, rg, 0, FUSED);
        return;
    }
    // Else two row groups per iteration, so that the register set holding
    // the next group's weights is fixed at compile time; the next group's
    // loads are issued before this group's MFMAs
    bool first = FUSED;   // (its gathers made during the activation work)
    while (rg < NRG) {
        const int rg1 = rg + G;
        wload(1, rg1);   // zeros past the last group
        process(0, rg, 0, first);
        first = false;
        if (rg1 >= NRG)
            break;
        const int rg2 = rg1 + G;
        wload(0, rg2);
        process(1, rg1, 1, false);
        rg = rg2;
    }
}

template <bool FUSED, int KB, int TB, bool F16W, int MW>
hipError_t launch_roles(const uint16_t *X, const int8_t *Wq, const float *sW, const uint16_t *W16,
                        uint32_t thr_mag,
                        int64_t T, int64_t K, int64_t N, uint16_t *Y, int32_t *acc, const char *ws,
                        const WsLayout &L, hipStream_t s)
{
    const int nrg = (int)((N + kDRows - 1) / kDRows);
    const dim3 grid((unsigned)(nrg < kDecodeMaxBlocks ? nrg : kDecodeMaxBlocks));
    const dim3 block(kDThreads + 64 * MW);
    const int32_t *meta = FUSED ? nullptr : reinterpret_cast<const int32_t *>(ws + L.meta);
    const int32_t *idx = FUSED ? nullptr : reinterpret_cast<const int32_t *>(ws + L.idx);
    const float *sX = FUSED ? nullptr : reinterpret_cast<const float *>(ws + L.sX);
    const int8_t *Xq = FUSED ? nullptr : reinterpret_cast<const int8_t *>(ws + L.Xq);
    const uint16_t *XO = FUSED ? nullptr : reinterpret_cast<const uint16_t *>(ws + L.XO);
    if (acc)
        hipLaunchKernelGGL((k_decode<FUSED, KB, TB, F16W, true, MW>), grid, block, 0, s, X, Wq,
                           sW, W16, thr_mag, (int)T, (int)K, (int)N, meta, idx, sX, Xq, XO, Y, acc);
    else
        hipLaunchKernelGGL((k_decode<FUSED, KB, TB, F16W, false, MW>), grid, block, 0, s, X, Wq,
                           sW, W16, thr_mag, (int)T, (int)K, (int)N, meta, idx, sX, Xq, XO, Y, acc);
    return hipGetLastError();
}

// The MFMA-wave variants where they apply: the fused kernel with K <= 4096,
// MW = 4 with one row group per workgroup, MW = 8 with more row groups than
// workgroups and T <= 8.  (MW = 8 at one row group per workgroup measured
// slower than MW = 4: 6.9 against 5.8 us at 8x4096x4096.)
template <bool FUSED, int KB, int TB, bool F16W>
hipError_t launch_kb(const uint16_t *X, const int8_t *Wq, const float *sW, const uint16_t *W16,
                     uint32_t thr_mag,
                     int64_t T, int64_t K, int64_t N, uint16_t *Y, int32_t *acc, const char *ws,
                     const WsLayout &L, hipStream_t s)
{
    if constexpr (FUSED && KB == 8) {
        if ((N + kDRows - 1) / kDRows <= kDecodeMaxBlocks)
            return launch_roles<FUSED, KB, TB, F16W, 4>(X, Wq, sW, W16, thr_mag, T, K, N, Y, acc,
                                                        ws, L, s);
        if constexpr (TB == 8)
            return launch_roles<FUSED, KB, TB, F16W, 8>(X, Wq, sW, W16, thr_mag, T, K, N, Y, acc,
                                                        ws, L, s);
    }
    return launch_roles<FUSED, KB, TB, F16W, 0>(X, Wq, sW, W16, thr_mag, T, K, N, Y, acc, ws,
                                                L, s);
}

} // namespace

bool decode_shape(int64_t T, int64_t K)
{
    return T >= 1 && T <= kDecodeMaxT && K >= 16 && K <= kDecodeMaxK;
}

// KB (weight 16-byte loads per lane and row group) by K, TB by T.
template <bool FUSED, bool F16W>
hipError_t launch_decode(const uint16_t *X, const int8_t *Wq, const float *sW, const uint16_t *W16,
                         uint32_t thr_mag, int64_t T, int64_t K, int64_t N, uint16_t *Y,
                         int32_t *acc, const char *ws, const WsLayout &L, hipStream_t s)
{
    if (K <= 4096)
        return T <= 8 ? launch_kb<FUSED, 8, 8, F16W>(X, Wq, sW, W16, thr_mag, T, K, N, Y, acc, ws, L, s)
                      : launch_kb<FUSED, 8, 16, F16W>(X, Wq, sW, W16, thr_mag, T, K, N, Y, acc, ws, L, s);
    return T <= 8 ? launch_kb<FUSED, 16, 8, F16W>(X, Wq, sW, W16, thr_mag, T, K, N, Y, acc, ws, L, s)
                  : launch_kb<FUSED, 16, 16, F16W>(X, Wq, sW, W16, thr_mag, T, K, N, Y, acc, ws, L, s);
}

hipError_t launch_decode_fused(const uint16_t *X, const int8_t *Wq, const float *sW,
                               const uint16_t *W16, uint16_t thr_mag, int64_t T, int64_t K,
                               int64_t N, uint16_t *Y, hipStream_t s)
{
    static const WsLayout none{};
    if (W16)
        return launch_decode<true, true>(X, Wq, sW, W16, thr_mag, T, K, N, Y, nullptr, nullptr, none, s);
    return launch_decode<true, false>(X, Wq, sW, nullptr, thr_mag, T, K, N, Y, nullptr, nullptr, none, s);
}

hipError_t launch_decode_gemm(const int8_t *Wq, const float *sW, const uint16_t *W16, int64_t T,
                              int64_t K, int64_t N, uint16_t *Y, int32_t *acc, const char *ws,
                              const WsLayout &L, hipStream_t s)
{
    if (W16)
        return launch_decode<false, true>(nullptr, Wq, sW, W16, 0, T, K, N, Y, acc, ws, L, s);
    return launch_decode<false, false>(nullptr, Wq, sW, nullptr, 0, T, K, N, Y, acc, ws, L, s);
}

} // namespace li8
