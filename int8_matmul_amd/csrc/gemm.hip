// int8 x int8 -> int32 GEMM with the LLM.int8() epilogue, for gfx950.
//
//   acc[t,n] = sum_j Xq[t,j] * Wq[n,j]                      (exact, int32)
//   D[t,n]   = fl32(acc * sX[t])
//   D       += sum_{i < nO} XO[t,i] * WO[n,i]               (fp16 MFMA, fp32)
//   Y[t,n]   = fp16(fl32(D * sW[n]))
//
// XO / WO are the outlier columns of X (fp16) and of Wq (int8 codes, exact
// in fp16) gathered into compact matrices by the prepare kernel.  Adding
// the raw outlier product to acc*sX before the per-channel scale sW is the
// same sum as  acc*sX*sW + sum X * (Wq*sW)  (the pages' decomposition:
// hncyxsy.com/news/230290, section 2.1 - the int8 product of the normal
// columns and the fp16 product of the outlier columns, added in the fp16
// domain), up to fp32 rounding; with no outlier columns it is exactly
// fp16(fl32(fl32(acc * sX) * sW)).
//
// Structure (both operands K-contiguous, "NT"):
//  - BM x BN output tile per workgroup of WM x WN waves; each wave owns an
//    (FM*32) x (FN*32) sub-tile computed with v_mfma_i32_32x32x32_i8.
//  - K is consumed in stages of BKS bytes held in a ring of NS LDS buffers,
//    filled by buffer_load ... lds (global -> LDS without VGPRs).  A stage
//    is requested NS stages ahead.  A lane whose 16-byte chunk lies past K
//    gets an out-of-range buffer offset, for which the hardware returns
//    zeros, so a ragged K needs no branch.
//  - MFMA fragments are double-buffered in registers: the LDS reads of
//    k-step s+1 are interleaved one-to-one with the MFMAs of k-step s.  The one barrier
//    per stage sits before the MFMAs of the stage's last k-step, after all
//    reads of the stage were issued, so the MFMA pipe has queued work when
//    a wave reaches it.
//  - 16-byte chunks are XOR-swizzled per row in LDS so that fragment reads
//    (32 rows x 16 bytes per half-wave) hit distinct banks.
//  - Workgroups are renumbered so that each XCD (the hardware deals
//    workgroups to the 8 XCDs round-robin) gets a contiguous run of tiles,
//    and tiles are ordered in groups of GM row-tiles, so that the tiles
//    running together on one XCD share operand rows in its L2.
//  - Epilogue: per 32x32 block, dequantize, add the outlier MFMA, scale,
//    convert to fp16 into LDS; then each wave writes its sub-tile with
//    16-byte stores.
#include <type_traits>
#include <utility>

#include "li8_internal.h"
#include "quant_math.h"

namespace li8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
#define LI8_LDS __attribute__((address_space(3)))

// Buffer resource over `bytes` bytes at p (raw buffer, offsets in bytes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, 0x00020000);
}

// 16 bytes per lane from rsrc at voffset + soffset into LDS at lds + 16*lane.
__device__ __forceinline__ void load_to_lds(__amdgpu_buffer_rsrc_t r, void *lds, int voffset,
                                            int soffset)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LI8_LDS void *)lds, 16, voffset, soffset, 0, 0);
}

// B (4 or 16) bytes per lane from rsrc at voffset into LDS at lds + B*lane.
// (Called from a device function: the builtin written inside a kernel's
// lambda makes the host pass drop the kernel's launch stub.)
template <int B>
__device__ __forceinline__ void load_to_lds_n(__amdgpu_buffer_rsrc_t r, void *lds, int voffset)
{
    static_assert(B == 4 || B == 16, "bytes per lane");
    if constexpr (B == 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LI8_LDS void *)lds, 4, voffset, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LI8_LDS void *)lds, 16, voffset, 0, 0, 0);
}

template <int CPR>
__device__ __forceinline__ int swz(int row)
{
    static_assert(CPR == 4 || CPR == 8, "16-byte chunks per LDS row");
    if constexpr (CPR == 8)
        return (row ^ (row >> 3)) & 7;
    else
        return ((row >> 1) ^ (row >> 3)) & 3;
}

// Wait until at most N buffer loads of this wave are in flight and all its
// LDS reads are done, then barrier.  The compiler does not track the LDS
// writes of buffer_load ... lds, so this wait is what orders them.
template <int N>
__device__ __forceinline__ void wait_loads_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

constexpr int kOutOfRange = (int)0x80000000;   // buffer offset past any operand

// f(integral_constant<int, I>) for each I of the sequence, in order.
template <int... I, class F>
__device__ __forceinline__ void for_each_index(std::integer_sequence<int, I...>, F &&f)
{
    (f(std::integral_constant<int, I>{}), ...);
}

template <int BM, int BN, int BKS, int NS, int WM, int WN, int GM, bool F16W, bool STORE_ACC>
__global__ __launch_bounds__(WM *WN * 64) void k_gemm(
    const int8_t *__restrict__ Xq, const int8_t *__restrict__ Wq,
    const float *__restrict__ sX, const float *__restrict__ sW,
    const int32_t *__restrict__ meta, const uint16_t *__restrict__ XO,
    const int8_t *__restrict__ WO, const int32_t *__restrict__ idx_g,
    const int32_t *__restrict__ wpre_g, int T, int K, int N, int tiles_m, int tiles_n,
    uint16_t *__restrict__ Y, int32_t *__restrict__ acc_out)
{
    constexpr int NT = WM * WN * 64, NW = WM * WN;
    constexpr int FM = BM / (WM * 32);
    constexpr int FN = BN / (WN * 32);
    constexpr int CPR = BKS / 16;              // 16-byte chunks per LDS row
    constexpr int KS = BKS / 32;               // MFMA k-steps per stage
    constexpr int ASZ = BM * BKS, SSZ = (BM + BN) * BKS;
    constexpr int LA = BM * CPR / NT, LB = BN * CPR / NT;   // loads per lane per stage
    constexpr int RS = FN * 32 + 8;            // epilogue staging row stride (halves)
    constexpr int STG = NW * (FM * 32) * RS * 2;
    // Epilogue operands prefetched into LDS at entry, past the ring: token
    // scales, feature scales and the first 16-column chunk of XO and WO.
    // The staging rows may overlap them; the staging barrier orders that.
    constexpr int WOE = F16W ? 2 : 1;          // bytes per WO element
    // Fold (int8 path, kFoldMin < nO <= CAP, K <= kFoldMaxK): the tile's
    // outlier weight columns are copied out of each K stage of the weight
    // while it sits in LDS, into WOT in the WO chunk layout (rank r of row
    // n at (r/16)*BN*16 + n*16 + r%16), so the prepare kernel need not
    // gather them from Wq, a second read of the weight when the outlier
    // columns are spread over K.  It needs the outlier list and the prefix
    // counts per bit-set word (stage s starts at word 4s).
    constexpr int CAP = (F16W || BN > 128) ? 0 : 256;
    constexpr int NWMAX = kFoldMaxK / 32;      // bit-set words
    constexpr int PF_SX = NS * SSZ, PF_SW = PF_SX + 4 * BM, PF_XO = PF_SW + 4 * BN;
    constexpr int PF_WO = PF_XO + 32 * BM;     // chunk 0 of the gathered WO, or WOT when folding
    constexpr int WO_B = (16 * WOE * BN > BN * CAP) ? 16 * WOE * BN : BN * CAP;
    constexpr int PF_IDX = PF_WO + WO_B, PF_WPRE = PF_IDX + 4 * CAP;
    constexpr int PF_DUMMY = PF_WPRE + (CAP > 0 ? 4 * (NWMAX + 1) : 0);
    constexpr int PF_END = PF_DUMMY + (CAP > 0 ? NT : 0);
    constexpr int LDSB = (PF_END > STG) ? PF_END : STG;
    static_assert(FM * WM * 32 == BM && FN * WN * 32 == BN, "tile shape");
    static_assert(LA * NT == BM * CPR && LB * NT == BN * CPR, "loader shape");
    static_assert(KS % 2 == 0 && NS >= 2 && BKS == 32 * KS, "pipeline shape");
    __shared__ __attribute__((aligned(1024))) int8_t lds[LDSB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid / WN, wn = wid % WN;

    // ---- tile of this workgroup ----
    int bid = blockIdx.x;
    {
        const int nblk = tiles_m * tiles_n;
        const int per = nblk / 8, rem = nblk % 8, xcd = bid % 8, loc = bid / 8;
        bid = (xcd < rem) ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
    }
    const int width = GM * tiles_n;
    const int first_m = (bid / width) * GM;
    const int gm = min(tiles_m - first_m, GM);
    const int tile_m = first_m + (bid % width) % gm;
    const int tile_n = (bid % width) / gm;
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    // have every kernel argument the epilogue uses in registers before the
    // main loop: a scalar load in flight across it would make the compiler
    // wait for all LDS reads instead of the older half
    asm volatile("" ::"s"(sX), "s"(sW), "s"(XO), "s"(WO), "s"(Y), "s"(acc_out));
    const int nO = min(max(meta[0], 0), K);   // (a bad workspace cannot lengthen the loop)
    asm volatile("" ::"s"(nO));
    const int nk = (K + BKS - 1) / BKS;
    const bool fold = CAP > 0 && nO > kFoldMin && nO <= CAP && K <= kFoldMaxK;   // (uniform)

    // ---- global -> LDS loaders: load i of this lane fills LDS chunk
    // p = i*NT + wid*64 + lane of the stage (row p / CPR, physical chunk
    // p % CPR), which holds logical chunk (p % CPR) ^ swz(row) ----
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(Xq, T * K);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(Wq, N * K);
    int voA[LA], voB[LB], kmA[LA], kmB[LB];
#pragma unroll
    for (int i = 0; i < LA; i++) {
        const int p = i * NT + wid * 64 + lane, row = p / CPR, q = (p % CPR) ^ swz<CPR>(row);
        voA[i] = min(m0 + row, T - 1) * K + q * 16;
        kmA[i] = K - q * 16;   // the chunk is inside the row while k0 < kmA
    }
#pragma unroll
    for (int i = 0; i < LB; i++) {
        const int p = i * NT + wid * 64 + lane, row = p / CPR, q = (p % CPR) ^ swz<CPR>(row);
        voB[i] = min(n0 + row, N - 1) * K + q * 16;
        kmB[i] = K - q * 16;
    }
    auto issue = [&](int kt) {
        const int k0 = kt * BKS;
        int8_t *st = lds + (kt % NS) * SSZ;
#pragma unroll
        for (int i = 0; i < LA; i++)
            load_to_lds(rA, st + (i * NT + wid * 64) * 16, (k0 < kmA[i]) ? voA[i] : kOutOfRange, k0);
#pragma unroll
        for (int i = 0; i < LB; i++)
            load_to_lds(rB, st + ASZ + (i * NT + wid * 64) * 16, (k0 < kmB[i]) ? voB[i] : kOutOfRange,
                        k0);
    };

    // ---- MFMA fragments: lane l supplies row (l & 31) of each 32-row
    // block and the 16 bytes of chunk 2*kk + (l >> 5) of k-step kk ----
    const int arow0 = wm * FM * 32 + (lane & 31);
    const int brow0 = wn * FN * 32 + (lane & 31);
    const int khalf = lane >> 5;
    int offA[FM][KS], offB[FN][KS];
#pragma unroll
    for (int kk = 0; kk < KS; kk++) {
        const int q = kk * 2 + khalf;
#pragma unroll
        for (int a = 0; a < FM; a++) {
            const int row = arow0 + a * 32;
            offA[a][kk] = row * BKS + ((q ^ swz<CPR>(row)) * 16);
        }
#pragma unroll
        for (int b = 0; b < FN; b++) {
            const int row = brow0 + b * 32;
            offB[b][kk] = ASZ + row * BKS + ((q ^ swz<CPR>(row)) * 16);
        }
    }

    v16i acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; a++)
#pragma unroll
        for (int b = 0; b < FN; b++)
            acc[a][b] = v16i{};

    v4i fa[2][FM], fb[2][FN];
    auto lread = [&](int set, int kt, int kk) {
        const int8_t *base = lds + (kt % NS) * SSZ;
#pragma unroll
        for (int a = 0; a < FM; a++)
            fa[set][a] = *reinterpret_cast<const v4i *>(base + offA[a][kk]);
#pragma unroll
        for (int b = 0; b < FN; b++)
            fb[set][b] = *reinterpret_cast<const v4i *>(base + offB[b][kk]);
    };
    // weight fragment first: acc[a][b] is the transposed block (features x
    // tokens), which puts four consecutive output features in each group of
    // four accumulator registers
    auto mfmas = [&](int set) {
#pragma unroll
        for (int a = 0; a < FM; a++)
#pragma unroll
            for (int b = 0; b < FN; b++)
                acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[set][b], fa[set][a], acc[a][b],
                                                                 0, 0, 0);
    };
    // One stage.  WAIT: buffer loads allowed in flight at the barrier;
    // ISSUE: request stage kt+NS into the buffer just released; LAST: no
    // next stage.
    // Fold: copy stage kt's outlier columns (landed, in its ring buffer)
    // into WOT.  Each thread reads one (rank, row) item right after the
    // barrier that made the stage visible, when this wave has no LDS read
    // in flight, and writes it after the MFMAs of that k-step have issued,
    // so that the MFMAs do not wait behind the read's latency.  The read and
    // the write are issued whether or not the item exists (an absent item
    // re-reads a valid byte and stores to a dummy byte of its own), so the
    // LDS operations in flight stay countable; a stage with more than NT
    // items copies the rest in a loop.  (Measured against four items per
    // thread read and written at once: 13B FFN 69.3 -> 62.9 us per call;
    // 4096 x 4096 x 11008 with 29 outlier columns 209.9 -> 204.6 us.  Two
    // or four items per thread with the split were slower on 256-wide
    // tiles, whose registers are nearly all taken.)
    const int32_t *idx_l = reinterpret_cast<const int32_t *>(lds + PF_IDX);
    const int32_t *wpre_l = reinterpret_cast<const int32_t *>(lds + PF_WPRE);
    int8_t *wot = lds + PF_WO;
    const int nwords = (K + 31) / 32;
    int8_t xv = 0;          // the item read
    int xlo = 0, xn = 0;    // first rank and item count of the stage read
    auto extract_read = [&](int kt) {
        const int lo = __builtin_amdgcn_readfirstlane(wpre_l[min(KS * kt, nwords)]);
        const int hi = __builtin_amdgcn_readfirstlane(wpre_l[min(KS * kt + KS, nwords)]);
        const int n = (hi - lo) * BN;
        const int8_t *bst = lds + (kt % NS) * SSZ + ASZ;
        const int it = min(tid, max(n - 1, 0));
        const int rr = it / BN, row = it - rr * BN;
        const int c = min(max(idx_l[min(lo + rr, CAP - 1)] - kt * BKS, 0), BKS - 1);
        xv = bst[row * BKS + (((c >> 4) ^ swz<CPR>(row)) << 4) + (c & 15)];
        xlo = lo;
        xn = n;
    };
    auto extract_write = [&](int kt) {
        {
            const int it = min(tid, max(xn - 1, 0));
            const int rr = it / BN, row = it - rr * BN, r = min(xlo + rr, CAP - 1);
            int8_t *dst = tid < xn ? wot + (r >> 4) * (BN * 16) + row * 16 + (r & 15) : lds + PF_DUMMY + tid;
            *dst = xv;
        }
        if (xn > NT) {   // more than NT / BN outlier columns in this stage
            const int8_t *bst = lds + (kt % NS) * SSZ + ASZ;
            for (int it = NT + tid; it < xn; it += NT) {
                const int rr = it / BN, row = it - rr * BN, r = xlo + rr;
                const int c = idx_l[r] - kt * BKS;
                wot[(r >> 4) * (BN * 16) + row * 16 + (r & 15)] =
                    bst[row * BKS + (((c >> 4) ^ swz<CPR>(row)) << 4) + (c & 15)];
            }
        }
    };
    auto stage = [&](int kt, auto wait_c, auto issue_c, auto last_c, auto fold_c) {
        constexpr int WAIT = decltype(wait_c)::value;
        constexpr bool ISSUE = decltype(issue_c)::value;
        constexpr bool LAST = decltype(last_c)::value;
        constexpr bool FOLD = decltype(fold_c)::value;
        // k-step kk (a compile-time constant: the fold's loop must not stop
        // the unrolling)
        auto kstep = [&](auto kk_c) {
            constexpr int kk = decltype(kk_c)::value;
            constexpr int cur = kk & 1;
            // Each fragment read of the next k-step is paired with one MFMA
            // of this one, so that the reads do not arrive in a burst that
            // the other wave on the SIMD must wait behind.  (The global ->
            // LDS loads of the last k-step stay grouped: each needs its own
            // M0 value, and the scheduler keeps them together.)
            constexpr int NMF = FM * FN, NRD = FM + FN;
            if constexpr (kk + 1 < KS) {
                __builtin_amdgcn_sched_barrier(0);
                lread(cur ^ 1, kt, kk + 1);
                mfmas(cur);
#pragma unroll
                for (int i = 0; i < NMF; i++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (i < NRD)
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            } else if constexpr (!LAST) {
                wait_loads_barrier<WAIT>();   // stage kt+1 landed; stage kt read by all
                if constexpr (FOLD) {   // stage kt+1 landed: read its outlier columns
                    extract_read(kt + 1);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if constexpr (ISSUE)
                    issue(kt + NS);
                lread(cur ^ 1, kt + 1, 0);
                mfmas(cur);
                constexpr int NLD = ISSUE ? LA + LB : 0;
#pragma unroll
                for (int i = 0; i < NMF; i++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (i < NRD)
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    if (i < NLD)
                        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (FOLD) {   // and write them, behind the MFMAs
                    extract_write(kt + 1);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                __builtin_amdgcn_sched_barrier(0);
                mfmas(cur);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        for_each_index(std::make_integer_sequence<int, KS>{}, kstep);
    };
    using TF = std::false_type;
    using TT = std::true_type;
    using W0 = std::integral_constant<int, 0>;
    using WS = std::integral_constant<int, (LA + LB) * (NS - 2)>;

    // epilogue prefetch, issued ahead of the first stages: loads complete in
    // order, so once all but the last LA+LB loads of a lane are done, stage
    // 0 and the prefetch have landed while stage 1 may still be in flight;
    // rows past T or N read zeros or clamp, and are never stored
    const __amdgpu_buffer_rsrc_t rXO = make_rsrc(XO, (int)(2u * (unsigned)T * (unsigned)K));
    const __amdgpu_buffer_rsrc_t rWO = make_rsrc(WO, (int)((unsigned)WOE * (unsigned)N * (unsigned)K));
    {
        auto prefetch = [&](__amdgpu_buffer_rsrc_t r, int off, auto bytes_c, int n, auto voff) {
            constexpr int B = decltype(bytes_c)::value;   // bytes per lane
#pragma unroll
            for (int j0 = wid * 64; j0 < n; j0 += NT) {
                const int c = j0 + lane;
                if (c < n)
                    load_to_lds_n<B>(r, lds + off + j0 * B, voff(c));
            }
        };
        using B4 = std::integral_constant<int, 4>;
        using B16 = std::integral_constant<int, 16>;
        const int sxb = T < (1 << 29) ? 4 * T : 0x7fffffff;
        const int swb = N < (1 << 29) ? 4 * N : 0x7fffffff;
        prefetch(make_rsrc(sX, sxb), PF_SX, B4{}, BM,
                 [&](int c) { return (int)(4u * (unsigned)(m0 + c)); });
        prefetch(make_rsrc(sW, swb), PF_SW, B4{}, BN,
                 [&](int c) { return (int)(4u * (unsigned)(n0 + c)); });
        if (nO > 0) {   // then K >= 16: chunk 0 lies inside every row
            prefetch(rXO, PF_XO, B16{}, 2 * BM, [&](int c) {
                return (int)((unsigned)min(m0 + (c >> 1), T - 1) * 32u + 16u * (c & 1));
            });
        }
        if (fold) {   // the outlier list and the word prefix counts (zeros past their ends)
            const int nw = (K + 31) / 32;
            prefetch(make_rsrc(idx_g, 4 * K), PF_IDX, B4{}, CAP, [&](int c) { return 4 * c; });
            prefetch(make_rsrc(wpre_g, 4 * (nw + 1)), PF_WPRE, B4{}, NWMAX + 1, [&](int c) { return 4 * c; });
        }
        else if (nO > 0) {   // chunk 0 of the gathered WO
            if constexpr (F16W)
                prefetch(rWO, PF_WO, B16{}, 2 * BN, [&](int c) {
                    return (int)((unsigned)min(n0 + (c >> 1), N - 1) * 32u + 16u * (c & 1));
                });
            else
                prefetch(rWO, PF_WO, B16{}, BN,
                         [&](int c) { return (int)((unsigned)min(n0 + c, N - 1) * 16u); });
        }
    }
#pragma unroll
    for (int s = 0; s < NS; s++)
        if (s < nk)
            issue(s);
    if (nk >= NS) {
        wait_loads_barrier<(NS - 1) * (LA + LB)>();   // stage 0 landed
        lread(0, 0, 0);
    } else if (nk > 0) {
        wait_loads_barrier<0>();
        lread(0, 0, 0);
    }

    // the main loop, in a second copy with the fold's copies when this
    // call folds (the other copy is the plain loop)
    auto main_loop = [&](auto fold_c) {
        if constexpr (decltype(fold_c)::value) {   // stage 0 landed at the prologue's barrier
            extract_read(0);
            extract_write(0);
        }
        int kt = 0;
        for (; kt + NS < nk; kt++)      // steady state
            stage(kt, WS{}, TT{}, TF{}, fold_c);
        for (; kt + 1 < nk; kt++)       // drain
            stage(kt, W0{}, TF{}, TF{}, fold_c);
        if (kt < nk)
            stage(kt, W0{}, TF{}, TT{}, fold_c);
    };
    if (fold)
        main_loop(TT{});
    else
        main_loop(TF{});

    // ---- epilogue ----
    // acc[a][b], lane l, register r: token t = tok0 + 32a + (l & 31), feature
    // n = fea0 + 32b + 8*(r/4) + (r%4), with tok0 / fea0 the first token and
    // (for this half-wave) feature of the wave's sub-tile.
    const int tok0 = m0 + wm * FM * 32 + (lane & 31);
    const int fea0 = n0 + wn * FN * 32 + 4 * khalf;
    if constexpr (STORE_ACC) {
#pragma unroll
        for (int a = 0; a < FM; a++)
#pragma unroll
            for (int b = 0; b < FN; b++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int t = tok0 + 32 * a, n = fea0 + 32 * b + 8 * (r >> 2) + (r & 3);
                    if (t < T && n < N)
                        acc_out[(int64_t)t * N + n] = acc[a][b][r];
                }
    }
    if (nk == 0 || fold)   // prefetched operands landed; fold: every wave's WOT copies done
        wait_loads_barrier<0>();
    // token scales from the prefetch
    const int ltok = wm * FM * 32 + (lane & 31);                 // local token row
    const int lfea = wn * FN * 32 + (lane & 31);                 // local weight row
    float sx[FM];
#pragma unroll
    for (int a = 0; a < FM; a++)
        sx[a] = *reinterpret_cast<const float *>(lds + PF_SX + 4 * (ltok + 32 * a));
    // outlier operands, chunk c: lane l supplies 8 of the 16 columns
    // (8*(l/32)..) of the weight row of block b and the token row of block
    // a; buffer loads with a fixed per-lane offset and the chunk's offset
    // in the scalar operand
    // (WO: int8 codes [N,K], or in the fp16-weight variant fp16 [N,K])
    const int nch = (nO + 15) >> 4;
    int voX[FM], voW[FN];
#pragma unroll
    for (int a = 0; a < FM; a++)
        voX[a] = (int)((unsigned)min(tok0 + 32 * a, T - 1) * 32u + khalf * 16u);
#pragma unroll
    for (int b = 0; b < FN; b++)
        voW[b] = (int)((unsigned)min(n0 + wn * FN * 32 + 32 * b + (lane & 31), N - 1) * 16u * WOE +
                       khalf * 8 * WOE);
    // chunk c of the outlier operands starts at c * cXO bytes of XO and c * cWO of WO
    const unsigned cXO = 32u * (unsigned)T, cWO = 16u * WOE * (unsigned)N;
    v8h ox[2][FM];
    v2u ow[2][FN];     // int8 codes
    v8h ow16[2][FN];   // fp16 weight (the fp16-weight variant)
    auto oload = [&](int set, int c) {
#pragma unroll
        for (int a = 0; a < FM; a++)
            ox[set][a] = __builtin_bit_cast(v8h, __builtin_amdgcn_raw_buffer_load_b128(rXO, voX[a], (int)(cXO * (unsigned)c), 0));
        if constexpr (F16W) {
#pragma unroll
            for (int b = 0; b < FN; b++)
                ow16[set][b] =
                    __builtin_bit_cast(v8h, __builtin_amdgcn_raw_buffer_load_b128(rWO, voW[b], (int)(cWO * (unsigned)c), 0));
        } else if (fold) {   // the tile's copy in LDS (ranks past nO: stale codes times XO's zero pad)
#pragma unroll
            for (int b = 0; b < FN; b++)
                ow[set][b] = *reinterpret_cast<const v2u *>(wot + c * (BN * 16) + (lfea + 32 * b) * 16 + khalf * 8);
        } else {
#pragma unroll
            for (int b = 0; b < FN; b++)
                ow[set][b] = __builtin_amdgcn_raw_buffer_load_b64(rWO, voW[b], (int)(cWO * (unsigned)c), 0);
        }
    };
    // chunk 0 from the prefetch
    auto oload0 = [&]() {
#pragma unroll
        for (int a = 0; a < FM; a++)
            ox[0][a] = *reinterpret_cast<const v8h *>(lds + PF_XO + (ltok + 32 * a) * 32 + khalf * 16);
#pragma unroll
        for (int b = 0; b < FN; b++) {
            if constexpr (F16W)
                ow16[0][b] = *reinterpret_cast<const v8h *>(lds + PF_WO + (lfea + 32 * b) * 32 + khalf * 16);
            else
                ow[0][b] = *reinterpret_cast<const v2u *>(lds + PF_WO + (lfea + 32 * b) * 16 + khalf * 8);
        }
    };
    if (nch > 0)
        oload0();   // (when folding, PF_WO holds WOT, whose chunk 0 has the same layout)

    // feature scales, four consecutive per float4
    float4 sw[FN][4];
    auto load_sw = [&]() {   // from the prefetch (fea0 - n0 is a multiple of 4)
#pragma unroll
        for (int b = 0; b < FN; b++)
#pragma unroll
            for (int g = 0; g < 4; g++)
                sw[b][g] = *reinterpret_cast<const float4 *>(lds + PF_SW + 4 * (fea0 - n0 + 32 * b + 8 * g));
    };
    // D = fl32(acc * sX); in the fp16-weight variant D = fl32(D * sW) here,
    // before the outlier product (which is then in output units)
    v16f d[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; a++)
#pragma unroll
        for (int b = 0; b < FN; b++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                d[a][b][r] = (float)acc[a][b][r] * sx[a];
    if constexpr (F16W) {
        load_sw();
#pragma unroll
        for (int a = 0; a < FM; a++)
#pragma unroll
            for (int b = 0; b < FN; b++)
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    d[a][b][4 * g] *= sw[b][g].x;
                    d[a][b][4 * g + 1] *= sw[b][g].y;
                    d[a][b][4 * g + 2] *= sw[b][g].z;
                    d[a][b][4 * g + 3] *= sw[b][g].w;
                }
    }
    // D += XO . WO^T over the outlier columns (codes are exact in fp16),
    // the next chunk's loads in flight during this chunk's MFMAs
    // `keep` is all ones, or zero for a chunk past the end (its codes are
    // then masked to 0): the MFMAs run unconditionally so that the loads
    // stay where they were issued, ahead of their use
    auto omfma = [&](int set, uint32_t keep) {
        v8h wb[FN];
#pragma unroll
        for (int b = 0; b < FN; b++) {
            if constexpr (F16W) {
                v4i w = __builtin_bit_cast(v4i, ow16[set][b]);
                w &= (int)keep;
                wb[b] = __builtin_bit_cast(v8h, w);
            } else {
                const uint32_t w[2] = {ow[set][b][0] & keep, ow[set][b][1] & keep};
#pragma unroll
                for (int e = 0; e < 8; e++)
                    wb[b][e] = (_Float16)(float)(int8_t)((w[e >> 2] >> (8 * (e & 3))) & 0xffu);
            }
        }
#pragma unroll
        for (int a = 0; a < FM; a++)
#pragma unroll
            for (int b = 0; b < FN; b++)
                d[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wb[b], ox[set][a], d[a][b], 0, 0, 0);
    };
    // chunk 0 (from the prefetch), then two chunks per iteration with both
    // loads in flight together; a chunk index past the end re-reads the
    // last chunk (a valid address) and is masked.  The scheduling barriers
    // keep the compiler from moving the loads down next to their use.
    if (nch > 0)
        omfma(0, ~0u);
    for (int c = 1; c < nch; c += 2) {
        oload(1, c);
        oload(0, min(c + 1, nch - 1));
        __builtin_amdgcn_sched_barrier(0);
        omfma(1, ~0u);
        omfma(0, (c + 1 < nch) ? ~0u : 0u);
        __builtin_amdgcn_sched_barrier(0);
    }

    if constexpr (!F16W)
        load_sw();
    // Y = fp16(fl32(D * sW)), four consecutive features per 8-byte LDS write
    // into the wave's staging rows (one row per token).  The ring buffers
    // are reused for the staging: every wave must be done reading them.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    uint16_t *stg = reinterpret_cast<uint16_t *>(lds) + wid * (FM * 32) * RS;
#pragma unroll
    for (int a = 0; a < FM; a++)
#pragma unroll
        for (int b = 0; b < FN; b++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const float s4[4] = {sw[b][g].x, sw[b][g].y, sw[b][g].z, sw[b][g].w};
                float p[4];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    // fl32(D * sW) first, then one rounding to fp16: the
                    // empty asm keeps the compiler from fusing the product
                    // and the conversion into a single-rounding
                    // v_fma_mixlo_f16
                    p[j] = d[a][b][4 * g + j];
                    if constexpr (!F16W)
                        p[j] *= s4[j];
                    asm("" : "+v"(p[j]));
                }
                *reinterpret_cast<uint2 *>(stg + (a * 32 + (lane & 31)) * RS + b * 32 + 8 * g +
                                           4 * khalf) = make_uint2(pack_f16x2(p[0], p[1]), pack_f16x2(p[2], p[3]));
            }
    // each wave stores its own sub-tile (only its own LDS rows: no barrier).
    // Non-temporal stores: Y is not read again by this kernel, and output
    // left dirty in the L2 is written back when the kernel ends, which the
    // next kernel waits for (the 13B call: 77 -> 73 us)
    constexpr int CPRW = FN * 32 / 8;   // 16-byte chunks per sub-tile row
    constexpr int NCH = FM * 32 * CPRW;
    const int rbase = m0 + wm * FM * 32, cbase = n0 + wn * FN * 32;
    if ((N & 7) == 0) {
#pragma unroll
        for (int i = 0; i < NCH / 64; i++) {
            const int id = i * 64 + lane, row = id / CPRW, ch = id % CPRW;
            const v4i v = *reinterpret_cast<const v4i *>(stg + row * RS + ch * 8);
            const int grow = rbase + row, gcol = cbase + ch * 8;
            if (grow < T && gcol < N)
                __builtin_nontemporal_store(v, reinterpret_cast<v4i *>(Y + (int64_t)grow * N + gcol));
        }
    } else {   // rows not 16-byte aligned: element stores
        for (int i = 0; i < NCH / 64; i++) {
            const int id = i * 64 + lane, row = id / CPRW, ch = id % CPRW;
            const int grow = rbase + row;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const int gcol = cbase + ch * 8 + e;
                if (grow < T && gcol < N)
                    Y[(int64_t)grow * N + gcol] = stg[row * RS + ch * 8 + e];
            }
        }
    }
}

template <int BM, int BN, int BKS, int NS, int WM, int WN, int GM, bool F16W>
hipError_t launch_cfg(const int8_t *Wq, const float *sW, int64_t T, int64_t K, int64_t N,
                      uint16_t *Y, int32_t *acc, const char *ws, const WsLayout &L, hipStream_t s,
                      const int8_t *WOx)
{
    const int tiles_m = (int)((T + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    const dim3 grid((unsigned)(tiles_m * tiles_n));
    const dim3 block(WM * WN * 64);
    const int8_t *Xq = reinterpret_cast<const int8_t *>(ws + L.Xq);
    const float *sX = reinterpret_cast<const float *>(ws + L.sX);
    const int32_t *meta = reinterpret_cast<const int32_t *>(ws + L.meta);
    const uint16_t *XO = reinterpret_cast<const uint16_t *>(ws + L.XO);
    const int8_t *WO = WOx ? WOx : reinterpret_cast<const int8_t *>(ws + L.WO);
    const int32_t *idx = reinterpret_cast<const int32_t *>(ws + L.idx);
    const int32_t *wpre = reinterpret_cast<const int32_t *>(ws + L.wpre);
    if (acc)
        hipLaunchKernelGGL((k_gemm<BM, BN, BKS, NS, WM, WN, GM, F16W, true>), grid, block, 0, s, Xq, Wq,
                           sX, sW, meta, XO, WO, idx, wpre, (int)T, (int)K, (int)N, tiles_m, tiles_n, Y,
                           acc);
    else
        hipLaunchKernelGGL((k_gemm<BM, BN, BKS, NS, WM, WN, GM, F16W, false>), grid, block, 0, s, Xq, Wq,
                           sX, sW, meta, XO, WO, idx, wpre, (int)T, (int)K, (int)N, tiles_m, tiles_n, Y,
                           acc);
    return hipGetLastError();
}

} // namespace

// Tile shape: 256x256 by default; 256x192 (8 waves of 64x96) or 256x128
// (8 waves of 64x64) when the 256x256 grid leaves a large part of the last
// round of workgroups empty (few tokens per 256 rows, or a tile count just
// above a multiple of the CU count).  Cost model: rounds of workgroups over
// the 256 CUs times the work of one tile, the smaller tiles charged 15 %
// and 35 % more per operation: their lower reuse costs cycles and, under
// the power-limited clock of calls back to back, energy.  (Measured: at
// 2048 x 4096 x 11008 the 256x192 grid's 1.81 rounds beat the 256x256
// grid's 1.34 and the 256x128 grid's 2.69; at 4096 x 4096 x 11008 the
// 256x256 grid's 2.69 rounds beat the 256x192 grid's 3.63; at
// 512 x 5120 x 13824 one round of 256x128 tiles beats both.)
constexpr int kCUs = 256;

GemmPlan gemm_plan(int64_t T, int64_t K, int64_t N)
{
    const int64_t tm = (T + 255) / 256;
    const int64_t big = tm * ((N + 255) / 256), mid = tm * ((N + 191) / 192),
                  small = tm * ((N + 127) / 128);
    const double cost_big = (double)((big + kCUs - 1) / kCUs);
    const double cost_mid = 0.75 * 1.15 * (double)((mid + kCUs - 1) / kCUs);
    const double cost_small = 0.5 * 1.35 * (double)((small + kCUs - 1) / kCUs);
    // the most outlier columns the int8 GEMM copies out of its weight
    // stages (its CAP), for K <= kFoldMaxK (its LDS copy of the bit set):
    // 256 on 128-wide tiles; the wider tiles never copy them (measured
    // slower than the prepare kernel's gather at every count tried: the
    // copies cost the 256- and 192-wide main loops 19 and 10 us at about 30
    // outlier columns, where the gather costs 4-5 us)
    const bool fold_k = K <= kFoldMaxK;
    if (cost_small < cost_big && cost_small <= cost_mid)
        return {256, 128, fold_k ? 256 : 0};
    if (cost_mid < cost_big)
        return {256, 192, 0};
    return {256, 256, 0};
}

hipError_t launch_gemm(const int8_t *Wq, const float *sW, int64_t T, int64_t K, int64_t N,
                       uint16_t *Y, int32_t *acc, const char *ws, const WsLayout &L, bool fp16w,
                       hipStream_t s, const int8_t *WO)
{
    const GemmPlan p = gemm_plan(T, K, N);
    if (p.bn == 128)
        return fp16w ? launch_cfg<256, 128, 128, 2, 4, 2, 4, true>(Wq, sW, T, K, N, Y, acc, ws, L, s, WO)
                     : launch_cfg<256, 128, 128, 2, 4, 2, 4, false>(Wq, sW, T, K, N, Y, acc, ws, L, s, WO);
    if (p.bn == 192)
        return fp16w ? launch_cfg<256, 192, 128, 2, 4, 2, 4, true>(Wq, sW, T, K, N, Y, acc, ws, L, s, WO)
                     : launch_cfg<256, 192, 128, 2, 4, 2, 4, false>(Wq, sW, T, K, N, Y, acc, ws, L, s, WO);
    return fp16w ? launch_cfg<256, 256, 128, 2, 2, 4, 4, true>(Wq, sW, T, K, N, Y, acc, ws, L, s, WO)
                 : launch_cfg<256, 256, 128, 2, 2, 4, 4, false>(Wq, sW, T, K, N, Y, acc, ws, L, s, WO);
}

} // namespace li8
