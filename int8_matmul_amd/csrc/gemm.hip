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
// Both operands are K-contiguous ("NT").  Tiles: BM x BN per workgroup,
// BK = 128 bytes of K per stage, two LDS stages, WM x WN waves each owning
// an (FM*32) x (FN*32) sub-tile computed with v_mfma_i32_32x32x32_i8.
// Global -> register -> LDS staging with an XOR swizzle of the 16-byte
// chunks so that both the row-wise LDS writes and the MFMA fragment reads
// hit distinct banks.
#include "li8_internal.h"

namespace li8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int BK = 128;          // bytes of K per stage
constexpr int CPR = BK / 16;     // 16-byte chunks per tile row

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & (CPR - 1); }

template <int BM, int BN, int WM, int WN, bool STORE_ACC>
__global__ __launch_bounds__(WM *WN * 64) void k_gemm(
    const int8_t *__restrict__ Xq, const int8_t *__restrict__ Wq,
    const float *__restrict__ sX, const float *__restrict__ sW,
    const int32_t *__restrict__ meta, const uint16_t *__restrict__ XO,
    const int8_t *__restrict__ WO, int T, int K, int N, int tiles_m,
    uint16_t *__restrict__ Y, int32_t *__restrict__ acc_out)
{
    constexpr int NT = WM * WN * 64;
    constexpr int FM = BM / (WM * 32);
    constexpr int FN = BN / (WN * 32);
    constexpr int CA = BM * CPR / NT;   // 16-byte chunks per thread per stage (A)
    constexpr int CB = BN * CPR / NT;
    static_assert(FM * WM * 32 == BM && FN * WN * 32 == BN, "tile shape");
    static_assert(CA * NT == BM * CPR && CB * NT == BN * CPR, "loader shape");

    __shared__ __attribute__((aligned(16))) int8_t lds_a[2][BM * BK];
    __shared__ __attribute__((aligned(16))) int8_t lds_b[2][BN * BK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int wm = wid / WN, wn = wid % WN;
    const int tile_m = blockIdx.x % tiles_m;
    const int tile_n = blockIdx.x / tiles_m;
    const int m0 = tile_m * BM, n0 = tile_n * BN;

    // ---- per-thread loader coordinates ----
    const int8_t *ga[CA];
    const int8_t *gb[CB];
    int la[CA], lb[CB], ka[CA], kb[CB];
#pragma unroll
    for (int i = 0; i < CA; i++) {
        const int c = tid + i * NT, row = c / CPR, q = c % CPR;
        ga[i] = Xq + (int64_t)min(m0 + row, T - 1) * K + q * 16;
        ka[i] = q * 16;
        la[i] = row * BK + ((q ^ swz(row)) * 16);
    }
#pragma unroll
    for (int i = 0; i < CB; i++) {
        const int c = tid + i * NT, row = c / CPR, q = c % CPR;
        gb[i] = Wq + (int64_t)min(n0 + row, N - 1) * K + q * 16;
        kb[i] = q * 16;
        lb[i] = row * BK + ((q ^ swz(row)) * 16);
    }

    v16i acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; a++)
#pragma unroll
        for (int b = 0; b < FN; b++)
            acc[a][b] = v16i{};

    const int nk = (K + BK - 1) / BK;
    v4i ra[CA], rb[CB];
    auto gload = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < CA; i++)
            ra[i] = (k0 + ka[i] < K) ? *reinterpret_cast<const v4i *>(ga[i] + k0) : v4i{};
#pragma unroll
        for (int i = 0; i < CB; i++)
            rb[i] = (k0 + kb[i] < K) ? *reinterpret_cast<const v4i *>(gb[i] + k0) : v4i{};
    };
    auto lstore = [&](int st) {
#pragma unroll
        for (int i = 0; i < CA; i++)
            *reinterpret_cast<v4i *>(&lds_a[st][la[i]]) = ra[i];
#pragma unroll
        for (int i = 0; i < CB; i++)
            *reinterpret_cast<v4i *>(&lds_b[st][lb[i]]) = rb[i];
    };

    // fragment rows owned by this lane
    const int arow0 = wm * FM * 32 + (lane & 31);
    const int brow0 = wn * FN * 32 + (lane & 31);
    const int khalf = lane >> 5;

    if (nk > 0) {
        gload(0);
        lstore(0);
        __syncthreads();
    }
    for (int kt = 0; kt < nk; kt++) {
        const int st = kt & 1;
        if (kt + 1 < nk)
            gload(kt + 1);
#pragma unroll
        for (int kk = 0; kk < BK / 32; kk++) {
            const int q = kk * 2 + khalf;
            v4i fa[FM], fb[FN];
#pragma unroll
            for (int a = 0; a < FM; a++) {
                const int row = arow0 + a * 32;
                fa[a] = *reinterpret_cast<const v4i *>(&lds_a[st][row * BK + ((q ^ swz(row)) * 16)]);
            }
#pragma unroll
            for (int b = 0; b < FN; b++) {
                const int row = brow0 + b * 32;
                fb[b] = *reinterpret_cast<const v4i *>(&lds_b[st][row * BK + ((q ^ swz(row)) * 16)]);
            }
#pragma unroll
            for (int a = 0; a < FM; a++)
#pragma unroll
                for (int b = 0; b < FN; b++)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[a], fb[b], acc[a][b], 0, 0, 0);
        }
        if (kt + 1 < nk)
            lstore(st ^ 1);
        __syncthreads();
    }

    // ---- epilogue ----
    // 32x32 MFMA result layout: lane l, register r -> column (l & 31),
    // row 8*(r/4) + 4*(l/32) + (r%4) of the 32x32 block.
    const int nO = meta[0];
    const int nch = (nO + 15) >> 4;
    v16f d[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; a++) {
        float sx[16];
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int row = m0 + wm * FM * 32 + a * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
            sx[r] = sX[min(row, T - 1)];
        }
#pragma unroll
        for (int b = 0; b < FN; b++) {
            if constexpr (STORE_ACC) {
                const int col = n0 + wn * FN * 32 + b * 32 + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int row = m0 + wm * FM * 32 + a * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
                    if (row < T && col < N)
                        acc_out[(int64_t)row * N + col] = acc[a][b][r];
                }
            }
#pragma unroll
            for (int r = 0; r < 16; r++)
                d[a][b][r] = (float)acc[a][b][r] * sx[r];
        }
    }
    for (int c = 0; c < nch; c++) {
        v8h xa[FM], wb[FN];
#pragma unroll
        for (int a = 0; a < FM; a++) {
            const int row = min(m0 + arow0 + a * 32, T - 1);
            xa[a] = *reinterpret_cast<const v8h *>(XO + (int64_t)row * K + c * 16 + khalf * 8);
        }
#pragma unroll
        for (int b = 0; b < FN; b++) {
            const int col = min(n0 + brow0 + b * 32, N - 1);
            const uint2 u = *reinterpret_cast<const uint2 *>(WO + (int64_t)col * K + c * 16 + khalf * 8);
            const uint32_t w[2] = {u.x, u.y};
#pragma unroll
            for (int e = 0; e < 8; e++)
                wb[b][e] = (_Float16)(float)(int8_t)((w[e >> 2] >> (8 * (e & 3))) & 0xffu);
        }
#pragma unroll
        for (int a = 0; a < FM; a++)
#pragma unroll
            for (int b = 0; b < FN; b++)
                d[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xa[a], wb[b], d[a][b], 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < FN; b++) {
        const int col = n0 + wn * FN * 32 + b * 32 + (lane & 31);
        const float sw = sW[min(col, N - 1)];
#pragma unroll
        for (int a = 0; a < FM; a++) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int row = m0 + wm * FM * 32 + a * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
                if (row < T && col < N) {
                    // fl32(D * sW) first, then one rounding to fp16: the empty
                    // asm keeps the compiler from fusing the product and the
                    // conversion into a single-rounding v_fma_mixlo_f16
                    float p = d[a][b][r] * sw;
                    asm("" : "+v"(p));
                    const _Float16 h = (_Float16)p;
                    Y[(int64_t)row * N + col] = __builtin_bit_cast(uint16_t, h);
                }
            }
        }
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_tile(const int8_t *Wq, const float *sW, int64_t T, int64_t K, int64_t N,
                       uint16_t *Y, int32_t *acc, const char *ws, const WsLayout &L,
                       hipStream_t s)
{
    const int tiles_m = (int)((T + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    const dim3 grid((unsigned)(tiles_m * tiles_n));
    const dim3 block(WM * WN * 64);
    const int8_t *Xq = reinterpret_cast<const int8_t *>(ws + L.Xq);
    const float *sX = reinterpret_cast<const float *>(ws + L.sX);
    const int32_t *meta = reinterpret_cast<const int32_t *>(ws + L.meta);
    const uint16_t *XO = reinterpret_cast<const uint16_t *>(ws + L.XO);
    const int8_t *WO = reinterpret_cast<const int8_t *>(ws + L.WO);
    if (acc)
        hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN, true>), grid, block, 0, s, Xq, Wq, sX, sW,
                           meta, XO, WO, (int)T, (int)K, (int)N, tiles_m, Y, acc);
    else
        hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN, false>), grid, block, 0, s, Xq, Wq, sX, sW,
                           meta, XO, WO, (int)T, (int)K, (int)N, tiles_m, Y, acc);
    return hipGetLastError();
}

} // namespace

hipError_t launch_gemm(const int8_t *Wq, const float *sW, int64_t T, int64_t K, int64_t N,
                       uint16_t *Y, int32_t *acc, const char *ws, const WsLayout &L,
                       hipStream_t s)
{
    return launch_tile<256, 256, 2, 4>(Wq, sW, T, K, N, Y, acc, ws, L, s);
}

} // namespace li8
