/*
 * CPU oracle for the LLM.int8() mixed-precision decomposition matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no code, header or table with the HIP
 * library: it has its own binary16 conversion and its own loops.
 *
 * What it computes, step by step, as the pages define the method:
 *
 *   Symmetric absmax quantization (lowentro.cn "model quantization" notes,
 *   Q2; tqpw.cn/news/5683, section 2.1): one scale s = absmax / (2^(8-1)-1)
 *   = absmax / 127, code q = round(r / s), zero point 0, dequantized value
 *   s * q.  Codes are clipped to [-127, 127] (notes Q11).
 *
 *   Vector-wise granularity (hncyxsy.com/news/230290, section 2.1; notes
 *   Q3): the weight gets one scale per output feature (row n of W[N,K]); the
 *   activation gets one scale per token (row t of X[T,K]).
 *
 *   Mixed-precision decomposition (hncyxsy.com/news/230290, section 2.1;
 *   notes Q4; tqpw.cn/news/5683, section 3.1): feature columns j of X in
 *   which some |x| exceeds the threshold (6.0) are outliers.  Those columns
 *   of X and of the weight are multiplied in floating point; the remaining
 *   columns go through the int8 matmul; the two parts are added and the sum
 *   is returned in fp16.
 *
 * Readings taken where the pages leave a step open:
 *   - "exceeds" is strict: |x| > threshold.
 *   - The outlier set is one set of columns per call, the union over all
 *     rows of X.
 *   - The token scale is the absmax over the normal columns only; outlier
 *     columns get code 0 in Xq.  A row (or weight row) whose absmax is 0 has
 *     scale 0 and all codes 0.
 *   - Scales are fp32; the code is round-half-to-even of the fp32 quotient
 *     fl32(r / s), clamped to [-127, 127].
 *   - The int8 products are summed exactly (int32).  The dequantized value is
 *     fl32(fl32(acc * sX[t]) * sW[n]).
 *   - The weight used for the outlier columns is the dequantized int8 weight
 *     Wq[n,j] * sW[n] (only Wq and sW are kept once the weight is quantized);
 *     a variant takes the original fp16 weight there instead.
 *     The outlier sum and the final addition are done in fp64 and rounded
 *     once, half-to-even, to fp16.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared -ffp-contract=off oracle.c -lm.
 * Never with -ffast-math: the oracle relies on IEEE division and on rintf
 * rounding half-to-even (the default rounding mode).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- IEEE-754 binary16 <-> double, written from the format definition ---- */

/* Exact value of a binary16 bit pattern. */
double oracle_h2d(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);               /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);   /* (1.m) * 2^(e-15) */
    return sign ? -v : v;
}

/* Round a double to the nearest binary16, ties to even. */
uint16_t oracle_d2h(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return 0x7e00;
    if (a >= 65520.0)                 /* halfway between 65504 and 2^16 rounds up */
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {        /* subnormal range, step 2^-24 */
        double q = rint(ldexp(a, 24)); /* exact scaling, then ties-to-even */
        return sign | (uint16_t)q;    /* q == 1024 is the smallest normal */
    }
    int E;
    frexp(a, &E);                     /* a = f * 2^E, f in [0.5, 1) */
    int ue = E - 1;                   /* a in [2^ue, 2^(ue+1)) */
    double r = rint(ldexp(a, 10 - ue)); /* significand in [1024, 2048] */
    if (r == 2048.0) {
        r = 1024.0;
        ue += 1;
    }
    if (ue > 15)
        return sign | 0x7c00;
    return sign | (uint16_t)(((ue + 15) << 10) | ((int)r - 1024));
}

void oracle_h2d_array(const uint16_t *h, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_h2d(h[i]);
}

void oracle_d2h_array(const double *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_d2h(x[i]);
}

/* ---- symmetric absmax int8 code of one value given its fp32 scale ---- */

static int8_t code_of(float r, float s)
{
    if (s == 0.0f)
        return 0;                     /* absmax 0: the whole vector is zero */
    float q = rintf(r / s);           /* fl32 quotient, ties to even */
    if (q > 127.0f)
        q = 127.0f;
    if (q < -127.0f)
        q = -127.0f;
    return (int8_t)q;
}

/*
 * Weight quantization, once per weight: one scale per output feature.
 *   sW[n] = fl32(max_k |W[n,k]| / 127),  Wq[n,k] = clamp(rne(fl32(W/sW)))
 */
void oracle_quantize_weight(const uint16_t *W, int64_t N, int64_t K,
                            int8_t *Wq, float *sW)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        const uint16_t *w = W + n * K;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; k++) {
            float a = (float)fabs(oracle_h2d(w[k]));
            if (a > amax)
                amax = a;
        }
        float s = amax / 127.0f;
        sW[n] = s;
        for (int64_t k = 0; k < K; k++)
            Wq[n * K + k] = code_of((float)oracle_h2d(w[k]), s);
    }
}

/*
 * Outlier feature columns: flags[j] = 1 iff some row t has |X[t,j]| > thr.
 * idx lists the flagged columns in ascending order; *nO is their count.
 */
void oracle_detect_outliers(const uint16_t *X, int64_t T, int64_t K, double thr,
                            uint8_t *flags, int32_t *nO, int32_t *idx)
{
    memset(flags, 0, (size_t)K);
    for (int64_t t = 0; t < T; t++)
        for (int64_t j = 0; j < K; j++)
            if (fabs(oracle_h2d(X[t * K + j])) > thr)
                flags[j] = 1;
    int32_t c = 0;
    for (int64_t j = 0; j < K; j++)
        if (flags[j])
            idx[c++] = (int32_t)j;
    *nO = c;
}

/*
 * Token-wise quantization over the normal columns (flags[j] == 0):
 *   sX[t] = fl32(max_{j normal} |X[t,j]| / 127)
 *   Xq[t,j] = 0 for outlier columns, else clamp(rne(fl32(X/sX)))
 * Works on any set of rows given the call's flags.
 */
void oracle_quantize_rows(const uint16_t *X, int64_t R, int64_t K,
                          const uint8_t *flags, int8_t *Xq, float *sX)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < R; t++) {
        const uint16_t *x = X + t * K;
        float amax = 0.0f;
        for (int64_t j = 0; j < K; j++) {
            if (flags[j])
                continue;
            float a = (float)fabs(oracle_h2d(x[j]));
            if (a > amax)
                amax = a;
        }
        float s = amax / 127.0f;
        sX[t] = s;
        for (int64_t j = 0; j < K; j++)
            Xq[t * K + j] = flags[j] ? 0 : code_of((float)oracle_h2d(x[j]), s);
    }
}

/* acc[t,n] = sum_j Xq[t,j] * Wq[n,j], exact in integers. */
void oracle_int8_gemm(const int8_t *Xq, const int8_t *Wq, int64_t R, int64_t N,
                      int64_t K, int32_t *acc)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < R; t++) {
        for (int64_t n = 0; n < N; n++) {
            const int8_t *a = Xq + t * K;
            const int8_t *b = Wq + n * K;
            int64_t s = 0;
            for (int64_t j = 0; j < K; j++)
                s += (int64_t)a[j] * (int64_t)b[j];
            acc[t * N + n] = (int32_t)s;
        }
    }
}

/*
 * Output of the decomposition for rows X[0..R) given their acc and sX:
 *   D = fl32(fl32(acc * sX[t]) * sW[n])                    (int8 part)
 *   E = sum_{j outlier} X[t,j] * (Wq[n,j] * sW[n])  in fp64  (fp16 part)
 *   Y = fp16_rne(D + E)
 */
void oracle_decomposed_output(const uint16_t *X, const int32_t *acc,
                              const float *sX, const int8_t *Wq, const float *sW,
                              const int32_t *idx, int32_t nO,
                              int64_t R, int64_t K, int64_t N, uint16_t *Y)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < R; t++) {
        for (int64_t n = 0; n < N; n++) {
            const uint16_t *x = X + t * K;
            float d = (float)acc[t * N + n] * sX[t];
            d = d * sW[n];
            double e = 0.0;
            for (int32_t i = 0; i < nO; i++) {
                int64_t j = idx[i];
                double w = (double)Wq[n * K + j] * (double)sW[n];
                e += oracle_h2d(x[j]) * w;
            }
            Y[t * N + n] = oracle_d2h((double)d + e);
        }
    }
}

/*
 * The variant in which the outlier columns are multiplied by the original
 * fp16 weight rather than by its dequantized codes (hncyxsy.com/news/230290,
 * section 2.1: the weight sub-matrix of the outlier columns is extracted and
 * multiplied in fp16 together with the outlier columns of X).  W16 is the
 * fp16 weight [N,K] that Wq and sW were quantized from.
 *   D = fl32(fl32(acc * sX[t]) * sW[n])             (int8 part, unchanged)
 *   E = sum_{j outlier} X[t,j] * W16[n,j]   in fp64 (fp16 part)
 *   Y = fp16_rne(D + E)
 */
void oracle_decomposed_output_fp16w(const uint16_t *X, const int32_t *acc,
                                    const float *sX, const float *sW, const uint16_t *W16,
                                    const int32_t *idx, int32_t nO,
                                    int64_t R, int64_t K, int64_t N, uint16_t *Y)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < R; t++) {
        for (int64_t n = 0; n < N; n++) {
            const uint16_t *x = X + t * K;
            float d = (float)acc[t * N + n] * sX[t];
            d = d * sW[n];
            double e = 0.0;
            for (int32_t i = 0; i < nO; i++) {
                int64_t j = idx[i];
                e += oracle_h2d(x[j]) * oracle_h2d(W16[n * K + j]);
            }
            Y[t * N + n] = oracle_d2h((double)d + e);
        }
    }
}

/* The whole call: Y[T,N] = decomposed X * W^T, plus optional stage outputs. */
/* W16 may be NULL (outliers times the dequantized codes) or the fp16 weight
   (the fp16-weight variant above). */
int oracle_linear(const uint16_t *X, const int8_t *Wq, const float *sW, const uint16_t *W16,
                  double thr, int64_t T, int64_t K, int64_t N, uint16_t *Y,
                  uint8_t *flags_out, int32_t *nO_out, int32_t *idx_out,
                  int8_t *Xq_out, float *sX_out, int32_t *acc_out)
{
    uint8_t *flags = flags_out ? flags_out : malloc((size_t)(K ? K : 1));
    int32_t *idx = idx_out ? idx_out : malloc(sizeof(int32_t) * (size_t)(K ? K : 1));
    int8_t *Xq = Xq_out ? Xq_out : malloc((size_t)(T * K > 0 ? T * K : 1));
    float *sX = sX_out ? sX_out : malloc(sizeof(float) * (size_t)(T ? T : 1));
    int32_t *acc = acc_out ? acc_out : malloc(sizeof(int32_t) * (size_t)(T * N > 0 ? T * N : 1));
    int32_t nO = 0;
    if (!flags || !idx || !Xq || !sX || !acc)
        return -1;
    oracle_detect_outliers(X, T, K, thr, flags, &nO, idx);
    oracle_quantize_rows(X, T, K, flags, Xq, sX);
    oracle_int8_gemm(Xq, Wq, T, N, K, acc);
    if (W16)
        oracle_decomposed_output_fp16w(X, acc, sX, sW, W16, idx, nO, T, K, N, Y);
    else
        oracle_decomposed_output(X, acc, sX, Wq, sW, idx, nO, T, K, N, Y);
    if (nO_out)
        *nO_out = nO;
    if (!flags_out) free(flags);
    if (!idx_out) free(idx);
    if (!Xq_out) free(Xq);
    if (!sX_out) free(sX);
    if (!acc_out) free(acc);
    return 0;
}

int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}

/*
 * SmoothQuant-style W8A8.  The exact rewrite x . W^T = (x / s) . (W * s)^T
 * (lowentro.cn "model quantization" notes, Q9; hncyxsy.com/news/230290,
 * section 5.1) with one factor s_j per input channel moves quantization
 * difficulty from the activation to the weight; then both are quantized to
 * int8 with the same absmax scheme as above and multiplied with no outlier
 * decomposition.
 *
 * The factor (lowentro.cn notes, Q10).  Its formula line is garbled: it
 * prints a product, max|X_j|^alpha * max|W_j|^(1-alpha), and from it the
 * value max|W_j| at alpha = 0.  It is read here as the quotient
 *   s_j = ax_j^alpha / aw_j^(1-alpha)
 * because the same answer says what the factor has to achieve and only the
 * quotient achieves it.  After the rewrite the channel's ranges are
 * ax_j / s_j (activation) and aw_j * s_j (weight):
 *   - alpha = 0.5 is to balance them: ax/s = aw*s  <=>  s = sqrt(ax / aw);
 *   - alpha = 1 moves all of the activation's difficulty to the weight,
 *     s = ax (the activation range becomes 1; both forms agree here);
 *   - alpha = 0 moves all of the weight's difficulty to the activation, so
 *     the weight range becomes 1: s = 1 / aw.  The product's s = aw would
 *     instead square the weight's range, the opposite of what the answer
 *     describes, so its printed alpha = 0 value is not taken.
 * (hncyxsy.com section 5.1 calls alpha = 0 "no migration", which neither
 * form gives; not taken either.)
 *
 * Other readings:
 *   ax_j = max_t |X_cal[t,j]| over a calibration batch, aw_j = max_n
 *   |W[n,j]|; s_j computed in fp64, rounded to fp32; s_j = 1 when ax_j or
 *   aw_j is 0 (the channel carries nothing).
 *   W'[n,j] = fl32(W[n,j] * s_j), then the weight absmax quantization.
 *   X'[t,j] = fl32(X[t,j] * fl32(1 / s_j)), then the token absmax
 *   quantization over all columns; Y = fp16(fl32(fl32(acc * sX') * sW')).
 */
void oracle_sq_factors(const float *ax, const float *aw, double alpha, int64_t K, float *s)
{
    for (int64_t j = 0; j < K; j++) {
        if (ax[j] == 0.0f || aw[j] == 0.0f)
            s[j] = 1.0f;
        else
            s[j] = (float)(pow((double)ax[j], alpha) / pow((double)aw[j], 1.0 - alpha));
    }
}

/* max |X[t,j]| over the rows, per column, as fp32 (exact for fp16 values) */
void oracle_column_absmax(const uint16_t *X, int64_t R, int64_t K, float *out)
{
    for (int64_t j = 0; j < K; j++) {
        double m = 0.0;
        for (int64_t t = 0; t < R; t++) {
            double v = fabs(oracle_h2d(X[t * K + j]));
            if (v > m)
                m = v;
        }
        out[j] = (float)m;
    }
}

/* absmax code of an fp32 value for scale s (s > 0): rne(fl32(r / s)),
   clamped to [-127, 127] */
static int8_t sq_code(float r, float s)
{
    float q = rintf(r / s);
    if (q > 127.0f)
        q = 127.0f;
    if (q < -127.0f)
        q = -127.0f;
    return (int8_t)q;
}

void oracle_sq_quantize_weight(const uint16_t *W, const float *s, int64_t N, int64_t K,
                               int8_t *Wq, float *sW)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        float a = 0.0f;
        for (int64_t j = 0; j < K; j++) {
            float w = (float)oracle_h2d(W[n * K + j]) * s[j];
            if (fabsf(w) > a)
                a = fabsf(w);
        }
        const float sc = a / 127.0f;
        sW[n] = sc;
        for (int64_t j = 0; j < K; j++) {
            float w = (float)oracle_h2d(W[n * K + j]) * s[j];
            Wq[n * K + j] = sc > 0.0f ? sq_code(w, sc) : 0;
        }
    }
}

/* token side: smoothed codes and scales of rows X[0..R) */
void oracle_sq_quantize_rows(const uint16_t *X, const float *s, int64_t R, int64_t K,
                             int8_t *Xq, float *sX)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < R; t++) {
        float a = 0.0f;
        for (int64_t j = 0; j < K; j++) {
            float x = (float)oracle_h2d(X[t * K + j]) * (1.0f / s[j]);
            if (fabsf(x) > a)
                a = fabsf(x);
        }
        const float sc = a / 127.0f;
        sX[t] = sc;
        for (int64_t j = 0; j < K; j++) {
            float x = (float)oracle_h2d(X[t * K + j]) * (1.0f / s[j]);
            Xq[t * K + j] = sc > 0.0f ? sq_code(x, sc) : 0;
        }
    }
}

/* Y = fp16(fl32(fl32(acc * sX) * sW)) (no outlier term) */
void oracle_sq_output(const int32_t *acc, const float *sX, const float *sW, int64_t R, int64_t N,
                      uint16_t *Y)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < R; t++) {
        for (int64_t n = 0; n < N; n++) {
            float d = (float)acc[t * N + n] * sX[t];
            d = d * sW[n];
            Y[t * N + n] = oracle_d2h((double)d);
        }
    }
}
