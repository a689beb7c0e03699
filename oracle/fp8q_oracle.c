/*
 * CPU oracle for block-scaled FP8 (E4M3) quantization and FP8 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow reference that the
 * GPU library is checked against.  Only the test suite, the smoke entry point
 * and the CPU-baseline leg of the benchmark may load it; the product path
 * never does.  It shares no code, header, table or constant generator with
 * the HIP kernels.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC
 *   (no FMA contraction, no flush-to-zero: every float operation below rounds
 *   once, to nearest-even, exactly as written).
 *
 * Sources of each definition (the web pages on FP8 training):
 *  - E4M3 = 4 exponent bits + 3 mantissa bits, finite range [-448, 448]:
 *    "FP8-RL" article, section 一 (weight sync); FP8-LM review, section 三
 *    (FP8 data formats); Introl FP8 infrastructure guide, section on the
 *    numerical-precision landscape.
 *  - Quantization is x_fp8 = Cast_FP8(x / s): FP8-LM review, section 三
 *    (tensor scaling formula).
 *  - A BF16 tensor becomes an FP8 tensor plus a smaller, wider-range scale
 *    tensor: Ling 2.0 FP8 blog, "where does the precision worry come from".
 *  - Fine-grained tile/block scales, one scale per tile: Ling 2.0 FP8 blog,
 *    "fine-grained quantization (per-tile/block wise scaling)"; 128x128
 *    weight blocks: "FP8-RL" article, section 一.
 *  - FP8 GEMM accumulates in FP32: Ling 2.0 FP8 blog, "where is error
 *    introduced".
 * Readings where the pages are silent (each listed in the design notes):
 *  scale s = amax/448 in fp32, stored as the dequantisation multiplier;
 *  x/s is an IEEE fp32 quotient, then rounded to E4M3 nearest-even with
 *  saturation at 448 (two-step rounding); OCP E4M3FN encoding (bias 7,
 *  subnormals, no infinities, NaN = S.1111.111); a zero tile (or a scale that
 *  underflows to 0) gets s = 0 and signed-zero codes; the GEMM adds each
 *  128-wide K chunk's fp32 partial sum, times SA*SB, into an fp32
 *  accumulator, in ascending k and chunk order, without FMA.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Sets the number of threads the parallel loops below run on (timing only:
   no result depends on it). */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Threads the parallel loops below run on (reported with CPU timings). */
int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* E4M3 codec (OCP E4M3FN)                                              */
/* ------------------------------------------------------------------ */

/* Decode: sign s, exponent field e (4 bits, bias 7), mantissa m (3 bits).
 * e == 0 is subnormal: m * 2^-9.  e == 15 && m == 7 is NaN. */
float orc_e4m3_decode(uint8_t c)
{
    int s = c >> 7;
    int e = (c >> 3) & 15;
    int m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return s ? -NAN : NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return (float)(s ? -v : v);
}

/* Round a non-negative double t (with few significant bits) to the nearest
 * integer, ties to even. */
static double round_half_even(double t)
{
    double fl = floor(t);
    double fr = t - fl;
    if (fr > 0.5)
        return fl + 1.0;
    if (fr < 0.5)
        return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* Encode an fp32 value: round to nearest E4M3 value, ties to the code with
 * an even mantissa LSB; magnitudes above 448 saturate to 448; the sign bit
 * of the code is the sign bit of v (so -0 and negative underflow give 0x80).
 * NaN maps to the NaN code with v's sign (outside the GPU contract). */
uint8_t orc_e4m3_encode(float v)
{
    uint32_t bits;
    memcpy(&bits, &v, 4);
    uint8_t sign = (uint8_t)((bits >> 31) << 7);
    if (isnan(v))
        return sign | 0x7F;
    double a = fabs((double)v);
    if (a > 448.0)
        return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: multiples of 2^-9; q == 8 is the min normal */
        double q = round_half_even(a * 512.0);
        return sign | (uint8_t)q;
    }
    int ex;
    double f = frexp(a, &ex);   /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;             /* a = (2f) * 2^e, 2f in [1, 2) */
    double q = round_half_even((2.0 * f - 1.0) * 8.0);
    if (q == 8.0) {
        e += 1;
        q = 0.0;
    }
    return sign | (uint8_t)((e + 7) << 3) | (uint8_t)q;
}

void orc_decode_array(const uint8_t* c, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_e4m3_decode(c[i]);
}

void orc_encode_array(const float* v, int64_t n, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_e4m3_encode(v[i]);
}

/* ------------------------------------------------------------------ */
/* Tile quantization                                                    */
/* ------------------------------------------------------------------ */

/* Quantize X[rows][cols] (row-major, contiguous fp32) with tiles of
 * tr rows x tc cols.  Tiles start at row 0 / col 0; tiles on the bottom and
 * right edges are clipped to the matrix.  For every tile:
 *   amax = max |x| over the tile (fp32),  s = amax / 448 (fp32 division),
 *   q    = encode(fp32(x / s))            (or signed zero if s == 0).
 * Outputs: q[rows][cols], s[ceil(rows/tr)][ceil(cols/tc)]. */
void orc_quant_tiles(const float* x, int64_t rows, int64_t cols, int64_t tr,
                     int64_t tc, uint8_t* q, float* s)
{
    int64_t tiles_r = (rows + tr - 1) / tr;
    int64_t tiles_c = (cols + tc - 1) / tc;
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
    for (int64_t ti = 0; ti < tiles_r; ++ti) {
        for (int64_t tj = 0; tj < tiles_c; ++tj) {
            int64_t r0 = ti * tr, r1 = r0 + tr < rows ? r0 + tr : rows;
            int64_t c0 = tj * tc, c1 = c0 + tc < cols ? c0 + tc : cols;
            float amax = 0.0f;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c) {
                    float a = fabsf(x[r * cols + c]);
                    if (a > amax)
                        amax = a;
                }
            float scale = amax / 448.0f;
            s[ti * tiles_c + tj] = scale;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c) {
                    float v = x[r * cols + c];
                    uint8_t code;
                    if (scale == 0.0f) {
                        code = signbit(v) ? 0x80 : 0x00;
                    } else {
                        float t = v / scale;
                        code = orc_e4m3_encode(t);
                    }
                    q[r * cols + c] = code;
                }
        }
    }
}

/* Power-of-two scales, the micro-scaling variant of block scaling
 * (Introl FP8 infrastructure guide, section on scaling strategies: Blackwell's
 * MXFP8 gives each block of a tensor its own scale factor; its Blackwell
 * section: the block scaling is done in hardware).  The pages do not say how
 * the block scale is chosen or stored; the reading taken here keeps the tile
 * shapes above and restricts s to a power of two 2^e, stored as the 8-bit
 * exponent byte e + 127 (E8M0), with
 *   e = the smallest integer >= -126 such that amax <= 448 * 2^e,
 * i.e. s = 2^ceil(log2(amax / 448)) taken without rounding, so that no value
 * of the tile saturates, and amax = 0 gives e = -126.  The comparison is made
 * in double, where 448 * 2^e and every fp32 amax are exact.  Codes are
 * encode(fp32(x / 2^e)); the quotient is exact unless it is below 2^-126,
 * where every code is a signed zero anyway. */
int orc_pow2_exponent(float amax)
{
    int e = -126;
    if ((double)amax > 448.0 * ldexp(1.0, e)) {
        int k;
        frexp((double)amax, &k);            /* amax = f * 2^k, 0.5 <= f < 1 */
        e = k - 10;                         /* 448 * 2^(k-10) < 2^(k-1) <= amax */
        while ((double)amax > 448.0 * ldexp(1.0, e))
            e++;
    }
    return e;
}

void orc_quant_tiles_pow2(const float* x, int64_t rows, int64_t cols, int64_t tr,
                          int64_t tc, uint8_t* q, uint8_t* ebyte)
{
    int64_t tiles_r = (rows + tr - 1) / tr;
    int64_t tiles_c = (cols + tc - 1) / tc;
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
    for (int64_t ti = 0; ti < tiles_r; ++ti) {
        for (int64_t tj = 0; tj < tiles_c; ++tj) {
            int64_t r0 = ti * tr, r1 = r0 + tr < rows ? r0 + tr : rows;
            int64_t c0 = tj * tc, c1 = c0 + tc < cols ? c0 + tc : cols;
            float amax = 0.0f;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c) {
                    float a = fabsf(x[r * cols + c]);
                    if (a > amax)
                        amax = a;
                }
            int e = orc_pow2_exponent(amax);
            ebyte[ti * tiles_c + tj] = (uint8_t)(e + 127);
            float scale = ldexpf(1.0f, e);
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c)
                    q[r * cols + c] = orc_e4m3_encode(x[r * cols + c] / scale);
        }
    }
}

/* E8M0 byte -> its power of two as fp32 (2^(b-127); byte 255 is NaN). */
void orc_e8m0_decode_array(const uint8_t* b, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = b[i] == 255 ? NAN : (float)ldexp(1.0, (int)b[i] - 127);
}

/* ------------------------------------------------------------------ */
/* Block-scaled GEMM                                                    */
/* ------------------------------------------------------------------ */

/* C[i][n] for the requested rows m = rows[i] (all rows if rows == NULL):
 *   C[m][n] = sum over chunks kb (ascending) of
 *             (sum over k in chunk kb (ascending) of dec(A[m][k]) * dec(B[n][k]))
 *             * (SA[m][kb] * SB[n][kb])
 * A[M][K] and B[N][K] are E4M3 codes with the contraction axis contiguous.
 * SA[M][KB] and SB[N][KB] are the scales already expanded to one value per
 * (row, chunk) and (column, chunk); KB = ceil(K / 128) and the last chunk
 * may be shorter than 128.  Every product of two E4M3 values is exact in
 * fp32; each addition and multiplication below rounds once (fp32). */
void orc_gemm_f32(int64_t M, int64_t N, int64_t K, const uint8_t* A,
                  const float* SA, const uint8_t* B, const float* SB,
                  const int64_t* rows, int64_t nrows, float* C)
{
    (void)M;
    const int64_t KB = (K + 127) / 128;
    float dec[256];
    for (int c = 0; c < 256; ++c)
        dec[c] = orc_e4m3_decode((uint8_t)c);
    /* B decoded and stored k-major so the n loop is contiguous */
    float* BT = (float*)malloc(sizeof(float) * (size_t)K * (size_t)N);
    float* SBT = (float*)malloc(sizeof(float) * (size_t)KB * (size_t)N);
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            BT[k * N + n] = dec[B[n * K + k]];
    for (int64_t kb = 0; kb < KB; ++kb)
        for (int64_t n = 0; n < N; ++n)
            SBT[kb * N + n] = SB[n * KB + kb];
#pragma omp parallel
    {
        float* p = (float*)malloc(sizeof(float) * (size_t)N);
        float* acc = (float*)malloc(sizeof(float) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < nrows; ++i) {
            int64_t m = rows ? rows[i] : i;
            for (int64_t n = 0; n < N; ++n)
                acc[n] = 0.0f;
            for (int64_t kb = 0; kb < KB; ++kb) {
                int64_t k0 = kb * 128, k1 = k0 + 128 < K ? k0 + 128 : K;
                for (int64_t n = 0; n < N; ++n)
                    p[n] = 0.0f;
                for (int64_t k = k0; k < k1; ++k) {
                    float a = dec[A[m * K + k]];
                    const float* bt = BT + k * N;
                    for (int64_t n = 0; n < N; ++n)
                        p[n] = p[n] + a * bt[n];
                }
                float sa = SA[m * KB + kb];
                const float* sb = SBT + kb * N;
                for (int64_t n = 0; n < N; ++n) {
                    float t = sa * sb[n];
                    acc[n] = acc[n] + p[n] * t;
                }
            }
            memcpy(C + i * N, acc, sizeof(float) * (size_t)N);
        }
        free(p);
        free(acc);
    }
    free(BT);
    free(SBT);
}

/* The same sum carried out in fp64 (the near-exact value of the definition),
 * plus the absolute-product sum
 *   R[m][n] = sum_kb |SA[m][kb] * SB[n][kb]| * sum_k |dec(A[m][k]) * dec(B[n][k])|
 * which bounds the rounding error of any fp32 evaluation order. */
void orc_gemm_f64(int64_t M, int64_t N, int64_t K, const uint8_t* A,
                  const float* SA, const uint8_t* B, const float* SB,
                  const int64_t* rows, int64_t nrows, double* C, double* R)
{
    (void)M;
    const int64_t KB = (K + 127) / 128;
    double dec[256];
    for (int c = 0; c < 256; ++c)
        dec[c] = (double)orc_e4m3_decode((uint8_t)c);
    double* BT = (double*)malloc(sizeof(double) * (size_t)K * (size_t)N);
    double* SBT = (double*)malloc(sizeof(double) * (size_t)KB * (size_t)N);
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            BT[k * N + n] = dec[B[n * K + k]];
    for (int64_t kb = 0; kb < KB; ++kb)
        for (int64_t n = 0; n < N; ++n)
            SBT[kb * N + n] = (double)SB[n * KB + kb];
#pragma omp parallel
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)N);
        double* pa = (double*)malloc(sizeof(double) * (size_t)N);
        double* acc = (double*)malloc(sizeof(double) * (size_t)N);
        double* racc = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < nrows; ++i) {
            int64_t m = rows ? rows[i] : i;
            for (int64_t n = 0; n < N; ++n) {
                acc[n] = 0.0;
                racc[n] = 0.0;
            }
            for (int64_t kb = 0; kb < KB; ++kb) {
                int64_t k0 = kb * 128, k1 = k0 + 128 < K ? k0 + 128 : K;
                for (int64_t n = 0; n < N; ++n) {
                    p[n] = 0.0;
                    pa[n] = 0.0;
                }
                for (int64_t k = k0; k < k1; ++k) {
                    double a = dec[A[m * K + k]];
                    const double* bt = BT + k * N;
                    for (int64_t n = 0; n < N; ++n) {
                        p[n] += a * bt[n];
                        pa[n] += fabs(a * bt[n]);
                    }
                }
                double sa = (double)SA[m * KB + kb];
                const double* sb = SBT + kb * N;
                for (int64_t n = 0; n < N; ++n) {
                    double t = sa * sb[n];
                    acc[n] += p[n] * t;
                    racc[n] += pa[n] * fabs(t);
                }
            }
            memcpy(C + i * N, acc, sizeof(double) * (size_t)N);
            memcpy(R + i * N, racc, sizeof(double) * (size_t)N);
        }
        free(p);
        free(pa);
        free(acc);
        free(racc);
    }
    free(BT);
    free(SBT);
}

/* ------------------------------------------------------------------ */
/* Adam with FP8 moments                                                */
/* ------------------------------------------------------------------ */

/* One AdamW step on fp32 parameters and fp32 moments (the decoupled-weight-
 * decay Adam of Loshchilov and Hutter, bias-corrected as in Kingma and Ba).
 * The hyperparameters are doubles; each derived scalar is computed in double
 * and rounded once to fp32:
 *   b1 = beta1, b2 = beta2, omb1 = 1 - beta1, omb2 = 1 - beta2,
 *   decay = 1 - lr * wd, step_size = lr / (1 - beta1^t),
 *   bc2_sqrt = sqrt(1 - beta2^t), epsf = eps;
 * then per element, every operation one fp32 rounding, in this order:
 *   p = p * decay;  m = b1 * m + omb1 * g;  v = b2 * v + (omb2 * g) * g;
 *   den = sqrt(v) / bc2_sqrt + epsf;  p = p - step_size * (m / den).
 * The pages name Adam's two moments as the optimizer state (Ling 2.0 FP8
 * blog, "FP8 Optimizer"); the step itself is the textbook one. */
void orc_adamw_step(int64_t n, float* p, const float* g, float* m, float* v, double lr, double beta1,
                    double beta2, double eps, double wd, int64_t t)
{
    const float b1 = (float)beta1, b2 = (float)beta2;
    const float omb1 = (float)(1.0 - beta1);
    const float omb2 = (float)(1.0 - beta2);
    const float decay = (float)(1.0 - lr * wd);
    const float step_size = (float)(lr / (1.0 - pow(beta1, (double)t)));
    const float bc2_sqrt = (float)sqrt(1.0 - pow(beta2, (double)t));
    const float epsf = (float)eps;
    for (int64_t i = 0; i < n; ++i) {
        float pi = p[i] * decay;
        float a = b1 * m[i];
        float b = omb1 * g[i];
        float mi = a + b;
        float c = b2 * v[i];
        float d = omb2 * g[i];
        float e = d * g[i];
        float vi = c + e;
        float r = sqrtf(vi);
        float q = r / bc2_sqrt;
        float den = q + epsf;
        float u = mi / den;
        float w = step_size * u;
        p[i] = pi - w;
        m[i] = mi;
        v[i] = vi;
    }
}

/* The same step with both moments held as E4M3 codes plus one fp32 scale per
 * 128 consecutive elements (the fine-grained compression of the moments in
 * the Ling 2.0 FP8 blog, "FP8 Optimizer", which points to block-wise
 * quantization): decode (code value times its block's scale), the fp32 step
 * above, and the 1x128 tile quantization of the new moments
 * (orc_quant_tiles on the flat vector).  mq/vq: n codes; ms/vs:
 * ceil(n/128) scales; all updated in place. */
void orc_adamw_fp8_step(int64_t n, float* p, const float* g, uint8_t* mq, float* ms, uint8_t* vq,
                        float* vs, double lr, double beta1, double beta2, double eps, double wd, int64_t t)
{
    if (n <= 0)
        return;
    float* m = (float*)malloc(sizeof(float) * (size_t)n);
    float* v = (float*)malloc(sizeof(float) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) {
        m[i] = orc_e4m3_decode(mq[i]) * ms[i / 128];
        v[i] = orc_e4m3_decode(vq[i]) * vs[i / 128];
    }
    orc_adamw_step(n, p, g, m, v, lr, beta1, beta2, eps, wd, t);
    orc_quant_tiles(m, 1, n, 1, 128, mq, ms);
    orc_quant_tiles(v, 1, n, 1, 128, vq, vs);
    free(m);
    free(v);
}

/* fp32 -> bf16 bit pattern, round to nearest even (finite inputs). */
void orc_f32_to_bf16(const float* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, &x[i], 4);
        uint32_t lower = u & 0xFFFFu;
        uint32_t upper = u >> 16;
        if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
            upper += 1u;
        out[i] = (uint16_t)upper;
    }
}

/* Number of elements with x != 0 whose code decodes to zero (underflow),
 * and the number of non-zero x.  Underflow as defined in the Ling 2.0 FP8
 * blog ("where is error introduced"): a non-zero element that becomes 0
 * after quantization. */
void orc_underflow_count(const float* x, const uint8_t* q, int64_t n,
                         int64_t* n_underflow, int64_t* n_nonzero)
{
    int64_t u = 0, nz = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (x[i] != 0.0f) {
            nz++;
            if ((q[i] & 0x7F) == 0)
                u++;
        }
    }
    *n_underflow = u;
    *n_nonzero = nz;
}
