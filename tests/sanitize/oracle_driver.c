/* Runs every function of oracle/fp8q_oracle.c on small, ragged inputs (tile
 * edges, one-element tiles, zero and subnormal tiles, K not a multiple of
 * 128, row subsets) so that a build with -fsanitize=address,undefined sees
 * each loop bound and each allocation.  Besides running clean it checks a few
 * facts that hold for any correct build: decode then encode is the identity
 * on the 254 finite codes, a tile holding 448 gets s = 1, the fp32 GEMM lies
 * within the rounding bound R * 2^-20 of the fp64 one, and the FP8-moment
 * AdamW step leaves finite parameters.  Exit status 0 iff all hold. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

float orc_e4m3_decode(uint8_t c);
uint8_t orc_e4m3_encode(float v);
void orc_decode_array(const uint8_t* c, int64_t n, float* out);
void orc_encode_array(const float* v, int64_t n, uint8_t* out);
void orc_quant_tiles(const float* x, int64_t rows, int64_t cols, int64_t tr, int64_t tc, uint8_t* q, float* s);
int orc_pow2_exponent(float amax);
void orc_quant_tiles_pow2(const float* x, int64_t rows, int64_t cols, int64_t tr, int64_t tc, uint8_t* q,
                          uint8_t* ebyte);
void orc_e8m0_decode_array(const uint8_t* b, int64_t n, float* out);
void orc_gemm_f32(int64_t M, int64_t N, int64_t K, const uint8_t* A, const float* SA, const uint8_t* B,
                  const float* SB, const int64_t* rows, int64_t nrows, float* C);
void orc_gemm_f64(int64_t M, int64_t N, int64_t K, const uint8_t* A, const float* SA, const uint8_t* B,
                  const float* SB, const int64_t* rows, int64_t nrows, double* C, double* R);
void orc_adamw_step(int64_t n, float* p, const float* g, float* m, float* v, double lr, double beta1,
                    double beta2, double eps, double wd, int64_t t);
void orc_adamw_fp8_step(int64_t n, float* p, const float* g, uint8_t* mq, float* ms, uint8_t* vq, float* vs,
                        double lr, double beta1, double beta2, double eps, double wd, int64_t t);
void orc_f32_to_bf16(const float* x, int64_t n, uint16_t* out);
void orc_underflow_count(const float* x, const uint8_t* q, int64_t n, int64_t* n_underflow, int64_t* n_nonzero);

static int failures = 0;
#define CHECK(cond, ...)                       \
    do {                                       \
        if (!(cond)) {                         \
            fprintf(stderr, __VA_ARGS__);      \
            fprintf(stderr, "\n");             \
            ++failures;                        \
        }                                      \
    } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double urand(void) /* xorshift64*, uniform in [0, 1) */
{
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return (double)((rng * 0x2545F4914F6CDD1Dull) >> 11) * 0x1p-53;
}
static float nrand(void) { return (float)(urand() * 2.0 - 1.0); }

static void* xmalloc(size_t n)
{
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static void codec(void)
{
    uint8_t codes[256];
    float vals[256];
    for (int c = 0; c < 256; ++c) codes[c] = (uint8_t)c;
    orc_decode_array(codes, 256, vals);
    uint8_t back[256];
    orc_encode_array(vals, 256, back);
    for (int c = 0; c < 256; ++c) {
        if ((c & 0x7F) == 0x7F) continue; /* NaN codes */
        CHECK(back[c] == c, "encode(decode(0x%02x)) = 0x%02x", c, back[c]);
        CHECK(orc_e4m3_encode(vals[c]) == c, "scalar encode of 0x%02x", c);
    }
    CHECK(orc_e4m3_encode(1e30f) == 0x7E && orc_e4m3_encode(-1e30f) == 0xFE, "saturation");
    CHECK(orc_e4m3_encode(-0.0f) == 0x80, "signed zero");
}

static void tiles(int64_t rows, int64_t cols, int64_t tr, int64_t tc)
{
    const int64_t n = rows * cols;
    const int64_t TR = (rows + tr - 1) / tr, TC = (cols + tc - 1) / tc;
    float* x = xmalloc(sizeof(float) * n);
    for (int64_t i = 0; i < n; ++i) {
        const double u = urand();
        x[i] = u < 0.05 ? 0.0f : u < 0.1 ? 1e-42f * nrand() : nrand() * (float)ldexp(1.0, (int)(urand() * 40) - 20);
    }
    if (n) x[0] = 448.0f; /* first tile: amax 448 unless a larger value shares it */
    uint8_t* q = xmalloc(n);
    float* s = xmalloc(sizeof(float) * TR * TC);
    uint8_t* e = xmalloc(TR * TC);
    orc_quant_tiles(x, rows, cols, tr, tc, q, s);
    orc_quant_tiles_pow2(x, rows, cols, tr, tc, q, e);
    float* se = xmalloc(sizeof(float) * TR * TC);
    orc_e8m0_decode_array(e, TR * TC, se);
    for (int64_t i = 0; i < TR * TC; ++i) {
        CHECK(s[i] >= 0.0f && isfinite(s[i]), "scale %lld", (long long)i);
        CHECK(se[i] > 0.0f, "pow2 scale %lld", (long long)i);
    }
    int64_t u = 0, nz = 0;
    orc_underflow_count(x, q, n, &u, &nz);
    CHECK(u >= 0 && u <= nz && nz <= n, "underflow count");
    uint16_t* b = xmalloc(sizeof(uint16_t) * n);
    orc_f32_to_bf16(x, n, b);
    free(x);
    free(q);
    free(s);
    free(e);
    free(se);
    free(b);
}

static void s_one(void)
{
    float x[128];
    for (int i = 0; i < 128; ++i) x[i] = (float)(i % 17) - 8.0f;
    x[5] = -448.0f;
    uint8_t q[128];
    float s;
    orc_quant_tiles(x, 1, 128, 1, 128, q, &s);
    CHECK(s == 1.0f, "tile with 448: s = %g", s);
}

static void gemm(int64_t M, int64_t N, int64_t K)
{
    const int64_t KB = (K + 127) / 128;
    uint8_t* A = xmalloc(M * K);
    uint8_t* B = xmalloc(N * K);
    float* SA = xmalloc(sizeof(float) * M * KB);
    float* SB = xmalloc(sizeof(float) * N * KB);
    for (int64_t i = 0; i < M * K; ++i) { A[i] = (uint8_t)(urand() * 254); if ((A[i] & 0x7F) == 0x7F) A[i] ^= 1; }
    for (int64_t i = 0; i < N * K; ++i) { B[i] = (uint8_t)(urand() * 254); if ((B[i] & 0x7F) == 0x7F) B[i] ^= 1; }
    for (int64_t i = 0; i < M * KB; ++i) SA[i] = (float)(urand() * 1e-2 + 1e-4);
    for (int64_t i = 0; i < N * KB; ++i) SB[i] = (float)(urand() * 1e-2 + 1e-4);
    int64_t rows[3] = {M - 1, 0, M / 2};
    float* C = xmalloc(sizeof(float) * M * N);
    double* C64 = xmalloc(sizeof(double) * M * N);
    double* R = xmalloc(sizeof(double) * M * N);
    orc_gemm_f32(M, N, K, A, SA, B, SB, NULL, M, C);
    orc_gemm_f64(M, N, K, A, SA, B, SB, NULL, M, C64, R);
    for (int64_t i = 0; i < M * N; ++i)
        CHECK(fabs((double)C[i] - C64[i]) <= R[i] * 0x1p-20 + 1e-37, "gemm %lldx%lldx%lld at %lld",
              (long long)M, (long long)N, (long long)K, (long long)i);
    float* Cr = xmalloc(sizeof(float) * 3 * N);
    double* Cr64 = xmalloc(sizeof(double) * 3 * N);
    double* Rr = xmalloc(sizeof(double) * 3 * N);
    orc_gemm_f32(M, N, K, A, SA, B, SB, rows, 3, Cr);
    orc_gemm_f64(M, N, K, A, SA, B, SB, rows, 3, Cr64, Rr);
    for (int i = 0; i < 3; ++i)
        for (int64_t n = 0; n < N; ++n)
            CHECK(Cr[i * N + n] == C[rows[i] * N + n], "row subset %d", i);
    free(A); free(B); free(SA); free(SB); free(C); free(C64); free(R); free(Cr); free(Cr64); free(Rr);
}

static void adam(int64_t n)
{
    const int64_t nb = (n + 127) / 128;
    float* p = xmalloc(sizeof(float) * n);
    float* p32 = xmalloc(sizeof(float) * n);
    float* g = xmalloc(sizeof(float) * n);
    float* m = xmalloc(sizeof(float) * n);
    float* v = xmalloc(sizeof(float) * n);
    uint8_t* mq = xmalloc(n);
    uint8_t* vq = xmalloc(n);
    float* ms = xmalloc(sizeof(float) * nb);
    float* vs = xmalloc(sizeof(float) * nb);
    for (int64_t i = 0; i < n; ++i) {
        p[i] = p32[i] = nrand();
        g[i] = 1e-3f * nrand();
        m[i] = v[i] = 0.0f;
        mq[i] = vq[i] = 0;
    }
    for (int64_t i = 0; i < nb; ++i) ms[i] = vs[i] = 0.0f;
    for (int t = 1; t <= 3; ++t) {
        orc_adamw_step(n, p32, g, m, v, 1e-3, 0.9, 0.999, 1e-8, 0.1, t);
        orc_adamw_fp8_step(n, p, g, mq, ms, vq, vs, 1e-3, 0.9, 0.999, 1e-8, 0.1, t);
    }
    for (int64_t i = 0; i < n; ++i)
        CHECK(isfinite(p[i]) && isfinite(p32[i]), "adam parameter %lld", (long long)i);
    free(p);
    free(p32); free(g); free(m); free(v); free(mq); free(vq); free(ms); free(vs);
}

int main(void)
{
    codec();
    s_one();
    const int64_t shapes[][2] = {{1, 1}, {1, 129}, {3, 128}, {130, 257}, {256, 128}, {129, 1}};
    for (unsigned i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i) {
        tiles(shapes[i][0], shapes[i][1], 1, 128);
        tiles(shapes[i][0], shapes[i][1], 128, 128);
        tiles(shapes[i][0], shapes[i][1], shapes[i][0], shapes[i][1]);
    }
    gemm(1, 1, 1);
    gemm(3, 5, 127);
    gemm(17, 33, 129);
    gemm(9, 130, 384);
    adam(1);
    adam(300);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle driver: all checks passed\n");
    return 0;
}
