/* Exhaustive pin for an E4M3 encoder: for every one of the 2^32 fp32 bit
 * patterns, the expected code is found by searching a table of all
 * representable E4M3 magnitudes for the nearest one (ties to the code with an
 * even mantissa bit), with magnitudes above the largest finite value (448)
 * saturating.  The table is built here from the format definition alone
 * (4 exponent bits with bias 7, 3 mantissa bits, subnormals, top code NaN);
 * it shares nothing with the encoder under test, which is passed in as a
 * function pointer. */
#include <math.h>
#include <stdint.h>
#include <string.h>

typedef uint8_t (*enc_fn)(float);

static double mag[127]; /* value of code c for c = 0x00..0x7E, increasing */

static void build_table(void)
{
    for (int c = 0; c < 127; ++c) {
        int e = c >> 3, m = c & 7;
        mag[c] = e == 0 ? m * 0x1p-9 : (1.0 + m * 0.125) * ldexp(1.0, e - 7);
    }
}

static uint8_t nearest(float v)
{
    uint32_t u;
    memcpy(&u, &v, 4);
    uint8_t sign = (uint8_t)((u >> 31) << 7);
    double a = fabs((double)v);
    if (a > mag[126])
        return sign | 126;
    int lo = 0, hi = 126; /* largest c with mag[c] <= a */
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (mag[mid] <= a) lo = mid; else hi = mid - 1;
    }
    if (lo == 126 || mag[lo] == a)
        return sign | (uint8_t)lo;
    double d0 = a - mag[lo], d1 = mag[lo + 1] - a;
    int c;
    if (d0 < d1) c = lo;
    else if (d1 < d0) c = lo + 1;
    else c = (lo % 2 == 0) ? lo : lo + 1;
    return sign | (uint8_t)c;
}

/* Returns the number of finite patterns where enc disagrees; writes the
 * first disagreeing pattern to *first_bad (or 0xFFFFFFFF if none). */
int64_t count_mismatches(enc_fn enc, uint32_t* first_bad)
{
    build_table();
    int64_t bad = 0;
    uint32_t first = 0xFFFFFFFFu;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t i = 0; i <= 0xFFFFFFFFLL; ++i) {
        uint32_t u = (uint32_t)i;
        float v;
        memcpy(&v, &u, 4);
        if (isnan(v))
            continue;
        if (enc(v) != nearest(v)) {
            bad++;
#pragma omp critical
            if (u < first) first = u;
        }
    }
    *first_bad = first;
    return bad;
}

/* The expected code for one value, for spot checks. */
uint8_t nearest_code(float v)
{
    build_table();
    return nearest(v);
}
