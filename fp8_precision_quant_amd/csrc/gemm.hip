// Host launchers of the block-scaled FP8 GEMM for gfx950 (CDNA4 FP8 MFMA).
//
//   C[m][n] = sum_kb SA(m,kb) * SB(n,kb) * sum_{k in chunk kb} dec(A[m][k]) * dec(B^[n][k])
//
// The FP8 Linear of the Ling 2.0 FP8 blog (BF16 Linear -> FP8 tensor + scale
// tensor -> FP8 GEMM with an FP32 accumulator, "where is error introduced"),
// with the fine-grained scales of its "fine-grained quantization" section:
// activations / gradients 1x128, weights 128x128 ("FP8-RL" article, 一).
// The kernel itself is in gemm_nk.hip.  It addresses every operand through
// 32-bit buffer offsets, so a dense call whose operands span 2 GiB or more is
// cut here into launches over slices of M (rows of A, their scales and of C)
// and, for a [N][K] B, of N (rows of B, their scales and columns of C); each
// slice is the same GEMM on a sub-block of the output.
#include <algorithm>
#include <atomic>

#include "fp8q_device.h"
#include "fp8q_internal.h"
#include "gemm_common.h"

namespace fp8q {

constexpr int BK = 128;

// Compute-unit count of the current device, cached per device (the query
// is not free).  Falls back to 256 (MI355X) if the query fails.
int device_cu_count()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        n = 256;
    }
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

namespace {

// Largest multiple of `unit` that is at most v (0 if v < unit).
int64_t floor_to(int64_t v, int64_t unit) { return v < unit ? 0 : v - v % unit; }

// Calls launch(slice) for every slice of the dense GEMM g such that each
// slice's operands span less than 2 GiB.  `sbytes` is the size of one scale
// (4 for fp32, 1 for E8M0 bytes), `cbytes` that of one output element.
// Returns false (nothing launched) if no slicing fits: a [K][N] B of 2 GiB or
// more, or a single 256-row slice that is already too large.
template <typename F>
bool for_each_slice(const GemmArgs& g, int sa_mode, int sb_mode, bool b_kn, int sbytes, int cbytes,
                    F&& launch)
{
    const int64_t lim = ((int64_t)1 << 31) - 1;
    const int64_t step = 256;   // a multiple of both tile edges and of the 128-wide scale blocks
    // rows of A (and of its row scales) per launch; the kernel reads up to a
    // tile of rows past the end of each operand, hence the margins
    int64_t rows_m = lim / std::max<int64_t>(g.lda, 1);
    if (sa_mode == SA_ROW) rows_m = std::min(rows_m, lim / std::max<int64_t>(g.ldsa * sbytes, 1));
    rows_m -= 2 * step;
    rows_m = g.M <= rows_m ? g.M : floor_to(rows_m, step);
    // rows of [N][K] B (and of its scale grid) per launch
    int64_t rows_n = g.N;
    if (!b_kn) {
        int64_t r = lim / std::max<int64_t>(g.ldb, 1);
        if (sb_mode == SB_ROW) r = std::min(r, lim / std::max<int64_t>(g.ldsb * sbytes, 1));
        if (sb_mode == SB_BLOCK) r = std::min(r, (lim / std::max<int64_t>(g.ldsb * sbytes, 1) - 2) * 128);
        r -= 2 * step;
        rows_n = g.N <= r ? g.N : floor_to(r, step);
    }
    if (rows_m <= 0 || rows_n <= 0) return false;
    for (int64_t m0 = 0; m0 < g.M; m0 += rows_m) {
        for (int64_t n0 = 0; n0 < g.N; n0 += rows_n) {
            GemmArgs s = g;
            s.M = std::min(rows_m, g.M - m0);
            s.N = std::min(rows_n, g.N - n0);
            s.a = g.a + m0 * g.lda;
            if (sa_mode == SA_ROW)
                s.sa = reinterpret_cast<const float*>(reinterpret_cast<const char*>(g.sa) + m0 * g.ldsa * sbytes);
            if (!b_kn) {
                s.b = g.b + n0 * g.ldb;
                const int64_t sb_rows = sb_mode == SB_ROW ? n0 : sb_mode == SB_BLOCK ? n0 / 128 : 0;
                s.sb = reinterpret_cast<const float*>(reinterpret_cast<const char*>(g.sb) + sb_rows * g.ldsb * sbytes);
            } else {
                // [K][N] B: the columns n0.. of every K row, their 128-wide scale blocks
                s.b = g.b + n0;
                if (sb_mode == SB_BLOCK)
                    s.sb = reinterpret_cast<const float*>(reinterpret_cast<const char*>(g.sb) + (n0 / 128) * sbytes);
            }
            s.c = reinterpret_cast<char*>(g.c) + (m0 * g.ldc + n0) * cbytes;
            if (g.cs) s.cs = g.cs + m0 * g.ldcs + n0 / 128;
            if (!launch(s)) return false;
        }
    }
    return true;
}

int sa_mode_of(int kind) { return kind == FP8Q_ROW_1x128 ? SA_ROW : SA_TENSOR; }
int sb_mode_of(int kind)
{
    return kind == FP8Q_ROW_1x128 ? SB_ROW : (kind == FP8Q_BLOCK_128x128 ? SB_BLOCK : SB_TENSOR);
}

}  // namespace

bool launch_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const float* sa,
                 int64_t ldsa, int sa_kind, const uint8_t* b, int64_t ldb, int b_layout,
                 const float* sb, int64_t ldsb, int sb_kind, void* c, int64_t ldc, int c_dtype,
                 hipStream_t st)
{
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.a = a; g.lda = lda; g.sa = sa; g.ldsa = ldsa;
    g.b = b; g.ldb = ldb; g.sb = sb; g.ldsb = ldsb;
    g.c = c; g.ldc = ldc;
    g.KB = (int)((K + BK - 1) / BK);
    g.num_cus = device_cu_count();
    const bool kn = b_layout == FP8Q_B_KN;
    const int sa_mode = sa_mode_of(sa_kind), sb_mode = sb_mode_of(sb_kind);
    const int out = c_dtype == FP8Q_BF16 ? OUT_BF16 : OUT_F32;
    return for_each_slice(g, sa_mode, sb_mode, kn, 4, c_dtype == FP8Q_BF16 ? 2 : 4, [&](const GemmArgs& s) {
        return launch_gemm_nk(s, sa_mode, sb_mode, kn, out, st);
    });
}

bool launch_gemm_e4m3(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const float* sa,
                      int64_t ldsa, int sa_kind, const uint8_t* b, int64_t ldb, int b_layout,
                      const float* sb, int64_t ldsb, int sb_kind, uint8_t* q, int64_t ldq, float* s,
                      int64_t lds, hipStream_t st)
{
    if (sb_kind == FP8Q_ROW_1x128) return false;   // row-scaled B: fp32/bf16 output only
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.a = a; g.lda = lda; g.sa = sa; g.ldsa = ldsa;
    g.b = b; g.ldb = ldb; g.sb = sb; g.ldsb = ldsb;
    g.c = q; g.ldc = ldq;
    g.cs = s; g.ldcs = lds;
    g.KB = (int)((K + BK - 1) / BK);
    g.num_cus = device_cu_count();
    const bool kn = b_layout == FP8Q_B_KN;
    const int sa_mode = sa_mode_of(sa_kind), sb_mode = sb_mode_of(sb_kind);
    return for_each_slice(g, sa_mode, sb_mode, kn, 4, 1, [&](const GemmArgs& sl) {
        return launch_gemm_nk(sl, sa_mode, sb_mode, kn, OUT_E4M3, st);
    });
}

bool launch_gemm_e8m0(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const uint8_t* ea,
                      int64_t ldea, const uint8_t* b, int64_t ldb, int b_layout, const uint8_t* eb,
                      int64_t ldeb, int eb_kind, void* c, int64_t ldc, int c_dtype, hipStream_t st)
{
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.a = a; g.lda = lda; g.sa = reinterpret_cast<const float*>(ea); g.ldsa = ldea;
    g.b = b; g.ldb = ldb; g.sb = reinterpret_cast<const float*>(eb); g.ldsb = ldeb;
    g.c = c; g.ldc = ldc;
    g.KB = (int)((K + BK - 1) / BK);
    g.num_cus = device_cu_count();
    const bool kn = b_layout == FP8Q_B_KN;
    const int sb_mode = eb_kind == FP8Q_ROW_1x128 ? SB_ROW : SB_BLOCK;
    const bool bf = c_dtype == FP8Q_BF16;
    return for_each_slice(g, SA_ROW, sb_mode, kn, 1, bf ? 2 : 4, [&](const GemmArgs& s) {
        return launch_gemm_nk_e8m0(s, sb_mode, kn, bf, st);
    });
}

bool launch_grouped_gemm(int64_t G, int64_t M_pad, int64_t N, int64_t K, const uint8_t* a,
                         int64_t lda, const float* sa, int64_t ldsa, const int32_t* offsets,
                         const uint8_t* b, const float* sb, void* c, int64_t ldc, int c_dtype,
                         hipStream_t st)
{
    GemmArgs g{};
    g.M = M_pad; g.N = N; g.K = K;
    g.a = a; g.lda = lda; g.sa = sa; g.ldsa = ldsa;
    g.b = b; g.ldb = K; g.sb = sb;
    g.KB = (int)((K + BK - 1) / BK);
    g.ldsb = g.KB;
    g.c = c; g.ldc = ldc;
    g.offsets = offsets;
    g.G = (int)G;
    g.b_group_stride = N * K;
    g.sb_group_stride = ((N + 127) / 128) * (int64_t)g.KB;
    g.num_cus = device_cu_count();
    if (launch_grouped_gemm_w4(g, c_dtype == FP8Q_BF16, false, st)) return true;
    return launch_grouped_gemm_nk(g, c_dtype == FP8Q_BF16, false, st);
}

bool launch_grouped_gemm_e4m3(int64_t G, int64_t M_pad, int64_t N, int64_t K, const uint8_t* a,
                              int64_t lda, const float* sa, int64_t ldsa, const int32_t* offsets,
                              const uint8_t* b, const float* sb, uint8_t* q, int64_t ldq, float* s,
                              int64_t lds, hipStream_t st)
{
    GemmArgs g{};
    g.M = M_pad; g.N = N; g.K = K;
    g.a = a; g.lda = lda; g.sa = sa; g.ldsa = ldsa;
    g.b = b; g.ldb = K; g.sb = sb;
    g.KB = (int)((K + BK - 1) / BK);
    g.ldsb = g.KB;
    g.c = q; g.ldc = ldq;
    g.cs = s; g.ldcs = lds;
    g.offsets = offsets;
    g.G = (int)G;
    g.b_group_stride = N * K;
    g.sb_group_stride = ((N + 127) / 128) * (int64_t)g.KB;
    g.num_cus = device_cu_count();
    return launch_grouped_gemm_w4_e4m3(g, st);
}

bool launch_grouped_gemm_dgrad(int64_t G, int64_t M_pad, int64_t N, int64_t K, const uint8_t* a,
                               int64_t lda, const float* sa, int64_t ldsa, const int32_t* offsets,
                               const uint8_t* w, const float* sw, void* c, int64_t ldc, int c_dtype,
                               hipStream_t st)
{
    // dX[m][k] = sum_n dY[m][n] W_e[n][k]: contraction over W's rows, so in
    // GEMM terms M = M_pad, N = K, K = N and B is W_e read as stored ([K][N])
    GemmArgs g{};
    g.M = M_pad; g.N = K; g.K = N;
    g.a = a; g.lda = lda; g.sa = sa; g.ldsa = ldsa;
    g.b = w; g.ldb = K; g.sb = sw;
    g.KB = (int)((N + BK - 1) / BK);
    g.ldsb = (K + 127) / 128;
    g.c = c; g.ldc = ldc;
    g.offsets = offsets;
    g.G = (int)G;
    g.b_group_stride = N * K;
    g.sb_group_stride = (int64_t)g.KB * g.ldsb;
    g.num_cus = device_cu_count();
    if (launch_grouped_gemm_w4(g, c_dtype == FP8Q_BF16, true, st)) return true;
    return launch_grouped_gemm_nk(g, c_dtype == FP8Q_BF16, true, st);
}

bool launch_grouped_gemm_wgrad(int64_t G, int64_t M_pad, int64_t N, int64_t K, const uint8_t* a,
                               int64_t lda, const float* sa, int64_t ldsa, const uint8_t* b,
                               int64_t ldb, const float* sb, int64_t ldsb, const int32_t* offsets,
                               float* c, int64_t ldc, hipStream_t st)
{
    // dW_e[n][k] = sum over the group's tokens t of dYT[n][t] XT[k][t]: rows
    // of A and B are N and K, the contraction runs over the group's tokens
    GemmArgs g{};
    g.M = N; g.N = K; g.K = M_pad;
    g.a = a; g.lda = lda; g.sa = sa; g.ldsa = ldsa;
    g.b = b; g.ldb = ldb; g.sb = sb; g.ldsb = ldsb;
    g.KB = (int)(M_pad / BK);
    g.c = c; g.ldc = ldc;
    g.offsets = offsets;
    g.G = (int)G;
    g.c_group_stride = N * ldc;
    g.num_cus = device_cu_count();
    return launch_grouped_wgrad_w4(g, st);
}

}  // namespace fp8q
