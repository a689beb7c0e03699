// C ABI of libfp8q: argument validation, device check, dispatch.
//
// Every entry point validates all of its arguments on the host before it
// enqueues anything, never allocates or synchronizes (except in the debug
// mode FP8Q_CHECK=1), and reports a pending launch error as FP8Q_ERR_LAUNCH.  Operation semantics are documented in
// include/fp8q.h.
#include <atomic>
#include <cmath>
#include <cstring>

#include "fp8q_internal.h"

namespace {

constexpr int64_t kTile = 128;
constexpr int64_t kMaxIndex = (int64_t)1 << 31;
// grouped GEMMs keep the group offsets in LDS
constexpr int64_t kMaxGroups = 1024;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(int dtype) { return dtype == FP8Q_BF16 ? 2 : 4; }

bool dtype_ok(int d) { return d == FP8Q_F32 || d == FP8Q_BF16; }

// Per-device cache: 0 = unknown, 1 = gfx950, 2 = other / query failed.
std::atomic<int> g_arch_state[64];

int check_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return FP8Q_ERR_DEVICE;
    }
    if (dev >= 64) return FP8Q_ERR_DEVICE;
    int st = g_arch_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            st = 2;
        } else {
            st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        }
        g_arch_state[dev].store(st, std::memory_order_release);
    }
    return st == 1 ? FP8Q_OK : FP8Q_ERR_DEVICE;
}

// A pending launch error; with FP8Q_CHECK=1 the stream is also synchronized
// so that an error of the work itself is reported by the call that enqueued it.
int launch_status(hipStream_t stream)
{
    if (hipGetLastError() != hipSuccess) return FP8Q_ERR_LAUNCH;
    if (fp8q::debug_checks_enabled() && hipStreamSynchronize(stream) != hipSuccess) {
        (void)hipGetLastError();
        return FP8Q_ERR_LAUNCH;
    }
    return FP8Q_OK;
}

// FP8Q_CHECK=1: the group offsets are checked on the device first.
int offsets_status(const int32_t* offsets, int64_t G, int64_t M_pad, hipStream_t stream)
{
    if (!fp8q::debug_checks_enabled()) return FP8Q_OK;
    return fp8q::check_group_offsets(offsets, G, M_pad, stream);
}

}  // namespace

extern "C" {

const char* fp8q_status_string(int status)
{
    switch (status) {
    case FP8Q_OK: return "FP8Q_OK";
    case FP8Q_ERR_NULL: return "FP8Q_ERR_NULL: a required pointer is NULL";
    case FP8Q_ERR_SHAPE: return "FP8Q_ERR_SHAPE: invalid size, leading dimension or grid size";
    case FP8Q_ERR_ALIGN: return "FP8Q_ERR_ALIGN: pointer or row stride not 16-byte aligned";
    case FP8Q_ERR_UNSUPPORTED: return "FP8Q_ERR_UNSUPPORTED: unsupported dtype, scale kind or layout";
    case FP8Q_ERR_DEVICE: return "FP8Q_ERR_DEVICE: current device is not gfx950 or not available";
    case FP8Q_ERR_LAUNCH: return "FP8Q_ERR_LAUNCH: kernel launch failed";
    default: return "unknown fp8q status";
    }
}

int fp8_quant_blockwise(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                        int kind, uint8_t* q, int64_t ldq, float* s, int64_t lds, hipStream_t stream)
{
    if (!dtype_ok(x_dtype)) return FP8Q_ERR_UNSUPPORTED;
    if (kind != FP8Q_ROW_1x128 && kind != FP8Q_BLOCK_128x128 && kind != FP8Q_TENSOR)
        return FP8Q_ERR_UNSUPPORTED;
    if (rows < 0 || cols < 0) return FP8Q_ERR_SHAPE;
    if (rows == 0 || cols == 0) return FP8Q_OK;
    if (!x || !q || !s) return FP8Q_ERR_NULL;
    const int64_t tiles_c = cdiv(cols, kTile);
    if (ldx < cols || ldq < cols) return FP8Q_ERR_SHAPE;
    if (kind != FP8Q_TENSOR && lds < tiles_c) return FP8Q_ERR_SHAPE;
    if (kind == FP8Q_ROW_1x128 && rows * tiles_c >= kMaxIndex) return FP8Q_ERR_SHAPE;
    if (kind == FP8Q_BLOCK_128x128 && cdiv(rows, kTile) * tiles_c >= kMaxIndex) return FP8Q_ERR_SHAPE;
    if (kind == FP8Q_TENSOR && rows * cdiv(cols, 8) >= kMaxIndex) return FP8Q_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(q) || (ldx * elem_size(x_dtype)) % 16 || ldq % 16)
        return FP8Q_ERR_ALIGN;
    if (kind == FP8Q_TENSOR && (reinterpret_cast<uintptr_t>(s) & 3u)) return FP8Q_ERR_ALIGN;
    int st = check_device();
    if (st != FP8Q_OK) return st;
    fp8q::launch_quant_blockwise(x, x_dtype, rows, cols, ldx, kind, q, ldq, s, lds,
                                 stream);
    return launch_status(stream);
}

int fp8_quant_transpose(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                        uint8_t* q_row, int64_t ldq_row, float* s_row, int64_t lds_row,
                        uint8_t* q_colT, int64_t ldq_colT, float* s_colT, int64_t lds_colT,
                        hipStream_t stream)
{
    if (!dtype_ok(x_dtype)) return FP8Q_ERR_UNSUPPORTED;
    if (rows < 0 || cols < 0) return FP8Q_ERR_SHAPE;
    if (rows == 0 || cols == 0) return FP8Q_OK;
    const bool want_row = q_row || s_row;
    const bool want_col = q_colT || s_colT;
    if (!x) return FP8Q_ERR_NULL;
    if (want_row && (!q_row || !s_row)) return FP8Q_ERR_NULL;
    if (want_col && (!q_colT || !s_colT)) return FP8Q_ERR_NULL;
    if (!want_row && !want_col) return FP8Q_OK;
    if (ldx < cols) return FP8Q_ERR_SHAPE;
    if (want_row && (ldq_row < cols || lds_row < cdiv(cols, kTile))) return FP8Q_ERR_SHAPE;
    if (want_col && (ldq_colT < rows || lds_colT < cdiv(rows, kTile))) return FP8Q_ERR_SHAPE;
    if (cdiv(rows, kTile) * cdiv(cols, kTile) >= kMaxIndex) return FP8Q_ERR_SHAPE;
    if (!aligned16(x) || (ldx * elem_size(x_dtype)) % 16) return FP8Q_ERR_ALIGN;
    if (want_row && (!aligned16(q_row) || ldq_row % 16)) return FP8Q_ERR_ALIGN;
    if (want_col && (!aligned16(q_colT) || ldq_colT % 16)) return FP8Q_ERR_ALIGN;
    int st = check_device();
    if (st != FP8Q_OK) return st;
    fp8q::launch_quant_transpose(x, x_dtype, rows, cols, ldx, want_row ? q_row : nullptr, ldq_row,
                                 s_row, lds_row, want_col ? q_colT : nullptr, ldq_colT, s_colT,
                                 lds_colT, stream);
    return launch_status(stream);
}

int fp8_quant_blockwise_e8m0(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                             int kind, uint8_t* q, int64_t ldq, uint8_t* e, int64_t lde, hipStream_t stream)
{
    if (!dtype_ok(x_dtype)) return FP8Q_ERR_UNSUPPORTED;
    if (kind != FP8Q_ROW_1x128 && kind != FP8Q_BLOCK_128x128) return FP8Q_ERR_UNSUPPORTED;
    if (rows < 0 || cols < 0) return FP8Q_ERR_SHAPE;
    if (rows == 0 || cols == 0) return FP8Q_OK;
    if (!x || !q || !e) return FP8Q_ERR_NULL;
    const int64_t tiles_c = cdiv(cols, kTile);
    if (ldx < cols || ldq < cols || lde < tiles_c) return FP8Q_ERR_SHAPE;
    if (kind == FP8Q_ROW_1x128 && rows * tiles_c >= kMaxIndex) return FP8Q_ERR_SHAPE;
    if (kind == FP8Q_BLOCK_128x128 && cdiv(rows, kTile) * tiles_c >= kMaxIndex) return FP8Q_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(q) || (ldx * elem_size(x_dtype)) % 16 || ldq % 16)
        return FP8Q_ERR_ALIGN;
    int st = check_device();
    if (st != FP8Q_OK) return st;
    fp8q::launch_quant_blockwise_e8m0(x, x_dtype, rows, cols, ldx, kind, q, ldq, e, lde,
                                      stream);
    return launch_status(stream);
}

int fp8_quant_transpose_e8m0(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* q_row, int64_t ldq_row, uint8_t* e_row, int64_t lde_row,
                             uint8_t* q_colT, int64_t ldq_colT, uint8_t* e_colT, int64_t lde_colT,
                             hipStream_t stream)
{
    if (!dtype_ok(x_dtype)) return FP8Q_ERR_UNSUPPORTED;
    if (rows < 0 || cols < 0) return FP8Q_ERR_SHAPE;
    if (rows == 0 || cols == 0) return FP8Q_OK;
    const bool want_row = q_row || e_row;
    const bool want_col = q_colT || e_colT;
    if (!x) return FP8Q_ERR_NULL;
    if (want_row && (!q_row || !e_row)) return FP8Q_ERR_NULL;
    if (want_col && (!q_colT || !e_colT)) return FP8Q_ERR_NULL;
    if (!want_row && !want_col) return FP8Q_OK;
    if (ldx < cols) return FP8Q_ERR_SHAPE;
    if (want_row && (ldq_row < cols || lde_row < cdiv(cols, kTile))) return FP8Q_ERR_SHAPE;
    if (want_col && (ldq_colT < rows || lde_colT < cdiv(rows, kTile))) return FP8Q_ERR_SHAPE;
    if (cdiv(rows, kTile) * cdiv(cols, kTile) >= kMaxIndex) return FP8Q_ERR_SHAPE;
    if (!aligned16(x) || (ldx * elem_size(x_dtype)) % 16) return FP8Q_ERR_ALIGN;
    if (want_row && (!aligned16(q_row) || ldq_row % 16)) return FP8Q_ERR_ALIGN;
    if (want_col && (!aligned16(q_colT) || ldq_colT % 16)) return FP8Q_ERR_ALIGN;
    int st = check_device();
    if (st != FP8Q_OK) return st;
    fp8q::launch_quant_transpose_e8m0(x, x_dtype, rows, cols, ldx, want_row ? q_row : nullptr, ldq_row,
                                      e_row, lde_row, want_col ? q_colT : nullptr, ldq_colT, e_colT,
                                      lde_colT, stream);
    return launch_status(stream);
}

int fp8_gemm_e8m0(int64_t M, int64_t N, int64_t K,
                  const uint8_t* a, int64_t lda, const uint8_t* ea, int64_t ldea,
                  const uint8_t* b, int64_t ldb, int b_layout,
                  const uint8_t* eb, int64_t ldeb, int eb_kind,
                  void* c, int64_t ldc, int c_dtype, hipStream_t stream)
{
    if (!dtype_ok(c_dtype)) return FP8Q_ERR_UNSUPPORTED;
    if (b_layout != FP8Q_B_NK && b_layout != FP8Q_B_KN) return FP8Q_ERR_UNSUPPORTED;
    if (eb_kind != FP8Q_ROW_1x128 && eb_kind != FP8Q_BLOCK_128x128) return FP8Q_ERR_UNSUPPORTED;
    if (eb_kind == FP8Q_ROW_1x128 && b_layout == FP8Q_B_KN) return FP8Q_ERR_UNSUPPORTED;
    if (M < 0 || N < 0 || K < 0) return FP8Q_ERR_SHAPE;
    if (M == 0 || N == 0) return FP8Q_OK;
    if (!c) return FP8Q_ERR_NULL;
    if (K > 0 && (!a || !b || !ea || !eb)) return FP8Q_ERR_NULL;
    const int64_t KB = cdiv(K, kTile);
    if (lda < K || ldc < N) return FP8Q_ERR_SHAPE;
    if (b_layout == FP8Q_B_NK ? ldb < K : ldb < N) return FP8Q_ERR_SHAPE;
    if (ldea < KB) return FP8Q_ERR_SHAPE;
    if (eb_kind == FP8Q_ROW_1x128 && ldeb < KB) return FP8Q_ERR_SHAPE;
    if (eb_kind == FP8Q_BLOCK_128x128 && (b_layout == FP8Q_B_NK ? ldeb < KB : ldeb < cdiv(N, kTile)))
        return FP8Q_ERR_SHAPE;
    if (cdiv(M, 256) * cdiv(N, 128) >= kMaxIndex || KB >= kMaxIndex) return FP8Q_ERR_SHAPE;
    if (K > 0 && (!aligned16(a) || !aligned16(b) || lda % 16 || ldb % 16)) return FP8Q_ERR_ALIGN;
    // the kernel reads each scale row as 4-byte words
    if (K > 0 && ((reinterpret_cast<uintptr_t>(ea) & 3u) || (reinterpret_cast<uintptr_t>(eb) & 3u) ||
                  ldea % 4 || ldeb % 4))
        return FP8Q_ERR_ALIGN;
    if (!aligned16(c) || (ldc * elem_size(c_dtype)) % 16) return FP8Q_ERR_ALIGN;
    int st = check_device();
    if (st != FP8Q_OK) return st;
    if (!fp8q::launch_gemm_e8m0(M, N, K, a, lda, ea, ldea, b, ldb, b_layout, eb, ldeb, eb_kind, c, ldc,
                                c_dtype, stream))
        return FP8Q_ERR_UNSUPPORTED;
    return launch_status(stream);
}

int fp8_adam_step(int64_t n, float* p, const void* g, int g_dtype, uint8_t* mq, float* ms,
                  uint8_t* vq, float* vs, double lr, double beta1, double beta2, double eps,
                  double weight_decay, int64_t step, hipStream_t stream)
{
    if (!dtype_ok(g_dtype)) return FP8Q_ERR_UNSUPPORTED;
    if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0) || step < 1 ||
        !std::isfinite(lr) || !std::isfinite(eps) || !std::isfinite(weight_decay))
        return FP8Q_ERR_UNSUPPORTED;
    if (n < 0) return FP8Q_ERR_SHAPE;
    if (n == 0) return FP8Q_OK;
    if (!p || !g || !mq || !ms || !vq || !vs) return FP8Q_ERR_NULL;
    if (cdiv(n, kTile) >= kMaxIndex) return FP8Q_ERR_SHAPE;
    if (!aligned16(p) || !aligned16(g) || !aligned16(mq) || !aligned16(vq) ||
        (reinterpret_cast<uintptr_t>(ms) & 3u) || (reinterpret_cast<uintptr_t>(vs) & 3u))
        return FP8Q_ERR_ALIGN;
    int st = check_device();
    if (st != FP8Q_OK) return st;
    // derived scalars: computed in double, each rounded once to fp32
    fp8q::AdamScalars a;
    a.b1 = (float)beta1;
    a.b2 = (float)beta2;
    a.omb1 = (float)(1.0 - beta1);
    a.omb2 = (float)(1.0 - beta2);
    a.decay = (float)(1.0 - lr * weight_decay);
    a.step_size = (float)(lr / (1.0 - std::pow(beta1, (double)step)));
    a.bc2_sqrt = (float)std::sqrt(1.0 - std::pow(beta2, (double)step));
    a.eps = (float)eps;
    fp8q::launch_adam_fp8(n, p, g, g_dtype, mq, ms, vq, vs, a, stream);
    return launch_status(stream);
}

// Validation of the operands of a dense GEMM (everything but the output).
// Returns FP8Q_OK, or a status; *empty is set when there is nothing to do.
static int gemm_operands_status(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda,
                                const float* sa, int64_t ldsa, int sa_kind, const uint8_t* b,
                                int64_t ldb, int b_layout, const float* sb, int64_t ldsb, int sb_kind,
                                bool* empty)
{
    *empty = false;
    if (b_layout != FP8Q_B_NK && b_layout != FP8Q_B_KN) return FP8Q_ERR_UNSUPPORTED;
    if (sa_kind != FP8Q_ROW_1x128 && sa_kind != FP8Q_TENSOR) return FP8Q_ERR_UNSUPPORTED;
    if (sb_kind != FP8Q_ROW_1x128 && sb_kind != FP8Q_BLOCK_128x128 && sb_kind != FP8Q_TENSOR)
        return FP8Q_ERR_UNSUPPORTED;
    if (sb_kind == FP8Q_ROW_1x128 && b_layout == FP8Q_B_KN) return FP8Q_ERR_UNSUPPORTED;
    if (M < 0 || N < 0 || K < 0) return FP8Q_ERR_SHAPE;
    if (M == 0 || N == 0) {
        *empty = true;
        return FP8Q_OK;
    }
    if (K > 0 && (!a || !b || !sa || !sb)) return FP8Q_ERR_NULL;
    const int64_t KB = cdiv(K, kTile);
    if (lda < K) return FP8Q_ERR_SHAPE;
    if (b_layout == FP8Q_B_NK ? ldb < K : ldb < N) return FP8Q_ERR_SHAPE;
    if (sa_kind == FP8Q_ROW_1x128 && ldsa < KB) return FP8Q_ERR_SHAPE;
    if (sb_kind == FP8Q_ROW_1x128 && ldsb < KB) return FP8Q_ERR_SHAPE;
    if (sb_kind == FP8Q_BLOCK_128x128 && (b_layout == FP8Q_B_NK ? ldsb < KB : ldsb < cdiv(N, kTile)))
        return FP8Q_ERR_SHAPE;
    if (cdiv(M, 256) * cdiv(N, 128) >= kMaxIndex || KB >= kMaxIndex) return FP8Q_ERR_SHAPE;
    if (K > 0 && (!aligned16(a) || !aligned16(b) || lda % 16 || ldb % 16)) return FP8Q_ERR_ALIGN;
    return FP8Q_OK;
}

int fp8_gemm_blockscaled_e4m3(int64_t M, int64_t N, int64_t K,
                              const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa, int sa_kind,
                              const uint8_t* b, int64_t ldb, int b_layout,
                              const float* sb, int64_t ldsb, int sb_kind,
                              uint8_t* q, int64_t ldq, float* s, int64_t lds, hipStream_t stream)
{
    bool empty;
    int st = gemm_operands_status(M, N, K, a, lda, sa, ldsa, sa_kind, b, ldb, b_layout, sb, ldsb,
                                  sb_kind, &empty);
    if (st != FP8Q_OK || empty) return st;
    if (sb_kind == FP8Q_ROW_1x128) return FP8Q_ERR_UNSUPPORTED;
    if (!q || !s) return FP8Q_ERR_NULL;
    if (ldq < N || lds < cdiv(N, kTile)) return FP8Q_ERR_SHAPE;
    if (!aligned16(q) || ldq % 16) return FP8Q_ERR_ALIGN;
    st = check_device();
    if (st != FP8Q_OK) return st;
    if (!fp8q::launch_gemm_e4m3(M, N, K, a, lda, sa, ldsa, sa_kind, b, ldb, b_layout, sb, ldsb, sb_kind,
                                q, ldq, s, lds, stream))
        return FP8Q_ERR_UNSUPPORTED;
    return launch_status(stream);
}

int fp8_gemm_blockscaled(int64_t M, int64_t N, int64_t K,
                         const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa, int sa_kind,
                         const uint8_t* b, int64_t ldb, int b_layout,
                         const float* sb, int64_t ldsb, int sb_kind,
                         void* c, int64_t ldc, int c_dtype, hipStream_t stream)
{
    if (!dtype_ok(c_dtype)) return FP8Q_ERR_UNSUPPORTED;
    if (b_layout != FP8Q_B_NK && b_layout != FP8Q_B_KN) return FP8Q_ERR_UNSUPPORTED;
    if (sa_kind != FP8Q_ROW_1x128 && sa_kind != FP8Q_TENSOR) return FP8Q_ERR_UNSUPPORTED;
    if (sb_kind != FP8Q_ROW_1x128 && sb_kind != FP8Q_BLOCK_128x128 && sb_kind != FP8Q_TENSOR)
        return FP8Q_ERR_UNSUPPORTED;
    if (sb_kind == FP8Q_ROW_1x128 && b_layout == FP8Q_B_KN) return FP8Q_ERR_UNSUPPORTED;
    if (M < 0 || N < 0 || K < 0) return FP8Q_ERR_SHAPE;
    if (M == 0 || N == 0) return FP8Q_OK;
    if (!c) return FP8Q_ERR_NULL;
    // with K == 0 the operands and scales hold no data and are never read
    if (K > 0 && (!a || !b || !sa || !sb)) return FP8Q_ERR_NULL;
    const int64_t KB = cdiv(K, kTile);
    if (lda < K || ldc < N) return FP8Q_ERR_SHAPE;
    if (b_layout == FP8Q_B_NK ? ldb < K : ldb < N) return FP8Q_ERR_SHAPE;
    if (sa_kind == FP8Q_ROW_1x128 && ldsa < KB) return FP8Q_ERR_SHAPE;
    if (sb_kind == FP8Q_ROW_1x128 && ldsb < KB) return FP8Q_ERR_SHAPE;
    if (sb_kind == FP8Q_BLOCK_128x128 && (b_layout == FP8Q_B_NK ? ldsb < KB : ldsb < cdiv(N, kTile)))
        return FP8Q_ERR_SHAPE;
    if (cdiv(M, 256) * cdiv(N, 128) >= kMaxIndex || KB >= kMaxIndex) return FP8Q_ERR_SHAPE;
    if (!aligned16(c) || (ldc * elem_size(c_dtype)) % 16) return FP8Q_ERR_ALIGN;
    if (K > 0 && (!aligned16(a) || !aligned16(b) || lda % 16 || ldb % 16)) return FP8Q_ERR_ALIGN;
    int st = check_device();
    if (st != FP8Q_OK) return st;
    if (!fp8q::launch_gemm(M, N, K, a, lda, sa, ldsa, sa_kind, b, ldb, b_layout, sb, ldsb, sb_kind, c,
                           ldc, c_dtype, stream))
        return FP8Q_ERR_UNSUPPORTED;
    return launch_status(stream);
}

int fp8_grouped_gemm(int64_t G, int64_t M_pad, int64_t N, int64_t K,
                     const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                     const int32_t* group_offsets,
                     const uint8_t* b, const float* sb,
                     void* c, int64_t ldc, int c_dtype, hipStream_t stream)
{
    if (!dtype_ok(c_dtype)) return FP8Q_ERR_UNSUPPORTED;
    if (G < 1 || M_pad < 0 || N < 0 || K < 0 || M_pad % kTile) return FP8Q_ERR_SHAPE;
    if (G > kMaxGroups) return FP8Q_ERR_UNSUPPORTED;
    if (M_pad == 0 || N == 0) return FP8Q_OK;
    if (!group_offsets || !c) return FP8Q_ERR_NULL;
    if (K > 0 && (!a || !sa || !b || !sb)) return FP8Q_ERR_NULL;
    const int64_t KB = cdiv(K, kTile);
    if (lda < K || ldc < N || ldsa < KB) return FP8Q_ERR_SHAPE;
    if (G >= kMaxIndex || (M_pad / kTile) * cdiv(N, 128) >= kMaxIndex) return FP8Q_ERR_SHAPE;
    if (!aligned16(c) || K % 16 || (ldc * elem_size(c_dtype)) % 16) return FP8Q_ERR_ALIGN;
    if (K > 0 && (!aligned16(a) || !aligned16(b) || lda % 16)) return FP8Q_ERR_ALIGN;
    if (reinterpret_cast<uintptr_t>(group_offsets) & 3u) return FP8Q_ERR_ALIGN;
    int st = check_device();
    if (st != FP8Q_OK) return st;
    st = offsets_status(group_offsets, G, M_pad, stream);
    if (st != FP8Q_OK) return st;
    if (!fp8q::launch_grouped_gemm(G, M_pad, N, K, a, lda, sa, ldsa, group_offsets, b, sb, c, ldc,
                                   c_dtype, stream))
        return FP8Q_ERR_UNSUPPORTED;
    return launch_status(stream);
}

int fp8_grouped_gemm_e4m3(int64_t G, int64_t M_pad, int64_t N, int64_t K,
                          const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                          const int32_t* group_offsets,
                          const uint8_t* b, const float* sb,
                          uint8_t* q, int64_t ldq, float* s, int64_t lds, hipStream_t stream)
{
    if (G < 1 || M_pad < 0 || N < 0 || K < 0 || M_pad % kTile) return FP8Q_ERR_SHAPE;
    if (G > kMaxGroups) return FP8Q_ERR_UNSUPPORTED;
    if (M_pad == 0 || N == 0) return FP8Q_OK;
    if (K == 0 || K % kTile) return FP8Q_ERR_UNSUPPORTED;
    if (!group_offsets || !q || !s || !a || !sa || !b || !sb) return FP8Q_ERR_NULL;
    const int64_t KB = K / kTile;
    if (lda < K || ldq < N || ldsa < KB || lds < cdiv(N, kTile)) return FP8Q_ERR_SHAPE;
    if (G >= kMaxIndex || (M_pad / kTile) * cdiv(N, 128) >= kMaxIndex) return FP8Q_ERR_SHAPE;
    if (!aligned16(q) || ldq % 16 || !aligned16(a) || !aligned16(b) || lda % 16) return FP8Q_ERR_ALIGN;
    if (reinterpret_cast<uintptr_t>(group_offsets) & 3u) return FP8Q_ERR_ALIGN;
    int st = check_device();
    if (st != FP8Q_OK) return st;
    st = offsets_status(group_offsets, G, M_pad, stream);
    if (st != FP8Q_OK) return st;
    if (!fp8q::launch_grouped_gemm_e4m3(G, M_pad, N, K, a, lda, sa, ldsa, group_offsets, b, sb, q, ldq, s,
                                        lds, stream))
        return FP8Q_ERR_UNSUPPORTED;
    return launch_status(stream);
}

int fp8_grouped_gemm_dgrad(int64_t G, int64_t M_pad, int64_t N, int64_t K,
                           const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                           const int32_t* group_offsets,
                           const uint8_t* w, const float* sw,
                           void* c, int64_t ldc, int c_dtype, hipStream_t stream)
{
    if (!dtype_ok(c_dtype)) return FP8Q_ERR_UNSUPPORTED;
    if (G < 1 || M_pad < 0 || N < 0 || K < 0 || M_pad % kTile) return FP8Q_ERR_SHAPE;
    if (G > kMaxGroups) return FP8Q_ERR_UNSUPPORTED;
    if (M_pad == 0 || K == 0) return FP8Q_OK;
    if (!group_offsets || !c) return FP8Q_ERR_NULL;
    if (N > 0 && (!a || !sa || !w || !sw)) return FP8Q_ERR_NULL;
    if (lda < N || ldc < K || ldsa < cdiv(N, kTile)) return FP8Q_ERR_SHAPE;
    if (G >= kMaxIndex || (M_pad / kTile) * cdiv(K, 128) >= kMaxIndex) return FP8Q_ERR_SHAPE;
    if (!aligned16(c) || K % 16 || (ldc * elem_size(c_dtype)) % 16) return FP8Q_ERR_ALIGN;
    if (N > 0 && (!aligned16(a) || !aligned16(w) || lda % 16)) return FP8Q_ERR_ALIGN;
    if (reinterpret_cast<uintptr_t>(group_offsets) & 3u) return FP8Q_ERR_ALIGN;
    int st = check_device();
    if (st != FP8Q_OK) return st;
    st = offsets_status(group_offsets, G, M_pad, stream);
    if (st != FP8Q_OK) return st;
    if (!fp8q::launch_grouped_gemm_dgrad(G, M_pad, N, K, a, lda, sa, ldsa, group_offsets, w, sw, c, ldc,
                                         c_dtype, stream))
        return FP8Q_ERR_UNSUPPORTED;
    return launch_status(stream);
}

int fp8_grouped_gemm_wgrad(int64_t G, int64_t M_pad, int64_t N, int64_t K,
                           const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                           const uint8_t* b, int64_t ldb, const float* sb, int64_t ldsb,
                           const int32_t* group_offsets,
                           float* c, int64_t ldc, hipStream_t stream)
{
    if (G < 1 || M_pad < 0 || N < 0 || K < 0 || M_pad % kTile) return FP8Q_ERR_SHAPE;
    if (G > kMaxGroups) return FP8Q_ERR_UNSUPPORTED;
    if (N == 0 || K == 0) return FP8Q_OK;
    if (!group_offsets || !c) return FP8Q_ERR_NULL;
    if (M_pad > 0 && (!a || !sa || !b || !sb)) return FP8Q_ERR_NULL;
    if (lda < M_pad || ldb < M_pad || ldc < K || ldsa < M_pad / kTile || ldsb < M_pad / kTile)
        return FP8Q_ERR_SHAPE;
    if (G >= kMaxIndex || G * cdiv(N, 128) * cdiv(K, 256) >= kMaxIndex) return FP8Q_ERR_SHAPE;
    if (!aligned16(c) || (ldc * 4) % 16) return FP8Q_ERR_ALIGN;
    if (M_pad > 0 && (!aligned16(a) || !aligned16(b) || lda % 16 || ldb % 16)) return FP8Q_ERR_ALIGN;
    if (reinterpret_cast<uintptr_t>(group_offsets) & 3u) return FP8Q_ERR_ALIGN;
    int st = check_device();
    if (st != FP8Q_OK) return st;
    st = offsets_status(group_offsets, G, M_pad, stream);
    if (st != FP8Q_OK) return st;
    if (!fp8q::launch_grouped_gemm_wgrad(G, M_pad, N, K, a, lda, sa, ldsa, b, ldb, sb, ldsb, group_offsets,
                                         c, ldc, stream))
        return FP8Q_ERR_UNSUPPORTED;
    return launch_status(stream);
}

}  // extern "C"
