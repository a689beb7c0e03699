// Fused quantize + transpose for gfx950.
//
// One read of X[rows][cols] yields (i) 1x128 row tiles along cols and (ii)
// 1x128 tiles along rows, stored transposed (X^T row tiles).  (ii) is the
// weight-gradient operand: dW contracts over tokens, so the gradient must be
// re-quantized with tiles along the token axis (Ling 2.0 FP8 blog: the
// "grad (transpose)" tensor that dw consumes; FP8 transposes are the slow
// step that made frameworks cache transposed copies, "FP8 on-demand
// transpose weight").
//
// One 512-thread workgroup per 128x128 block (four fit on a CU; a
// persistent form with two workgroups per CU, each loading its next block
// while it quantizes the current one, measured 5-12% slower).  Thread
// (g = tid/16, l = tid%16) holds rows 4g..4g+3 at columns 8l..8l+7.  Row
// amax: DPP across the 16 lanes of a row.  Column amax: per-thread max over
// its 4 rows, then across the 32 row groups through LDS.  Each scale and
// reciprocal is computed once (one thread per row / column) and shared
// through LDS.  The column codes are produced already in column order (the
// 4 rows of a thread packed in one dword), staged in LDS as the transposed
// block and written back as 16-byte row segments of X^T.
#include <type_traits>

#include "fp8q_device.h"
#include "fp8q_internal.h"
#include "quant_io.h"

namespace fp8q {

constexpr int kQtThreads = 512;
constexpr int kQtGroups = kQtThreads / 16;     // row groups of 16 lanes
constexpr int kQtRows = kTile / kQtGroups;     // rows per thread
constexpr int kStagePitch = 128;   // bytes per staged X^T row
constexpr int kColPitch = 130;     // floats per row group in the column-maxima array

// LDS layouts (64 banks of 4 bytes; a wave's 4-byte accesses take one pass
// when their 64 lanes hit distinct banks or share addresses):
//  * column maxima: row group g, column c = 8l + j at g * 130 + 8l + (j ^ (l >> 3));
//    the writes (fixed j: banks 2g + 8l + (j or j ^ 1)) and the per-column
//    reads (64 consecutive words) are conflict-free;
//  * column scales: column c at c + 4 (c >> 6).  The column-code pass reads
//    columns 8l + j (fixed j) for l = 0..15; without the skew l and l + 8
//    would share a bank;
//  * staged X^T block: X^T row c at physical row p(c) = c ^ ((c >> 6) & 1),
//    its 16-byte slot t (X rows 16t..16t+15, in order) at
//    p(c) * 128 + 16 (t ^ k(c)), k(c) = (c ^ (c >> 3)) & 7.  A code write
//    (column 8l + j, rows 4g..4g+3 of wave w = g / 4) hits bank
//    32 ((j & 1) ^ (l >> 3)) + 4 (w ^ j ^ (l & 7)) + g % 4: all 64 distinct.
//    A 16-byte read pass (16 lanes: two X^T rows, which p keeps in one
//    pair of physical rows) covers the 64 banks once.
__device__ __forceinline__ int colmax_idx(int c) { return 8 * (c >> 3) + ((c & 7) ^ ((c >> 6) & 1)); }
__device__ __forceinline__ int colscale_idx(int c) { return c + 4 * (c >> 6); }
__device__ __forceinline__ int stage_row(int c) { return c ^ ((c >> 6) & 1); }
__device__ __forceinline__ int stage_key(int c) { return (c ^ (c >> 3)) & 7; }

// Four values of one tile -> four codes (the 4-row column units).
template <typename S>
__device__ __forceinline__ uint32_t quant4_as(float a, float b, float c, float d, const TileScale& t)
{
    if constexpr (sizeof(S) == 4) {
        if (__builtin_amdgcn_ballot_w64(t.mode == 2) == 0) {
            const float v[4] = {a, b, c, d};
            float q[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float q0 = v[i] * t.y;
                const float e = __builtin_fmaf(q0, t.s, -v[i]);
                q[i] = __builtin_fmaf(-e, t.y, q0);
            }
            return pack4_e4m3(q[0], q[1], q[2], q[3]);
        }
        return quant4(a, b, c, d, t);
    } else {
        return pack4_e4m3(a * t.y, b * t.y, c * t.y, d * t.y);
    }
}

template <typename T, typename S>
__global__ __launch_bounds__(kQtThreads) void quant_transpose_kernel(
    const T* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
    uint8_t* __restrict__ q_row, int64_t ldq_row, S* __restrict__ s_row, int64_t lds_row,
    uint8_t* __restrict__ q_colT, int64_t ldq_colT, S* __restrict__ s_colT, int64_t lds_colT,
    FastDiv blocks_per_row)
{
    __shared__ float col_part[kQtGroups * kColPitch];   // per row-group column maxima
    __shared__ float row_amax[kTile];
    __shared__ float row_s[kTile], row_y[kTile];
    __shared__ int row_mode[kTile];
    __shared__ float col_s[kTile + 4], col_y[kTile + 4];
    __shared__ int col_mode[kTile + 4];
    __shared__ __attribute__((aligned(16))) uint8_t stage[kTile * kStagePitch];

    const int tid = threadIdx.x;
    const int l = tid & 15;
    const int g = tid >> 4;
    const bool do_row = q_row != nullptr;
    const bool do_col = q_colT != nullptr;

    // this block: rows [r0, r0 + 128), columns [c0, c0 + 128)
    const uint32_t b = blockIdx.x;
    const uint32_t rbu = fdiv(b, blocks_per_row);
    const int64_t rb = rbu, cb = b - rbu * blocks_per_row.d;
    const int64_t r0 = rb * kTile, c0 = cb * kTile;

    // FULL: the block lies inside the matrix, so no element, row or column
    // needs a bounds test (every block but those on the right and bottom
    // edges); the same body with the tests covers the edges
    auto body = [&](auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        float v[kQtRows][8];
        {
            Raw8<T> R[kQtRows];
            if constexpr (FULL) {
                const T* xb = x + (r0 + kQtRows * g) * ldx + c0 + 8 * l;
#pragma unroll
                for (int u = 0; u < kQtRows; ++u) raw_load_full(xb + u * ldx, R[u]);
#pragma unroll
                for (int u = 0; u < kQtRows; ++u) raw_f32_full(R[u], v[u]);
            } else {
#pragma unroll
                for (int u = 0; u < kQtRows; ++u) {
                    const int64_t r = r0 + kQtRows * g + u;
                    raw_load(x + (r < rows ? r : 0) * ldx, r < rows ? c0 + 8 * l : cols, cols, R[u]);
                }
#pragma unroll
                for (int u = 0; u < kQtRows; ++u) {
                    const int64_t r = r0 + kQtRows * g + u;
                    raw_f32(R[u], r < rows ? c0 + 8 * l : cols, cols, v[u]);
                }
            }
        }

        // row maxima (DPP over the 16 lanes of each row), column partial maxima
#pragma unroll
        for (int u = 0; u < kQtRows; ++u) {
            float m = fabsf(v[u][0]);
#pragma unroll
            for (int j = 1; j < 8; ++j) m = fmaxf(m, fabsf(v[u][j]));
            m = dpp_max16(m);
            if (l == 0) row_amax[kQtRows * g + u] = m;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float m = fabsf(v[0][j]);
#pragma unroll
            for (int u = 1; u < kQtRows; ++u) m = fmaxf(m, fabsf(v[u][j]));
            col_part[g * kColPitch + colmax_idx(8 * l + j)] = m;
        }
        __syncthreads();

        // one thread per column (tid < 128) and per row (128 <= tid < 256)
        if (tid < kTile) {
            const int ci = colmax_idx(tid);
            float m = col_part[ci];
#pragma unroll
            for (int k = 1; k < kQtGroups; ++k) m = fmaxf(m, col_part[k * kColPitch + ci]);
            TileScale ts = make_tile_scale<S>(m);
            const int si = colscale_idx(tid);
            col_s[si] = ts.s;
            col_y[si] = ts.y;
            col_mode[si] = ts.mode;
            if (do_col && (FULL || c0 + tid < cols))
                s_colT[(c0 + tid) * lds_colT + rb] = stored_scale<S>(ts);
        } else if (tid < 2 * kTile) {
            int i = tid - kTile;
            TileScale ts = make_tile_scale<S>(row_amax[i]);
            row_s[i] = ts.s;
            row_y[i] = ts.y;
            row_mode[i] = ts.mode;
            if (do_row && (FULL || r0 + i < rows))
                s_row[(r0 + i) * lds_row + cb] = stored_scale<S>(ts);
        }
        __syncthreads();

        if (do_row) {
            const int64_t c = c0 + 8 * l;
            uint8_t* const qb = q_row + (r0 + kQtRows * g) * ldq_row + c;
#pragma unroll
            for (int u = 0; u < kQtRows; ++u) {
                int i = kQtRows * g + u;
                TileScale ts{row_s[i], row_y[i], row_mode[i]};
                uint32_t lo, hi;
                quant8_as<S>(v[u], ts, lo, hi);
                if constexpr (FULL) {
                    *reinterpret_cast<uint2*>(qb + u * ldq_row) = make_uint2(lo, hi);
                } else {
                    const int64_t r = r0 + i;
                    if (r < rows && c < cols) store8(q_row + r * ldq_row, c, cols, lo, hi);
                }
            }
        }

        if (do_col) {
            // column j of this thread, rows 4g..4g+3, packed in row order
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int cj = 8 * l + j;
                const int si = colscale_idx(cj);
                TileScale ts{col_s[si], col_y[si], col_mode[si]};
                const uint32_t w = quant4_as<S>(v[0][j], v[1][j], v[2][j], v[3][j], ts);
                *reinterpret_cast<uint32_t*>(stage + stage_row(cj) * kStagePitch +
                                             16 * ((g >> 2) ^ stage_key(cj)) + 4 * (g & 3)) = w;
            }
            __syncthreads();
            // 8 threads per X^T row (16 bytes each), 64 rows per pass
#pragma unroll
            for (int pass = 0; pass < kTile / (kQtThreads / 8); ++pass) {
                int cr = pass * (kQtThreads / 8) + (tid >> 3);   // row of the staged X^T block
                int seg = (tid & 7) * 16;              // byte offset along X's rows
                int64_t cglob = c0 + cr;
                int64_t rglob = r0 + seg;
                const uint4 w = *reinterpret_cast<const uint4*>(stage + stage_row(cr) * kStagePitch +
                                                                16 * ((tid & 7) ^ stage_key(cr)));
                uint8_t* dst = q_colT + cglob * ldq_colT + rglob;
                if (FULL || (cglob < cols && rglob + 16 <= rows)) {
                    *reinterpret_cast<uint4*>(dst) = w;
                } else if (cglob < cols && rglob < rows) {
                    uint32_t wd[4] = {w.x, w.y, w.z, w.w};
                    for (int k = 0; k < 16 && rglob + k < rows; ++k)
                        dst[k] = (uint8_t)((wd[k >> 2] >> (8 * (k & 3))) & 0xFF);
                }
            }
        }
    };
    if (r0 + kTile <= rows && c0 + kTile <= cols)
        body(std::true_type{});
    else
        body(std::false_type{});
}

template <typename S>
static void launch_qt(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                      uint8_t* q_row, int64_t ldq_row, S* s_row, int64_t lds_row,
                      uint8_t* q_colT, int64_t ldq_colT, S* s_colT, int64_t lds_colT, hipStream_t st)
{
    const int64_t bc = (cols + kTile - 1) / kTile;
    const uint32_t total = (uint32_t)(bc * ((rows + kTile - 1) / kTile));
    const FastDiv fd = make_fastdiv((uint32_t)bc);
    if (x_dtype == FP8Q_BF16)
        hipLaunchKernelGGL((quant_transpose_kernel<uint16_t, S>), dim3(total), dim3(kQtThreads),
                           0, st, static_cast<const uint16_t*>(x), rows, cols, ldx, q_row, ldq_row, s_row,
                           lds_row, q_colT, ldq_colT, s_colT, lds_colT, fd);
    else
        hipLaunchKernelGGL((quant_transpose_kernel<float, S>), dim3(total), dim3(kQtThreads), 0, st,
                           static_cast<const float*>(x), rows, cols, ldx, q_row, ldq_row, s_row,
                           lds_row, q_colT, ldq_colT, s_colT, lds_colT, fd);
}

void launch_quant_transpose(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                            uint8_t* q_row, int64_t ldq_row, float* s_row, int64_t lds_row,
                            uint8_t* q_colT, int64_t ldq_colT, float* s_colT, int64_t lds_colT,
                            hipStream_t st)
{
    launch_qt<float>(x, x_dtype, rows, cols, ldx, q_row, ldq_row, s_row, lds_row, q_colT, ldq_colT,
                     s_colT, lds_colT, st);
}

void launch_quant_transpose_e8m0(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                                 uint8_t* q_row, int64_t ldq_row, uint8_t* e_row, int64_t lde_row,
                                 uint8_t* q_colT, int64_t ldq_colT, uint8_t* e_colT, int64_t lde_colT,
                                 hipStream_t st)
{
    launch_qt<uint8_t>(x, x_dtype, rows, cols, ldx, q_row, ldq_row, e_row, lde_row, q_colT, ldq_colT,
                       e_colT, lde_colT, st);
}

}  // namespace fp8q
