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
// One 512-thread workgroup per 128x128 block.  Thread (g = tid/16,
// l = tid%16) holds rows 4g..4g+3 at columns 8l..8l+7.  Row amax: DPP across
// the 16 lanes of a row.  Column amax: per-thread max over its 4 rows, then
// across the 32 row groups through LDS.  Each scale and reciprocal is
// computed once (one thread per row / column) and shared through LDS.  The
// column codes are produced already in column order (the 4 rows of a thread
// packed in one dword), staged in LDS as the transposed tile and written
// back as 16-byte row segments of X^T.  (With 512 threads the kernel needs
// 54 VGPRs and four workgroups fit on a CU; 256 threads with 8 rows each
// took 86 and were 7% slower on a 4096 x 14336 gradient.)
#include "fp8q_device.h"
#include "fp8q_internal.h"

namespace fp8q {

constexpr int kQtThreads = 512;
constexpr int kQtGroups = kQtThreads / 16;     // row groups of 16 lanes
constexpr int kQtRows = kTile / kQtGroups;     // rows per thread
constexpr int kStagePitch = 128;   // bytes per staged X^T row
constexpr int kColPitch = 130;     // floats per row group in the column-maxima array

// LDS layouts (64 banks of 4 bytes), checked with a bank model:
//  * column maxima: row group g, column c = 8l + j at g * 130 + 8l + (j ^ (l >> 3));
//    the b32 writes (fixed j) and the per-column reads are conflict-free;
//  * staged X^T tile: the 4-byte unit of column c, rows 4g..4g+3, at byte
//    c * 128 + 16 ((g / 4) ^ sw(c)) + 4 (g % 4), sw(c) = (c ^ (c >> 3)) & 7,
//    so the 16-byte slot t of X^T row c (rows 16t..16t+15, in order) sits at
//    c * 128 + 16 (t ^ sw(c)).  Writes are 2-way, reads 1-way.
__device__ __forceinline__ int colmax_idx(int c) { return 8 * (c >> 3) + ((c & 7) ^ ((c >> 6) & 1)); }
__device__ __forceinline__ int stage_key(int c) { return (c ^ (c >> 3)) & 7; }

template <typename T>
__device__ __forceinline__ void qt_load8(const T* row, int64_t c, int64_t cols, float v[8]);

template <>
__device__ __forceinline__ void qt_load8<uint16_t>(const uint16_t* row, int64_t c, int64_t cols, float v[8])
{
    if (c >= cols) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
        return;
    }
    uint4 p = *reinterpret_cast<const uint4*>(row + c);
    v[0] = bf16_lo(p.x); v[1] = bf16_hi(p.x);
    v[2] = bf16_lo(p.y); v[3] = bf16_hi(p.y);
    v[4] = bf16_lo(p.z); v[5] = bf16_hi(p.z);
    v[6] = bf16_lo(p.w); v[7] = bf16_hi(p.w);
    if (c + 8 > cols) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (c + i >= cols) v[i] = 0.0f;
    }
}

template <>
__device__ __forceinline__ void qt_load8<float>(const float* row, int64_t c, int64_t cols, float v[8])
{
    if (c >= cols) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
        return;
    }
    float4 a = *reinterpret_cast<const float4*>(row + c);
    float4 b = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c + 4 < cols) b = *reinterpret_cast<const float4*>(row + c + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    if (c + 8 > cols) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (c + i >= cols) v[i] = 0.0f;
    }
}

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
    uint8_t* __restrict__ q_colT, int64_t ldq_colT, S* __restrict__ s_colT, int64_t lds_colT)
{
    __shared__ float col_part[kQtGroups * kColPitch];   // per row-group column maxima
    __shared__ float row_amax[kTile];
    __shared__ float row_s[kTile], row_y[kTile];
    __shared__ int row_mode[kTile];
    __shared__ float col_s[kTile], col_y[kTile];
    __shared__ int col_mode[kTile];
    __shared__ __attribute__((aligned(16))) uint8_t stage[kTile * kStagePitch];

    const int tid = threadIdx.x;
    const int l = tid & 15;
    const int g = tid >> 4;
    const int64_t r0 = (int64_t)blockIdx.y * kTile;
    const int64_t c0 = (int64_t)blockIdx.x * kTile;
    const int64_t cb = blockIdx.x;     // tile index along cols (row tiles)
    const int64_t rb = blockIdx.y;     // tile index along rows (column tiles)
    const bool do_row = q_row != nullptr;
    const bool do_col = q_colT != nullptr;

    float v[kQtRows][8];
#pragma unroll
    for (int u = 0; u < kQtRows; ++u) {
        int64_t r = r0 + kQtRows * g + u;
        qt_load8<T>(x + (r < rows ? r : 0) * ldx, r < rows ? c0 + 8 * l : cols, cols, v[u]);
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
        col_s[tid] = ts.s;
        col_y[tid] = ts.y;
        col_mode[tid] = ts.mode;
        if (do_col && c0 + tid < cols)
            s_colT[(c0 + tid) * lds_colT + rb] = stored_scale<S>(ts);
    } else if (tid < 2 * kTile) {
        int i = tid - kTile;
        TileScale ts = make_tile_scale<S>(row_amax[i]);
        row_s[i] = ts.s;
        row_y[i] = ts.y;
        row_mode[i] = ts.mode;
        if (do_row && r0 + i < rows)
            s_row[(r0 + i) * lds_row + cb] = stored_scale<S>(ts);
    }
    __syncthreads();

    if (do_row) {
        const int64_t c = c0 + 8 * l;
#pragma unroll
        for (int u = 0; u < kQtRows; ++u) {
            int i = kQtRows * g + u;
            TileScale ts{row_s[i], row_y[i], row_mode[i]};
            uint32_t lo, hi;
            quant8_as<S>(v[u], ts, lo, hi);
            int64_t r = r0 + i;
            if (r < rows && c < cols) {
                uint8_t* dst = q_row + r * ldq_row;
                if (c + 8 <= cols) {
                    *reinterpret_cast<uint2*>(dst + c) = make_uint2(lo, hi);
                } else {
                    for (int k = 0; k < 8 && c + k < cols; ++k)
                        dst[c + k] = (uint8_t)((k < 4 ? lo >> (8 * k) : hi >> (8 * (k - 4))) & 0xFF);
                }
            }
        }
    }

    if (do_col) {
        // column j of this thread, rows 4g..4g+3, packed in row order
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            int cj = 8 * l + j;
            TileScale ts{col_s[cj], col_y[cj], col_mode[cj]};
            const uint32_t w = quant4_as<S>(v[0][j], v[1][j], v[2][j], v[3][j], ts);
            *reinterpret_cast<uint32_t*>(stage + cj * kStagePitch + 16 * ((g >> 2) ^ stage_key(cj)) + 4 * (g & 3)) = w;
        }
        __syncthreads();
        // 8 threads per X^T row (16 bytes each), 64 rows per pass
#pragma unroll
        for (int pass = 0; pass < kTile / (kQtThreads / 8); ++pass) {
            int cr = pass * (kQtThreads / 8) + (tid >> 3);   // row of the staged X^T tile
            int seg = (tid & 7) * 16;              // byte offset along X's rows
            int64_t cglob = c0 + cr;
            int64_t rglob = r0 + seg;
            if (cglob < cols && rglob < rows) {
                uint4 w = *reinterpret_cast<const uint4*>(stage + cr * kStagePitch + 16 * ((tid & 7) ^ stage_key(cr)));
                uint8_t* dst = q_colT + cglob * ldq_colT + rglob;
                if (rglob + 16 <= rows) {
                    *reinterpret_cast<uint4*>(dst) = w;
                } else {
                    uint32_t wd[4] = {w.x, w.y, w.z, w.w};
                    for (int k = 0; k < 16 && rglob + k < rows; ++k)
                        dst[k] = (uint8_t)((wd[k >> 2] >> (8 * (k & 3))) & 0xFF);
                }
            }
        }
    }
}

template <typename S>
static void launch_qt(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                      uint8_t* q_row, int64_t ldq_row, S* s_row, int64_t lds_row,
                      uint8_t* q_colT, int64_t ldq_colT, S* s_colT, int64_t lds_colT, hipStream_t st)
{
    dim3 grid((uint32_t)((cols + kTile - 1) / kTile), (uint32_t)((rows + kTile - 1) / kTile));
    if (x_dtype == FP8Q_BF16)
        hipLaunchKernelGGL((quant_transpose_kernel<uint16_t, S>), grid, dim3(kQtThreads), 0, st,
                           static_cast<const uint16_t*>(x), rows, cols, ldx, q_row, ldq_row, s_row,
                           lds_row, q_colT, ldq_colT, s_colT, lds_colT);
    else
        hipLaunchKernelGGL((quant_transpose_kernel<float, S>), grid, dim3(kQtThreads), 0, st,
                           static_cast<const float*>(x), rows, cols, ldx, q_row, ldq_row, s_row,
                           lds_row, q_colT, ldq_colT, s_colT, lds_colT);
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
