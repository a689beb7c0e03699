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
constexpr int kColPitch = 129;     // words per row group in the column-maxima array

// LDS layouts.  Measured on gfx950: a wave's 4-byte accesses are served in
// two halves of 32 lanes, each conflict-free when its lanes hit distinct
// word addresses mod 32 (or share one address); 8-byte reads take two
// cycles when the lanes read consecutive 8-byte words; 16-byte reads go in
// groups of 16 lanes, conflict-free when a group covers 256 contiguous
// bytes.  The compiler's merged form of two 8-byte reads (one instruction,
// two addresses) measured slower than two plain reads, and took 15 cycles
// with conflicts on 16-byte records 16 bytes apart, so the scale reads below
// are kept separate.
//  * column maxima: row group g, column c at 129 g + rot(c), rot rotating
//    each aligned run of 32 columns by 2 (c >> 5).  A write (fixed j, c =
//    8l + j, two row groups per half) hits banks g + 8 (l & 3) + 2 (l >> 2)
//    + j: 32 distinct; the per-column reads (32 consecutive columns, fixed
//    g) are a rotation;
//  * scale pairs {s', y'} (8 bytes; 8-byte accesses: 32 lanes per cycle,
//    conflict-free on distinct 8-byte slots mod 32) of column c at
//    c ^ ((c >> 5) & 3): the column pass reads columns 8l + j (fixed j) for
//    l = 0..15, slots 8 (l & 3) + (j ^ (l >> 2)), 16 distinct; the writers
//    (32 consecutive columns) a permutation of 32 slots.  Row pairs in row
//    order (a half-wave reads two rows);
//  * staged X^T block: X^T row c at byte 128 c, its 16-byte slot t (X rows
//    16t..16t+15) at 16 (t ^ k(c)), k(c) = (c ^ (c >> 3)) & 7, and within the
//    slot the dword of X rows 4g..4g+3 at position (g & 3) ^ (2 (c >> 6)).
//    A code write (column 8l + j, rows 4g..4g+3 of wave w = g / 4) hits bank
//    4 (w ^ k(c)) + ((g & 3) ^ 2 (l >> 3)): 32 distinct per half; a 16-byte
//    read group (two X^T rows, 8 slots each) covers 256 contiguous bytes.
__device__ __forceinline__ int colmax_idx(int c) { return (c & ~31) | ((c + 2 * (c >> 5)) & 31); }
__device__ __forceinline__ int csy_idx(int c) { return c ^ ((c >> 5) & 3); }
__device__ __forceinline__ int stage_key(int c) { return (c ^ (c >> 3)) & 7; }

// Maxima of |x| cross lanes and LDS as fp32 bit patterns: non-negative
// floats order like their bit patterns, so those maxima are integer maxima
// (exact; inputs are finite by contract).
// maxima of four values across the 16 lanes of a DPP row
template <int CTRL>
__device__ __forceinline__ void dpp_umax_step(uint32_t (&v)[4])
{
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = max(v[u], (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v[u], CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ void dpp_umax16x4(uint32_t (&v)[4])
{
    dpp_umax_step<0xB1>(v);    // quad [1,0,3,2]
    dpp_umax_step<0x4E>(v);    // quad [2,3,0,1]
    dpp_umax_step<0x141>(v);   // half-row mirror
    dpp_umax_step<0x140>(v);   // row mirror
}

// RN_fp32(x / s) for a tile with s >= 2^-90 or s = 0 (see quotient())
__device__ __forceinline__ float quotient_fast(float x, float s, float y)
{
    const float q0 = x * y;
    const float e = __builtin_fmaf(q0, s, -x);
    return __builtin_fmaf(-e, y, q0);
}

// Per-tile constants of the code passes, {s', y', p}: the codes are
// E4M3(RN(x p / s')) with y' = RN(1 / s').  p = 1 and s' = s except for
// 0 < s < 2^-90 (IEEE quotient tiles), where p = 2^64 and s' = s 2^64: both
// scalings are exact and x p / s' = x / s, and s' >= 2^-85 lies in the range
// where the corrected reciprocal gives the correctly rounded quotient.
__device__ __forceinline__ float4 pass_record(const TileScale& t)
{
    if (t.mode == 2) {
        const float sp = t.s * 0x1p64f;
        return make_float4(sp, 1.0f / sp, 0x1p64f, 0.0f);
    }
    return make_float4(t.s, t.y, 1.0f, 0.0f);
}

typedef float f2 __attribute__((ext_vector_type(2)));
// one 8-byte LDS read, not merged with its neighbours into a two-address read
typedef const volatile __attribute__((address_space(3))) f2 lds_f2;
__device__ __forceinline__ f2 lds_pair(const f2* p) { return *(lds_f2*)p; }

// Four values of one tile -> four codes.  FAST: every tile of the block has
// s >= 2^-90 or s = 0 (fp32 scales), or power-of-two scales; then s is
// normal, RN(amax / 448) is within 2^-24 relative of amax / 448, every
// quotient is at most 448 (1 + 2^-23) in magnitude and the clamp is not
// needed.  Otherwise the pre-scaled quotient and the clamp at 448 (a
// subnormal s can be far below amax / 448).
template <typename S, bool FAST>
__device__ __forceinline__ uint32_t quant4_as(float a, float b, float c, float d, f2 sy, float pre)
{
    if constexpr (sizeof(S) != 4) {
        return pack4_inrange(a * sy.y, b * sy.y, c * sy.y, d * sy.y);
    } else if constexpr (FAST) {
        return pack4_inrange(quotient_fast(a, sy.x, sy.y), quotient_fast(b, sy.x, sy.y), quotient_fast(c, sy.x, sy.y),
                             quotient_fast(d, sy.x, sy.y));
    } else {
        return pack4_e4m3(quotient_fast(a * pre, sy.x, sy.y), quotient_fast(b * pre, sy.x, sy.y),
                          quotient_fast(c * pre, sy.x, sy.y), quotient_fast(d * pre, sy.x, sy.y));
    }
}

static_assert(kQtRows == 4, "four rows per thread (one 16-byte write of the row maxima)");

template <typename T, typename S>
__global__ __launch_bounds__(kQtThreads) void quant_transpose_kernel(
    const T* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
    uint8_t* __restrict__ q_row, int64_t ldq_row, S* __restrict__ s_row, int64_t lds_row,
    uint8_t* __restrict__ q_colT, int64_t ldq_colT, S* __restrict__ s_colT, int64_t lds_colT,
    FastDiv blocks_per_row)
{
    __shared__ uint32_t col_part[kQtGroups * kColPitch];   // per row-group column maxima (|x| bits)
    __shared__ __attribute__((aligned(16))) uint32_t row_amax[kTile];
    __shared__ f2 col_sy[kTile];
    __shared__ f2 row_sy[kTile];
    __shared__ float col_pre[kTile], row_pre[kTile];
    __shared__ __attribute__((aligned(16))) int slow_wave[4];
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

        // row maxima (DPP over the 16 lanes of each row, the four rows'
        // steps interleaved), column partial maxima
        {
            uint32_t mb[kQtRows];
#pragma unroll
            for (int u = 0; u < kQtRows; ++u) {
                float m = fmaxf(fmaxf(fabsf(v[u][0]), fabsf(v[u][1])), fabsf(v[u][2]));
                m = fmaxf(fmaxf(m, fabsf(v[u][3])), fabsf(v[u][4]));
                m = fmaxf(fmaxf(m, fabsf(v[u][5])), fabsf(v[u][6]));
                mb[u] = __float_as_uint(fmaxf(m, fabsf(v[u][7])));
            }
            dpp_umax16x4(mb);
            if (l == 0) *reinterpret_cast<uint4*>(&row_amax[kQtRows * g]) = make_uint4(mb[0], mb[1], mb[2], mb[3]);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float cm = fmaxf(fmaxf(fmaxf(fabsf(v[0][j]), fabsf(v[1][j])), fabsf(v[2][j])), fabsf(v[3][j]));
                col_part[g * kColPitch + colmax_idx(8 * l + j)] = __float_as_uint(cm);
            }
        }
        __syncthreads();

        // one thread per column (tid < 128) and per row (128 <= tid < 256)
        if (tid < 2 * kTile) {
            TileScale ts;
            if (tid < kTile) {
                const int ci = colmax_idx(tid);
                uint32_t m = col_part[ci];
#pragma unroll
                for (int k = 1; k < kQtGroups; ++k) m = max(m, col_part[k * kColPitch + ci]);
                ts = make_tile_scale<S>(__uint_as_float(m));
                const float4 pr = pass_record(ts);
                col_sy[csy_idx(tid)] = f2{pr.x, pr.y};
                col_pre[tid] = pr.z;
                if (do_col && (FULL || c0 + tid < cols))
                    s_colT[(c0 + tid) * lds_colT + rb] = stored_scale<S>(ts);
            } else {
                const int i = tid - kTile;
                ts = make_tile_scale<S>(__uint_as_float(row_amax[i]));
                const float4 pr = pass_record(ts);
                row_sy[i] = f2{pr.x, pr.y};
                row_pre[i] = pr.z;
                if (do_row && (FULL || r0 + i < rows))
                    s_row[(r0 + i) * lds_row + cb] = stored_scale<S>(ts);
            }
            // waves 0-3: does any of their tiles need the IEEE quotient
            const bool any_slow = __builtin_amdgcn_ballot_w64(ts.mode == 2) != 0;
            if ((tid & 63) == 0) slow_wave[tid >> 6] = any_slow ? 1 : 0;
        }
        __syncthreads();

        auto passes = [&](auto fast_tag) {
            constexpr bool FAST = decltype(fast_tag)::value;
            if (do_row) {
                const int64_t c = c0 + 8 * l;
                uint8_t* const qb = q_row + (r0 + kQtRows * g) * ldq_row + c;
#pragma unroll
                for (int u = 0; u < kQtRows; ++u) {
                    const int i = kQtRows * g + u;
                    const f2 sy = lds_pair(&row_sy[i]);
                    const float pre = FAST ? 1.0f : row_pre[i];
                    const uint32_t lo = quant4_as<S, FAST>(v[u][0], v[u][1], v[u][2], v[u][3], sy, pre);
                    const uint32_t hi = quant4_as<S, FAST>(v[u][4], v[u][5], v[u][6], v[u][7], sy, pre);
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
                const int pos = 4 * ((g & 3) ^ (2 * (l >> 3)));
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int cj = 8 * l + j;
                    const f2 sy = lds_pair(&col_sy[csy_idx(cj)]);
                    const float pre = FAST ? 1.0f : col_pre[cj];
                    const uint32_t w = quant4_as<S, FAST>(v[0][j], v[1][j], v[2][j], v[3][j], sy, pre);
                    *reinterpret_cast<uint32_t*>(stage + cj * kStagePitch + 16 * ((g >> 2) ^ stage_key(cj)) + pos) = w;
                }
            }
        };
        const int4 sw = *reinterpret_cast<const int4*>(slow_wave);
        if (sizeof(S) != 4 || __builtin_amdgcn_readfirstlane(sw.x | sw.y | sw.z | sw.w) == 0)
            passes(std::true_type{});
        else
            passes(std::false_type{});

        if (do_col) {
            __syncthreads();
            // 8 threads per X^T row (16 bytes each), 64 rows per pass; rows
            // 64..127 hold their dwords in the order 2, 3, 0, 1
#pragma unroll
            for (int pass = 0; pass < kTile / (kQtThreads / 8); ++pass) {
                const int cr = pass * (kQtThreads / 8) + (tid >> 3);   // row of the staged X^T block
                const int seg = (tid & 7) * 16;              // byte offset along X's rows
                const int64_t cglob = c0 + cr;
                const int64_t rglob = r0 + seg;
                uint4 w = *reinterpret_cast<const uint4*>(stage + cr * kStagePitch + 16 * ((tid & 7) ^ stage_key(cr)));
                if (pass == 1) w = make_uint4(w.z, w.w, w.x, w.y);
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
