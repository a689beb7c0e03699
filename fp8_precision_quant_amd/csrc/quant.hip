// Tile quantizers for gfx950: 1x128 row tiles, 128x128 blocks and one scale
// per tensor; the tile kernels also write power-of-two scales as E8M0 bytes.
//
// Per tile: amax = max |x|, s = amax / 448, code = E4M3(RN(x / s)) (FP8-LM
// review, section 三, tensor scaling; Ling 2.0 FP8 blog, fine-grained
// per-tile/block scaling; 128x128 weight blocks: "FP8-RL" article, section
// 一).  These kernels are HBM-bound streams: 16-byte loads and stores, the
// amax reduction in registers and DPP, no LDS round trip for row tiles.
#include "fp8q_device.h"
#include "fp8q_internal.h"
#include "quant_io.h"

namespace fp8q {

// ---------------------------------------------------------------------------
// 1x128 row tiles
// ---------------------------------------------------------------------------
// A 16-lane DPP row owns one tile (8 elements per lane).  A 256-thread
// workgroup covers 16 consecutive tiles per step and runs U steps with all
// loads issued first, so each lane keeps U 16-byte loads (2U for fp32 input)
// in flight.  U = 1 (more, shorter workgroups) is fastest up to ~2^19 tiles
// (x 4096 x 4096: 12 us against 15 us with U = 4), U = 2 above (16384 x 8192:
// 74 us against 77 us).

constexpr int kRowThreads = 256;
constexpr uint32_t kRowSmallTiles = 1u << 19;

template <typename T, typename S, int U>
__global__ __launch_bounds__(kRowThreads) void quant_row_kernel(
    const T* __restrict__ x, int64_t cols, int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
    S* __restrict__ s, int64_t lds, uint32_t total_tiles, FastDiv tiles_per_row)
{
    constexpr int kRowUnroll = U;
    constexpr int kRowTilesPerBlock = (kRowThreads / 16) * kRowUnroll;
    const int lane16 = threadIdx.x & 15;
    const int group = threadIdx.x >> 4;
    const uint32_t base = blockIdx.x * kRowTilesPerBlock;

    float v[kRowUnroll][8];
    uint32_t row[kRowUnroll], tcol[kRowUnroll];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
        uint32_t t = base + u * (kRowThreads / 16) + group;
        bool live = t < total_tiles;
        uint32_t r = fdiv(live ? t : 0, tiles_per_row);
        row[u] = r;
        tcol[u] = (live ? t : 0) - r * tiles_per_row.d;
        int64_t c = (int64_t)tcol[u] * kTile + lane16 * 8;
        load8<T>(x + (int64_t)r * ldx, live ? c : cols, cols, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
        uint32_t t = base + u * (kRowThreads / 16) + group;
        float amax = dpp_max16(absmax8(v[u]));
        TileScale ts = make_tile_scale<S>(amax);
        uint32_t lo, hi;
        quant8_as<S>(v[u], ts, lo, hi);
        if (t < total_tiles) {
            int64_t c = (int64_t)tcol[u] * kTile + lane16 * 8;
            if (c < cols)
                store8(q + (int64_t)row[u] * ldq, c, cols, lo, hi);
            if (lane16 == 0)
                s[(int64_t)row[u] * lds + tcol[u]] = stored_scale<S>(ts);
        }
    }
}

// ---------------------------------------------------------------------------
// 128x128 blocks
// ---------------------------------------------------------------------------
// A 512-thread workgroup quantizes blocks b = blockIdx.x + i * gridDim.x:
// thread (g = tid/16, l = tid%16) holds rows g, g+32, g+64, g+96 at columns
// 8l..8l+7 (32 values), the block amax is reduced with DPP, readlane and LDS,
// then every value is cast.  The next block's loads are issued before the
// current block is reduced.  (512 threads with 4 rows each fit four waves
// per SIMD; 256 threads with 8 rows each took twice the registers and were
// 9% slower on a 14336 x 4096 weight.)

constexpr int kBlockThreads = 512;
constexpr int kBlockRows = kTile / (kBlockThreads / 16);   // rows per thread

template <typename T, typename S>
__global__ __launch_bounds__(kBlockThreads) void quant_block_kernel(
    const T* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* __restrict__ q,
    int64_t ldq, S* __restrict__ s, int64_t lds, uint32_t total_blocks, FastDiv blocks_per_row)
{
    __shared__ float wave_max[2][kBlockThreads / 64];
    const int l = threadIdx.x & 15;
    const int g = threadIdx.x >> 4;

    auto origin = [&](uint32_t b, int64_t& r0, int64_t& c) {
        const uint32_t br = fdiv(b, blocks_per_row);
        r0 = (int64_t)br * kTile;
        c = (int64_t)(b - br * blocks_per_row.d) * kTile + l * 8;
    };
    // a block inside the matrix needs no bounds test on any element
    auto interior = [&](int64_t r0, int64_t c) { return r0 + kTile <= rows && c - l * 8 + kTile <= cols; };
    auto load = [&](uint32_t b, Raw8<T>* R) {
        int64_t r0, c;
        origin(b, r0, c);
        if (interior(r0, c)) {
            const T* xb = x + (r0 + g) * ldx + c;
#pragma unroll
            for (int u = 0; u < kBlockRows; ++u) raw_load_full(xb + (kBlockThreads / 16) * u * ldx, R[u]);
            return;
        }
#pragma unroll
        for (int u = 0; u < kBlockRows; ++u) {
            const int64_t r = r0 + g + (kBlockThreads / 16) * u;
            raw_load(x + (r < rows ? r : 0) * ldx, r < rows ? c : cols, cols, R[u]);
        }
    };
    auto quantize = [&](uint32_t b, const Raw8<T>* R, int parity) {
        int64_t r0, c;
        origin(b, r0, c);
        const bool full = interior(r0, c);
        float v[kBlockRows][8];
        if (full) {
#pragma unroll
            for (int u = 0; u < kBlockRows; ++u) raw_f32_full(R[u], v[u]);
        } else {
#pragma unroll
            for (int u = 0; u < kBlockRows; ++u) raw_f32(R[u], c, cols, v[u]);
        }
        float m = 0.0f;
#pragma unroll
        for (int u = 0; u < kBlockRows; ++u) m = fmaxf(m, absmax8(v[u]));
        m = dpp_max16(m);
        m = fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 0)),
                        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 16))),
                  fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 32)),
                        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 48))));
        // two alternating slots: a wave that runs ahead into the next block
        // writes the other slot, so one barrier per block suffices
        if ((threadIdx.x & 63) == 0)
            wave_max[parity][threadIdx.x >> 6] = m;
        __syncthreads();
        float amax = wave_max[parity][0];
#pragma unroll
        for (int w = 1; w < kBlockThreads / 64; ++w) amax = fmaxf(amax, wave_max[parity][w]);
        const TileScale ts = make_tile_scale<S>(amax);
        uint8_t* const qb = q + (r0 + g) * ldq + c;
#pragma unroll
        for (int u = 0; u < kBlockRows; ++u) {
            const int64_t r = r0 + g + (kBlockThreads / 16) * u;
            uint32_t lo, hi;
            quant8_as<S>(v[u], ts, lo, hi);
            if (full)
                *reinterpret_cast<uint2*>(qb + (kBlockThreads / 16) * u * ldq) = make_uint2(lo, hi);
            else if (r < rows && c < cols)
                store8(q + r * ldq, c, cols, lo, hi);
        }
        if (threadIdx.x == 0)
            s[(int64_t)(r0 / kTile) * lds + (c - l * 8) / kTile] = stored_scale<S>(ts);
    };

    Raw8<T> A[kBlockRows], B[kBlockRows];
    uint32_t b = blockIdx.x;
    if (b >= total_blocks) return;
    load(b, A);
    for (;;) {
        const uint32_t b1 = b + gridDim.x;
        if (b1 < total_blocks) load(b1, B);
        quantize(b, A, 0);
        if (b1 >= total_blocks) break;
        const uint32_t b2 = b1 + gridDim.x;
        if (b2 < total_blocks) load(b2, A);
        quantize(b1, B, 1);
        if (b2 >= total_blocks) break;
        b = b2;
    }
}

// ---------------------------------------------------------------------------
// one scale per tensor: fill -> amax (atomic max on the fp32 bits, which
// order like the values for non-negative floats) -> cast -> store the scale.
// s[0] holds the amax bits until the last kernel replaces it by amax/448.
// ---------------------------------------------------------------------------

__global__ void tensor_fill_kernel(uint32_t* cell) { *cell = 0u; }

constexpr int kTensorThreads = 256;

template <typename T>
__global__ __launch_bounds__(kTensorThreads) void tensor_amax_kernel(
    const T* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, uint32_t* cell,
    FastDiv chunks_per_row, uint32_t total_chunks)
{
    __shared__ float wave_max[kTensorThreads / 64];
    float m = 0.0f;
    for (uint32_t i = blockIdx.x * kTensorThreads + threadIdx.x; i < total_chunks;
         i += gridDim.x * kTensorThreads) {
        uint32_t r = fdiv(i, chunks_per_row);
        int64_t c = (int64_t)(i - r * chunks_per_row.d) * 8;
        float v[8];
        load8<T>(x + (int64_t)r * ldx, c, cols, v);
        m = fmaxf(m, absmax8(v));
    }
    m = dpp_max16(m);
    m = fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 0)),
                    __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 16))),
              fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 32)),
                    __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 48))));
    if ((threadIdx.x & 63) == 0)
        wave_max[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float b = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
        atomicMax(cell, __float_as_uint(b));
    }
}

template <typename T>
__global__ __launch_bounds__(kTensorThreads) void tensor_cast_kernel(
    const T* __restrict__ x, int64_t cols, int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
    const uint32_t* cell, FastDiv chunks_per_row, uint32_t total_chunks)
{
    TileScale ts = make_scale(__uint_as_float(*cell));
    for (uint32_t i = blockIdx.x * kTensorThreads + threadIdx.x; i < total_chunks;
         i += gridDim.x * kTensorThreads) {
        uint32_t r = fdiv(i, chunks_per_row);
        int64_t c = (int64_t)(i - r * chunks_per_row.d) * 8;
        float v[8];
        load8<T>(x + (int64_t)r * ldx, c, cols, v);
        uint32_t lo, hi;
        quant8(v, ts, lo, hi);
        store8(q + (int64_t)r * ldq, c, cols, lo, hi);
    }
}

__global__ void tensor_finish_kernel(uint32_t* cell)
{
    float amax = __uint_as_float(*cell);
    *reinterpret_cast<float*>(cell) = amax / kE4M3Max;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

template <typename T, typename S>
static void launch_tiles(const void* xv, int64_t rows, int64_t cols, int64_t ldx, int kind,
                         uint8_t* q, int64_t ldq, S* s, int64_t lds, hipStream_t st)
{
    const T* x = static_cast<const T*>(xv);
    const int64_t tiles_c = (cols + kTile - 1) / kTile;
    const int64_t cus = device_cu_count();
    if (kind == FP8Q_ROW_1x128) {
        const uint32_t total = (uint32_t)(rows * tiles_c);
        if (total <= kRowSmallTiles) {
            const uint32_t blocks = (total + 15) / 16;
            hipLaunchKernelGGL((quant_row_kernel<T, S, 1>), dim3(blocks), dim3(kRowThreads), 0, st, x, cols,
                               ldx, q, ldq, s, lds, total, make_fastdiv((uint32_t)tiles_c));
        } else {
            const uint32_t blocks = (total + 31) / 32;
            hipLaunchKernelGGL((quant_row_kernel<T, S, 2>), dim3(blocks), dim3(kRowThreads), 0, st, x, cols,
                               ldx, q, ldq, s, lds, total, make_fastdiv((uint32_t)tiles_c));
        }
    } else {
        const uint32_t total = (uint32_t)(tiles_c * ((rows + kTile - 1) / kTile));
        // two resident 512-thread workgroups per CU (about 110 VGPRs per lane)
        uint32_t blocks = total < (uint32_t)(cus * 2) ? total : (uint32_t)(cus * 2);
        hipLaunchKernelGGL((quant_block_kernel<T, S>), dim3(blocks), dim3(kBlockThreads), 0, st, x,
                           rows, cols, ldx, q, ldq, s, lds, total, make_fastdiv((uint32_t)tiles_c));
    }
}

template <typename T>
static void launch_quant(const void* xv, int64_t rows, int64_t cols, int64_t ldx, int kind,
                         uint8_t* q, int64_t ldq, float* s, int64_t lds, hipStream_t st)
{
    if (kind != FP8Q_TENSOR) {
        launch_tiles<T, float>(xv, rows, cols, ldx, kind, q, ldq, s, lds, st);
    } else {
        const T* x = static_cast<const T*>(xv);
        uint32_t* cell = reinterpret_cast<uint32_t*>(s);
        int64_t cpr = (cols + 7) / 8;
        uint32_t total = (uint32_t)(rows * cpr);
        uint32_t blocks = (total + kTensorThreads - 1) / kTensorThreads;
        if (blocks > 4096) blocks = 4096;
        FastDiv fd = make_fastdiv((uint32_t)cpr);
        hipLaunchKernelGGL(tensor_fill_kernel, dim3(1), dim3(1), 0, st, cell);
        hipLaunchKernelGGL(tensor_amax_kernel<T>, dim3(blocks), dim3(kTensorThreads), 0, st, x,
                           rows, cols, ldx, cell, fd, total);
        hipLaunchKernelGGL(tensor_cast_kernel<T>, dim3(blocks), dim3(kTensorThreads), 0, st, x,
                           cols, ldx, q, ldq, cell, fd, total);
        hipLaunchKernelGGL(tensor_finish_kernel, dim3(1), dim3(1), 0, st, cell);
    }
}

void launch_quant_blockwise(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                            int kind, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                            hipStream_t st)
{
    if (x_dtype == FP8Q_BF16)
        launch_quant<uint16_t>(x, rows, cols, ldx, kind, q, ldq, s, lds, st);
    else
        launch_quant<float>(x, rows, cols, ldx, kind, q, ldq, s, lds, st);
}

void launch_quant_blockwise_e8m0(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                                 int kind, uint8_t* q, int64_t ldq, uint8_t* e, int64_t lde,
                                 hipStream_t st)
{
    if (x_dtype == FP8Q_BF16)
        launch_tiles<uint16_t, uint8_t>(x, rows, cols, ldx, kind, q, ldq, e, lde, st);
    else
        launch_tiles<float, uint8_t>(x, rows, cols, ldx, kind, q, ldq, e, lde, st);
}

}  // namespace fp8q
