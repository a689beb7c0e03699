// LDS layouts, buffer-resource loads and LDS read helpers shared by the
// block-scaled GEMM kernels on gfx950 (gemm_nk.hip, gemm_w4.hip): the 128 x
// 256 x 128 tile geometry, the XOR-swizzled 16-byte slots of K-contiguous
// stages, the [K][N] stage key, direct global -> LDS loads and the inline-asm
// LDS reads.
#pragma once

#include "gemm_common.h"

namespace fp8q {

namespace {

constexpr int TBM = 128;
constexpr int TBN = 256;
constexpr int TBK = 128;
constexpr int WTN = 64;              // columns per wave (all TBM rows)
constexpr int PMI = TBM / 16;        // 16-row blocks per wave
constexpr int NNI = WTN / 16;        // 16-column blocks per wave
constexpr int kStages = 3;
constexpr int kGroupM = 16;
constexpr int kAStage = TBM * TBK;   // bytes
constexpr int kBStage = TBN * TBK;
constexpr int kStageBytes = kAStage + kBStage; // A at 0, B at kAStage
// groups whose offsets fit in LDS (grouped launches with more are unsupported)
constexpr int kMaxLdsGroups = 1024;

typedef __attribute__((address_space(3))) void lds_void_t;

// 16-byte slot of logical chunk `chunk` in LDS row `row`.  The XOR key
// (row & 7) ^ ((row >> 3) & 1) makes the fragment reads (lane l: row
// 16 b + l % 16, chunk 2 (l / 16) + h) free of bank conflicts on gfx950
// (measured with SQ_LDS_BANK_CONFLICT; the keys row & 7 and (row >> 1) & 7
// conflict on a quarter of the cycles).  It depends on the row's low 4 bits
// only, so the fragment of block b is the fragment of block 0 plus b rows of 16.
__device__ __forceinline__ int swz_key(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int sw(int row, int chunk) { return row * TBK + ((chunk ^ swz_key(row)) << 4); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             (int)(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF), 0x00020000);
}

// One DMA wave-instruction fills 8 LDS rows (1 KB): lane l writes slot l & 7
// of row r0 + l / 8, which holds logical chunk (l & 7) ^ key(row).  The
// per-lane source offset (relative to the operand base, without the chunk's
// k0) is fixed for the whole K loop.  Rows past the operand's last row
// re-read the last row: they only feed outputs that are never stored.
__device__ __forceinline__ uint32_t dma_src_off(int r0, int lane, int64_t row0, int64_t rows_valid, int64_t ld)
{
    const int r = r0 + (lane >> 3);
    int64_t g = row0 + r;
    g = g < rows_valid ? g : rows_valid - 1;
    return (uint32_t)(g * ld + 16 * ((lane & 7) ^ swz_key(r)));
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, uint8_t* lds_rows, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds_rows, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t rs, float* lds_words, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds_words, 4, voff, soff, 0, 0);
}

// the same with the LDS destination given as a (wave-uniform) LDS address
__device__ __forceinline__ void dma16_at(__amdgpu_buffer_rsrc_t rs, uint32_t lds, uint32_t voff, uint32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(uintptr_t)lds, 16, voff, soff, 0, 0);
}

// waits until at most N LDS (or scalar) reads are pending; x is an operand
// so that its users stay below the wait
template <int N>
__device__ __forceinline__ void lgkm_wait(v8i& x)
{
    static_assert(N >= 0 && N < 16, "lgkmcnt immediate");
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "n"(N));
}

__device__ __forceinline__ void pin4(v8i& a, v8i& b, v8i& c, v8i& d)
{
    asm volatile("" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}

template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 16, "vmcnt immediate");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS reads of the compute phase are issued as inline asm, outside the
// compiler's view of LDS: otherwise it cannot tell the three stages apart
// and waits for every in-flight LDS DMA (vmcnt(0)) before each read, which
// serialises the load pipeline.  The one explicit lgkmcnt(0) below takes the
// loaded registers as operands, so every consumer is ordered after it.
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;
typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t lds_addr(const void* ptr) { return (uint32_t)(uintptr_t)(const lds_u8_t*)ptr; }

template <int OFF>
__device__ __forceinline__ v4i ds128(uint32_t addr)
{
    v4i v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}

template <int OFF>
__device__ __forceinline__ float ds32(uint32_t addr)
{
    float v;
    asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}

// one byte of LDS, zero-extended (the E8M0 scale bytes)
template <int OFF>
__device__ __forceinline__ int ds_u8(uint32_t addr)
{
    int v;
    asm volatile("ds_read_u8 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}

typedef int v2i __attribute__((ext_vector_type(2)));

// Transposing LDS read: within each 16-lane group, lane i receives byte
// (i & 7) of the 8-byte rows addressed by lanes 2j + (i >> 3), j = 0..7
// (measured on gfx950).  With those lanes pointing at 8 consecutive K rows of
// a [K][N] tile at columns n0 + 8 (i >> 3), lane i gets 8 consecutive K
// values of column n0 + i.
template <int OFF>
__device__ __forceinline__ v2i ds64tr(uint32_t addr)
{
    v2i v;
    asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}

__device__ __forceinline__ v8i cat4(v2i a, v2i b, v2i c, v2i d)
{
    return v8i{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// [K][N] operand stage: row r (a K index) holds 256 column bytes as 16
// slots of 16; slot = chunk ^ key(r).  The low 3 key bits spread the 8 rows
// one 16-lane group reads over distinct banks; bit 3 (from r & 32) puts
// neighbouring groups, 32 rows apart, in opposite halves of the bank space.
__device__ __forceinline__ int kn_key(int row) { return (row & 7) ^ ((row >> 2) & 8); }

__device__ __forceinline__ v8i cat(v4i lo, v4i hi)
{
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace

}  // namespace fp8q
