// Element loads and code stores of the quantizer kernels (quant.hip,
// quant_transpose.hip): 16-byte vector accesses of 8 consecutive elements,
// bf16 or fp32 in, E4M3 codes out.
#pragma once

#include "fp8q_device.h"

namespace fp8q {

// Loads elements [c, c+8) of a row into v[0..7]; elements at or beyond `cols`
// read as 0 (the 16-byte vectors never cross ld, see the ABI).
template <typename T>
__device__ __forceinline__ void load8(const T* row, int64_t c, int64_t cols, float v[8]);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* row, int64_t c, int64_t cols, float v[8])
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
__device__ __forceinline__ void load8<float>(const float* row, int64_t c, int64_t cols, float v[8])
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

__device__ __forceinline__ float absmax8(const float v[8])
{
    float m = fmaxf(fabsf(v[0]), fabsf(v[1]));
    m = fmaxf(m, fmaxf(fabsf(v[2]), fabsf(v[3])));
    m = fmaxf(m, fmaxf(fabsf(v[4]), fabsf(v[5])));
    m = fmaxf(m, fmaxf(fabsf(v[6]), fabsf(v[7])));
    return m;
}

// Stores 8 codes at q[c..c+8), clipped at `cols`.
__device__ __forceinline__ void store8(uint8_t* qrow, int64_t c, int64_t cols, uint32_t lo, uint32_t hi)
{
    if (c + 8 <= cols) {
        *reinterpret_cast<uint2*>(qrow + c) = make_uint2(lo, hi);
    } else {
        for (int i = 0; i < 8 && c + i < cols; ++i)
            qrow[c + i] = (uint8_t)((i < 4 ? lo >> (8 * i) : hi >> (8 * (i - 4))) & 0xFF);
    }
}

// Raw registers of 8 consecutive elements, so that loads can be issued a
// step ahead of their use and converted afterwards.
template <typename T> struct Raw8;
template <> struct Raw8<uint16_t> { uint4 v; };
template <> struct Raw8<float> { uint4 a, b; };

// Loads elements [c, c+8) of a row (c a multiple of 8).  For c < cols the
// 16-byte vectors lie within ld (see the ABI); c >= cols loads nothing.
__device__ __forceinline__ void raw_load(const uint16_t* row, int64_t c, int64_t cols, Raw8<uint16_t>& r)
{
    r.v = c < cols ? *reinterpret_cast<const uint4*>(row + c) : make_uint4(0, 0, 0, 0);
}
__device__ __forceinline__ void raw_load(const float* row, int64_t c, int64_t cols, Raw8<float>& r)
{
    r.a = c < cols ? *reinterpret_cast<const uint4*>(row + c) : make_uint4(0, 0, 0, 0);
    r.b = c + 4 < cols ? *reinterpret_cast<const uint4*>(row + c + 4) : make_uint4(0, 0, 0, 0);
}

// Loads and fp32 values of 8 elements known to lie inside the matrix (no
// bounds tests: blocks away from the right and bottom edges).
__device__ __forceinline__ void raw_load_full(const uint16_t* p, Raw8<uint16_t>& r)
{
    r.v = *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void raw_load_full(const float* p, Raw8<float>& r)
{
    r.a = *reinterpret_cast<const uint4*>(p);
    r.b = *reinterpret_cast<const uint4*>(p + 4);
}
__device__ __forceinline__ void raw_f32_full(const Raw8<uint16_t>& r, float v[8])
{
    v[0] = bf16_lo(r.v.x); v[1] = bf16_hi(r.v.x);
    v[2] = bf16_lo(r.v.y); v[3] = bf16_hi(r.v.y);
    v[4] = bf16_lo(r.v.z); v[5] = bf16_hi(r.v.z);
    v[6] = bf16_lo(r.v.w); v[7] = bf16_hi(r.v.w);
}
__device__ __forceinline__ void raw_f32_full(const Raw8<float>& r, float v[8])
{
    v[0] = __uint_as_float(r.a.x); v[1] = __uint_as_float(r.a.y);
    v[2] = __uint_as_float(r.a.z); v[3] = __uint_as_float(r.a.w);
    v[4] = __uint_as_float(r.b.x); v[5] = __uint_as_float(r.b.y);
    v[6] = __uint_as_float(r.b.z); v[7] = __uint_as_float(r.b.w);
}

// fp32 values of a raw load; elements at or beyond `cols` become 0.
__device__ __forceinline__ void raw_f32(const Raw8<uint16_t>& r, int64_t c, int64_t cols, float v[8])
{
    v[0] = bf16_lo(r.v.x); v[1] = bf16_hi(r.v.x);
    v[2] = bf16_lo(r.v.y); v[3] = bf16_hi(r.v.y);
    v[4] = bf16_lo(r.v.z); v[5] = bf16_hi(r.v.z);
    v[6] = bf16_lo(r.v.w); v[7] = bf16_hi(r.v.w);
    if (c + 8 > cols) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (c + i >= cols) v[i] = 0.0f;
    }
}
__device__ __forceinline__ void raw_f32(const Raw8<float>& r, int64_t c, int64_t cols, float v[8])
{
    v[0] = __uint_as_float(r.a.x); v[1] = __uint_as_float(r.a.y);
    v[2] = __uint_as_float(r.a.z); v[3] = __uint_as_float(r.a.w);
    v[4] = __uint_as_float(r.b.x); v[5] = __uint_as_float(r.b.y);
    v[6] = __uint_as_float(r.b.z); v[7] = __uint_as_float(r.b.w);
    if (c + 8 > cols) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (c + i >= cols) v[i] = 0.0f;
    }
}

}  // namespace fp8q
