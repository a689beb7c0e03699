// Device-side helpers shared by the gfx950 kernels of libfp8q.
//
// Quantization rule (FP8-LM review, section 三: x_fp8 = Cast_FP8(x / s)),
// with s = amax / 448 per tile; E4M3 range [-448, 448] ("FP8-RL" article,
// section 一).  The cast is round-to-nearest-even with saturation; the fp32
// quotient x / s is rounded once (IEEE) before the cast.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kTile = 128;
constexpr float kE4M3Max = 448.0f;
// Below this scale the corrected-reciprocal quotient can lose its exact
// residual; such tiles divide with the IEEE quotient instead.
constexpr float kFastScaleMin = 0x1p-90f;

// bf16 -> fp32 as a floating-point extension (exact; the compiler then knows
// the values are canonical and forms |x| maxima without quieting steps)
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return (float)__builtin_bit_cast(__bf16, (uint16_t)(pair & 0xFFFFu)); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return (float)__builtin_bit_cast(__bf16, (uint16_t)(pair >> 16)); }

// |x| max across the 16 lanes of a DPP row (lanes 16r .. 16r+15), for
// non-negative v: such floats order like their bit patterns, so the steps
// are integer maxima (no quieting steps; inputs are finite by contract).
// All lanes of the wave must be active.
__device__ __forceinline__ float dpp_max16(float v)
{
    uint32_t u = __float_as_uint(v);
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x141, 0xF, 0xF, false));  // half-row mirror
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x140, 0xF, 0xF, false));  // row mirror
    return __uint_as_float(u);
}

// Per-tile quantization constants: the scale s, its correctly rounded
// reciprocal y, and which division path the tile takes.
struct TileScale {
    float s;
    float y;
    int mode;   // 0: s == 0 (signed zeros), 1: corrected reciprocal, 2: IEEE quotient,
                // 3: power of two (x * y is exact)
};

__device__ __forceinline__ TileScale make_scale(float amax)
{
    TileScale t;
    t.s = amax / kE4M3Max;                 // IEEE fp32 division
    t.mode = t.s == 0.0f ? 0 : (t.s >= kFastScaleMin ? 1 : 2);
    t.y = t.mode == 1 ? 1.0f / t.s : 0.0f; // IEEE fp32 reciprocal
    return t;
}

// RN_fp32(x / s).  mode 1: q0 = RN(x*y) is within an ulp of x/s, the
// residual e = q0*s - x is exact (FMA, no underflow for s >= 2^-90 and the
// quotients that can round to a non-zero code), and RN(q0 - e*y) is the
// correctly rounded quotient (Markstein's theorem; Muller et al., Handbook
// of Floating-Point Arithmetic, division with an FMA).  The residual is
// formed as q0*s - x rather than x - q0*s so that x = -0 yields -0 (the sum
// of opposite zeros rounds to +0).
__device__ __forceinline__ float quotient(float x, const TileScale& t)
{
    if (t.mode == 1) {
        float q0 = x * t.y;
        float e = __builtin_fmaf(q0, t.s, -x);
        return __builtin_fmaf(-e, t.y, q0);
    }
    return x / t.s;
}

// Four fp32 values -> four E4M3 codes packed little-endian in a dword.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d)
{
    a = __builtin_amdgcn_fmed3f(a, -kE4M3Max, kE4M3Max);
    b = __builtin_amdgcn_fmed3f(b, -kE4M3Max, kE4M3Max);
    c = __builtin_amdgcn_fmed3f(c, -kE4M3Max, kE4M3Max);
    d = __builtin_amdgcn_fmed3f(d, -kE4M3Max, kE4M3Max);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// The same for values with |v| <= 448 (1 + 2^-23): their nearest E4M3 value
// is at most 448, so the conversion needs no clamp.  That holds for every
// quotient x / s of a tile with s = RN(amax / 448) normal and amax the
// tile's max |x| (s is within 2^-24 relative of amax / 448), and for x * 2^-e
// with power-of-two scales.
__device__ __forceinline__ uint32_t pack4_inrange(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Quantize four values of one tile.
__device__ __forceinline__ uint32_t quant4(float a, float b, float c, float d, const TileScale& t)
{
    if (t.mode == 0) {
        return ((__float_as_uint(a) >> 31) << 7) | ((__float_as_uint(b) >> 31) << 15) |
               ((__float_as_uint(c) >> 31) << 23) | ((__float_as_uint(d) >> 31) << 31);
    }
    return pack4_e4m3(quotient(a, t), quotient(b, t), quotient(c, t), quotient(d, t));
}

// Eight values of one tile -> eight codes (lo: values 0-3, hi: 4-7).  Tiles
// with s >= 2^-90 and zero tiles (s = 0, y = 0: the corrected reciprocal
// then yields x's signed zero) take the branch-free corrected reciprocal;
// only if some lane of the wave holds a tile with 0 < s < 2^-90 does the
// wave take the general path.
__device__ __forceinline__ void quant8(const float v[8], const TileScale& t, uint32_t& lo, uint32_t& hi)
{
    if (__builtin_amdgcn_ballot_w64(t.mode == 2) == 0) {
        float q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float q0 = v[i] * t.y;
            const float e = __builtin_fmaf(q0, t.s, -v[i]);
            q[i] = __builtin_fmaf(-e, t.y, q0);
        }
        lo = pack4_inrange(q[0], q[1], q[2], q[3]);
        hi = pack4_inrange(q[4], q[5], q[6], q[7]);
    } else {
        lo = quant4(v[0], v[1], v[2], v[3], t);
        hi = quant4(v[4], v[5], v[6], v[7], t);
    }
}

// Power-of-two scales, stored as E8M0 exponent bytes (the micro-scaling
// variant of block scaling; Introl FP8 infrastructure guide, scaling
// strategies and the Blackwell section).  s = 2^e with e the smallest integer
// >= -126 such that amax <= 448 * 2^e.  With amax = m * 2^k (1 <= m < 2) and
// 448 = 1.75 * 2^8 that is e = k - 8 if m <= 1.75 (mantissa field at most
// 0x600000), else k - 7; a zero or subnormal amax gives the floor -126.  The
// quotient x / s = x * 2^-e is then exact (or below 2^-126, where every code
// is a signed zero), so no division is needed, and |x / s| <= 448.
__device__ __forceinline__ int pow2_exponent(float amax)
{
    const uint32_t u = __float_as_uint(amax);
    if (u < 0x00800000u) return -126;
    const int e = (int)(u >> 23) - 135 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    return e < -126 ? -126 : e;
}

// Tile constants for a scale stored as S: float (s = amax / 448) or uint8_t
// (E8M0 byte of a power-of-two s; mode 3, y = 2^-e exactly).
template <typename S> __device__ __forceinline__ TileScale make_tile_scale(float amax);
template <> __device__ __forceinline__ TileScale make_tile_scale<float>(float amax) { return make_scale(amax); }
template <> __device__ __forceinline__ TileScale make_tile_scale<uint8_t>(float amax)
{
    const int e = pow2_exponent(amax);
    TileScale t;
    t.s = __uint_as_float((uint32_t)(e + 127) << 23);
    t.y = __uint_as_float((uint32_t)(127 - e) << 23);
    t.mode = 3;
    return t;
}

template <typename S> __device__ __forceinline__ S stored_scale(const TileScale& t);
template <> __device__ __forceinline__ float stored_scale<float>(const TileScale& t) { return t.s; }
template <> __device__ __forceinline__ uint8_t stored_scale<uint8_t>(const TileScale& t)
{
    return (uint8_t)(__float_as_uint(t.s) >> 23);
}

template <typename S>
__device__ __forceinline__ void quant8_as(const float v[8], const TileScale& t, uint32_t& lo, uint32_t& hi)
{
    if constexpr (sizeof(S) == 4) {
        quant8(v, t, lo, hi);
    } else {
        lo = pack4_inrange(v[0] * t.y, v[1] * t.y, v[2] * t.y, v[3] * t.y);
        hi = pack4_inrange(v[4] * t.y, v[5] * t.y, v[6] * t.y, v[7] * t.y);
    }
}

// Magic-number unsigned division by a runtime constant (Granlund-Montgomery),
// for 32-bit numerators.
struct FastDiv {
    uint32_t d, m, sh;
};

__host__ inline FastDiv make_fastdiv(uint32_t d)
{
    FastDiv f;
    f.d = d;
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    f.sh = s;
    f.m = (uint32_t)((((1ull << 32) * ((1ull << s) - d)) / d) + 1);
    return f;
}

__host__ __device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f)
{
    if (f.d == 1)
        return n;
    uint32_t t = (uint32_t)(((uint64_t)n * f.m) >> 32);
    return (t + ((n - t) >> 1)) >> (f.sh - 1);
}

}  // namespace fp8q
