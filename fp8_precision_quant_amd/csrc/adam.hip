// Fused AdamW step with FP8 moments for gfx950.
//
// Adam keeps two moments per parameter; holding both as E4M3 codes with one
// fp32 scale per 128 consecutive elements cuts their memory by about 74%
// against fp32 (Ling 2.0 FP8 blog, "FP8 Optimizer": both moments in FP8
// through fine-grained compression and decompression, after block-wise
// quantization).  One pass reads the parameters, the gradient and both coded
// moments, and writes the parameters and both moments re-quantized:
//   decode  m0 = dec(mq) * ms[block],  v0 = dec(vq) * vs[block];
//   step    p = p * decay;  m = b1 m0 + omb1 g;  v = b2 v0 + (omb2 g) g;
//           p = p - step_size * (m / (sqrt(v) / bc2_sqrt + eps));
//   encode  the 1x128 tile rule on m and v (s = amax / 448, exactly rounded
//           quotients, fp8q_device.h).
// Every fp32 operation is rounded once, in this order (no contraction into
// FMAs), so the result is bit-for-bit the definition.
//
// Layout: one 16-lane DPP row per 128-element block, 8 consecutive elements
// per lane: 32-byte parameter loads, 16-byte bf16 gradient loads, 8-byte code
// loads; the block amax of each moment is a DPP reduction within the row.
// A workgroup of 256 threads covers 16 blocks per step and runs kAdamUnroll
// steps with all loads issued first.  The pass is HBM-bound (about 14 bytes
// per parameter with a bf16 gradient).
#include "fp8q_device.h"
#include "fp8q_internal.h"

namespace fp8q {

constexpr int kAdamThreads = 256;
constexpr int kAdamUnroll = 2;
constexpr int kAdamBlocksPerWg = (kAdamThreads / 16) * kAdamUnroll;

typedef float v2f __attribute__((ext_vector_type(2)));

// eight E4M3 codes (little-endian in lo, hi) -> fp32 values (exact)
__device__ __forceinline__ void decode8(uint32_t lo, uint32_t hi, float v[8])
{
    const v2f a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
    const v2f b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
    const v2f c = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
    const v2f d = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
    v[0] = a.x; v[1] = a.y; v[2] = b.x; v[3] = b.y;
    v[4] = c.x; v[5] = c.y; v[6] = d.x; v[7] = d.y;
}

template <typename G>
__device__ __forceinline__ void load_grad8(const G* g, int64_t i0, int64_t n, float v[8]);

template <>
__device__ __forceinline__ void load_grad8<uint16_t>(const uint16_t* g, int64_t i0, int64_t n, float v[8])
{
    if (i0 + 8 <= n) {
        const uint4 w = *reinterpret_cast<const uint4*>(g + i0);
        v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
        v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
        v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
        v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = i0 + k < n ? __uint_as_float((uint32_t)g[i0 + k] << 16) : 0.0f;
    }
}

template <>
__device__ __forceinline__ void load_grad8<float>(const float* g, int64_t i0, int64_t n, float v[8])
{
    if (i0 + 8 <= n) {
        const float4 a = *reinterpret_cast<const float4*>(g + i0);
        const float4 b = *reinterpret_cast<const float4*>(g + i0 + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = i0 + k < n ? g[i0 + k] : 0.0f;
    }
}

// the eight values of a lane: parameters, gradient, decoded moments
struct AdamLane {
    float p[8], g[8], m[8], v[8];
};

template <typename G>
__global__ __launch_bounds__(kAdamThreads) void adam_fp8_kernel(
    float* __restrict__ p, const G* __restrict__ g, uint8_t* __restrict__ mq, float* __restrict__ ms,
    uint8_t* __restrict__ vq, float* __restrict__ vs, int64_t n, uint32_t nblocks, AdamScalars a)
{
#pragma clang fp contract(off)
    const int lane16 = threadIdx.x & 15;
    const int group = threadIdx.x >> 4;
    AdamLane L[kAdamUnroll];
    // loads first (blocks past the end, and elements past n, read as zero)
#pragma unroll
    for (int u = 0; u < kAdamUnroll; ++u) {
        const uint32_t b = (blockIdx.x * kAdamUnroll + u) * (kAdamThreads / 16) + group;
        const int64_t i0 = (int64_t)b * kTile + lane16 * 8;
        const bool live = b < nblocks && i0 < n;
        const int64_t e0 = live ? i0 : n;     // e0 >= n: nothing is read
        if (e0 + 8 <= n) {
            const float4 x = *reinterpret_cast<const float4*>(p + e0);
            const float4 y = *reinterpret_cast<const float4*>(p + e0 + 4);
            L[u].p[0] = x.x; L[u].p[1] = x.y; L[u].p[2] = x.z; L[u].p[3] = x.w;
            L[u].p[4] = y.x; L[u].p[5] = y.y; L[u].p[6] = y.z; L[u].p[7] = y.w;
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) L[u].p[k] = e0 + k < n ? p[e0 + k] : 0.0f;
        }
        load_grad8<G>(g, e0, n, L[u].g);
        uint32_t mlo = 0, mhi = 0, vlo = 0, vhi = 0;
        if (e0 + 8 <= n) {
            const uint2 mc = *reinterpret_cast<const uint2*>(mq + e0);
            const uint2 vc = *reinterpret_cast<const uint2*>(vq + e0);
            mlo = mc.x; mhi = mc.y; vlo = vc.x; vhi = vc.y;
        } else {
            for (int k = 0; k < 8 && e0 + k < n; ++k) {
                (k < 4 ? mlo : mhi) |= (uint32_t)mq[e0 + k] << (8 * (k & 3));
                (k < 4 ? vlo : vhi) |= (uint32_t)vq[e0 + k] << (8 * (k & 3));
            }
        }
        const float sm = live ? ms[b] : 0.0f;
        const float sv = live ? vs[b] : 0.0f;
        decode8(mlo, mhi, L[u].m);
        decode8(vlo, vhi, L[u].v);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            L[u].m[k] = L[u].m[k] * sm;
            L[u].v[k] = L[u].v[k] * sv;
        }
    }
#pragma unroll
    for (int u = 0; u < kAdamUnroll; ++u) {
        const uint32_t b = (blockIdx.x * kAdamUnroll + u) * (kAdamThreads / 16) + group;
        const int64_t i0 = (int64_t)b * kTile + lane16 * 8;
        const bool live = b < nblocks && i0 < n;
        float mx = 0.0f, vx = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float pi = L[u].p[k] * a.decay;
            const float t0 = a.b1 * L[u].m[k];
            const float t1 = a.omb1 * L[u].g[k];
            const float mi = t0 + t1;
            const float t2 = a.b2 * L[u].v[k];
            const float t3 = a.omb2 * L[u].g[k];
            const float t4 = t3 * L[u].g[k];
            const float vi = t2 + t4;
            const float r = __builtin_sqrtf(vi);
            const float q = r / a.bc2_sqrt;
            const float den = q + a.eps;
            const float upd = mi / den;
            const float w = a.step_size * upd;
            L[u].p[k] = pi - w;
            L[u].m[k] = mi;
            L[u].v[k] = vi;
            mx = fmaxf(mx, fabsf(mi));
            vx = fmaxf(vx, fabsf(vi));
        }
        // block amax within the 16-lane row (rows past the end hold zeros)
        const TileScale tm = make_scale(dpp_max16(mx));
        const TileScale tv = make_scale(dpp_max16(vx));
        uint32_t mlo, mhi, vlo, vhi;
        quant8(L[u].m, tm, mlo, mhi);
        quant8(L[u].v, tv, vlo, vhi);
        if (!live) continue;
        if (i0 + 8 <= n) {
            *reinterpret_cast<float4*>(p + i0) = make_float4(L[u].p[0], L[u].p[1], L[u].p[2], L[u].p[3]);
            *reinterpret_cast<float4*>(p + i0 + 4) = make_float4(L[u].p[4], L[u].p[5], L[u].p[6], L[u].p[7]);
            *reinterpret_cast<uint2*>(mq + i0) = make_uint2(mlo, mhi);
            *reinterpret_cast<uint2*>(vq + i0) = make_uint2(vlo, vhi);
        } else {
            for (int k = 0; k < 8 && i0 + k < n; ++k) {
                p[i0 + k] = L[u].p[k];
                mq[i0 + k] = (uint8_t)(((k < 4 ? mlo : mhi) >> (8 * (k & 3))) & 0xFF);
                vq[i0 + k] = (uint8_t)(((k < 4 ? vlo : vhi) >> (8 * (k & 3))) & 0xFF);
            }
        }
        if (lane16 == 0) {
            ms[b] = tm.s;
            vs[b] = tv.s;
        }
    }
}

void launch_adam_fp8(int64_t n, float* p, const void* g, int g_dtype, uint8_t* mq, float* ms,
                     uint8_t* vq, float* vs, const AdamScalars& a, hipStream_t st)
{
    const uint32_t nblocks = (uint32_t)((n + kTile - 1) / kTile);
    const uint32_t wgs = (nblocks + kAdamBlocksPerWg - 1) / kAdamBlocksPerWg;
    if (g_dtype == FP8Q_BF16)
        hipLaunchKernelGGL(adam_fp8_kernel<uint16_t>, dim3(wgs), dim3(kAdamThreads), 0, st, p,
                           static_cast<const uint16_t*>(g), mq, ms, vq, vs, n, nblocks, a);
    else
        hipLaunchKernelGGL(adam_fp8_kernel<float>, dim3(wgs), dim3(kAdamThreads), 0, st, p,
                           static_cast<const float*>(g), mq, ms, vq, vs, n, nblocks, a);
}

}  // namespace fp8q
