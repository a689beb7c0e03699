// Shared definitions of the block-scaled GEMM kernels (host and device).
#pragma once

#include "fp8q_device.h"

namespace fp8q {

enum { SA_ROW = 0, SA_TENSOR = 2 };
enum { SB_ROW = 0, SB_BLOCK = 1, SB_TENSOR = 2 };
// output of the GEMM: fp32, bf16, or E4M3 codes with 1x128 scales along N
enum { OUT_F32 = 0, OUT_BF16 = 1, OUT_E4M3 = 2 };

struct GemmArgs {
    int64_t M, N, K;
    const uint8_t* a;
    int64_t lda;
    const float* sa;
    int64_t ldsa;
    const uint8_t* b;
    int64_t ldb;
    const float* sb;
    int64_t ldsb;
    void* c;
    int64_t ldc;
    int KB;
    int tiles_m, tiles_n;
    int num_cus;             // compute units of the device (persistent grid size)
    // grouped GEMM: per-group B/SB strides and device group offsets
    const int32_t* offsets;
    int G;
    int64_t b_group_stride, sb_group_stride;
    int64_t c_group_stride;  // groups of K: elements between groups' output blocks
    float* cs;               // E4M3 output: its 1x128 scales cs[m * ldcs + n / 128]
    int64_t ldcs;
};

__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// bf16_rne(a) | bf16_rne(b) << 16 for finite a, b in one instruction (the
// packed conversion rounds to nearest even; checked equal to bf16_rne over
// every non-NaN fp32 pattern, denormals and infinities included)
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b)
{
    uint32_t d;
    asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
    return d;
}

// Zero the bytes of a 16-byte chunk at or beyond `valid` (0..16).
__device__ __forceinline__ uint4 mask_bytes(uint4 v, int valid)
{
    if (valid >= 16) return v;
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int keep = valid - 4 * i;
        uint32_t m = keep >= 4 ? 0xFFFFFFFFu : (keep <= 0 ? 0u : ((1u << (8 * keep)) - 1u));
        w[i] &= m;
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}


// Launch of the LDS-DMA pipelined kernel (forward, dgrad, wgrad,
// per-tensor); returns false if that kernel does not cover the call (the
// caller then uses the general kernel).
// `out` is OUT_F32, OUT_BF16 or OUT_E4M3 (codes in c, scales in cs).
bool launch_gemm_nk(const GemmArgs& g, int sa_mode, int sb_mode, bool b_kn, int out, hipStream_t st);
// The four-wave kernel (gemm_w4.hip) for dense calls with K a multiple of
// 128, B stored [N][K] or read as stored [K][N] (fp32, bf16 or E4M3 output);
// false if it does not cover the call.
bool launch_gemm_w4(const GemmArgs& g, int sa_mode, int sb_mode, bool b_kn, int out, hipStream_t st);
// ... and with power-of-two scales (E8M0 bytes, as launch_gemm_nk_e8m0).
bool launch_gemm_w4_e8m0(const GemmArgs& g, int sb_mode, bool b_kn, bool out_bf16, hipStream_t st);
// The four-wave kernel over groups of rows (MoE forward, B [N][K], and
// dgrad, B read as stored [K][N]; K % 128 == 0); false if it does not cover
// the call.
bool launch_grouped_gemm_w4(const GemmArgs& g, bool out_bf16, bool b_kn, hipStream_t st);
// ... the forward stored quantized (E4M3 codes + 1x128 scales); false if not covered.
bool launch_grouped_gemm_w4_e4m3(const GemmArgs& g, hipStream_t st);
// ... and over groups of K (MoE weight gradient); false if not covered.
bool launch_grouped_wgrad_w4(const GemmArgs& g, hipStream_t st);
// Grouped (MoE) launch of the same kernel: A row tiles select their expert
// through the device group offsets (B per expert as [N][K] for the forward,
// read as [K][N] for dgrad); false if the call is not covered.
bool launch_grouped_gemm_nk(const GemmArgs& g, bool out_bf16, bool b_kn, hipStream_t st);
// Dense launch with power-of-two scales: p.sa / p.sb point at E8M0 bytes
// (row-scaled A; block-scaled B as [N][K] or [K][N], or row-scaled [N][K]
// B), whose row strides are multiples of 4; false if the call is not covered.
bool launch_gemm_nk_e8m0(const GemmArgs& g, int sb_mode, bool b_kn, bool out_bf16, hipStream_t st);

}  // namespace fp8q
