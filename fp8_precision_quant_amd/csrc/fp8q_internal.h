// Internal launcher declarations of libfp8q (host side).  Every launcher
// assumes its arguments were validated by the C-ABI layer and only enqueues
// kernels on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fp8q.h"

namespace fp8q {

// compute units of the current device (cached per device)
int device_cu_count();

// FP8Q_CHECK=1 in the environment (read at every call)
bool debug_checks_enabled();
// Checks the group-offset contract on the device (synchronizes `st`):
// FP8Q_OK, FP8Q_ERR_SHAPE if violated, FP8Q_ERR_LAUNCH / _DEVICE on a HIP error.
int check_group_offsets(const int32_t* offsets, int64_t G, int64_t M_pad, hipStream_t st);

void launch_quant_blockwise(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                            int kind, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                            hipStream_t st);

void launch_quant_transpose(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                            uint8_t* q_row, int64_t ldq_row, float* s_row, int64_t lds_row,
                            uint8_t* q_colT, int64_t ldq_colT, float* s_colT, int64_t lds_colT,
                            hipStream_t st);

// power-of-two scales as E8M0 bytes (row tiles and 128x128 blocks)
void launch_quant_blockwise_e8m0(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                                 int kind, uint8_t* q, int64_t ldq, uint8_t* e, int64_t lde,
                                 hipStream_t st);
void launch_quant_transpose_e8m0(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                                 uint8_t* q_row, int64_t ldq_row, uint8_t* e_row, int64_t lde_row,
                                 uint8_t* q_colT, int64_t ldq_colT, uint8_t* e_colT, int64_t lde_colT,
                                 hipStream_t st);

// The GEMM launchers return false (nothing enqueued) for calls the kernel
// does not cover.
bool launch_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const float* sa,
                 int64_t ldsa, int sa_kind, const uint8_t* b, int64_t ldb, int b_layout,
                 const float* sb, int64_t ldsb, int sb_kind, void* c, int64_t ldc, int c_dtype,
                 hipStream_t st);

bool launch_grouped_gemm_dgrad(int64_t G, int64_t M_pad, int64_t N, int64_t K, const uint8_t* a,
                               int64_t lda, const float* sa, int64_t ldsa, const int32_t* offsets,
                               const uint8_t* w, const float* sw, void* c, int64_t ldc, int c_dtype,
                               hipStream_t st);
bool launch_grouped_gemm_wgrad(int64_t G, int64_t M_pad, int64_t N, int64_t K, const uint8_t* a,
                               int64_t lda, const float* sa, int64_t ldsa, const uint8_t* b,
                               int64_t ldb, const float* sb, int64_t ldsb, const int32_t* offsets,
                               float* c, int64_t ldc, hipStream_t st);
bool launch_gemm_e4m3(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const float* sa,
                      int64_t ldsa, int sa_kind, const uint8_t* b, int64_t ldb, int b_layout,
                      const float* sb, int64_t ldsb, int sb_kind, uint8_t* q, int64_t ldq, float* s,
                      int64_t lds, hipStream_t st);
bool launch_gemm_e8m0(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const uint8_t* ea,
                      int64_t ldea, const uint8_t* b, int64_t ldb, int b_layout, const uint8_t* eb,
                      int64_t ldeb, int eb_kind, void* c, int64_t ldc, int c_dtype, hipStream_t st);
bool launch_grouped_gemm(int64_t G, int64_t M_pad, int64_t N, int64_t K, const uint8_t* a,
                         int64_t lda, const float* sa, int64_t ldsa, const int32_t* offsets,
                         const uint8_t* b, const float* sb, void* c, int64_t ldc, int c_dtype,
                         hipStream_t st);
// The MoE forward stored quantized (E4M3 codes + 1x128 scales); false if not
// covered (K % 128 != 0, more than 1024 groups, or an operand of 2 GiB or more).
bool launch_grouped_gemm_e4m3(int64_t G, int64_t M_pad, int64_t N, int64_t K, const uint8_t* a,
                              int64_t lda, const float* sa, int64_t ldsa, const int32_t* offsets,
                              const uint8_t* b, const float* sb, uint8_t* q, int64_t ldq, float* s,
                              int64_t lds, hipStream_t st);

// AdamW with E4M3 moments: the step's fp32 scalars, each derived on the host
// in double from the hyperparameters and rounded once
struct AdamScalars {
    float b1, b2, omb1, omb2, decay, step_size, bc2_sqrt, eps;
};
void launch_adam_fp8(int64_t n, float* p, const void* g, int g_dtype, uint8_t* mq, float* ms,
                     uint8_t* vq, float* vs, const AdamScalars& a, hipStream_t st);

}  // namespace fp8q
