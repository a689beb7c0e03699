// Stand-ins for the kernel launchers of libfp8q, linked with the host code
// of the C-ABI layer (api.hip) for the sanitizer run: every case of the
// driver must be rejected by validation, so reaching any launcher, or the
// device check of the debug mode, is a failure.
#include <cstdio>
#include <cstdlib>

#include "../../fp8_precision_quant_amd/csrc/fp8q_internal.h"

namespace {
[[noreturn]] void reached(const char* what)
{
    std::fprintf(stderr, "validation let a call through to %s\n", what);
    std::abort();
}
}  // namespace

namespace fp8q {

int device_cu_count() { reached("device_cu_count"); }
bool debug_checks_enabled() { return false; }
int check_group_offsets(const int32_t*, int64_t, int64_t, hipStream_t) { reached("check_group_offsets"); }
void launch_quant_blockwise(const void*, int, int64_t, int64_t, int64_t, int, uint8_t*, int64_t, float*, int64_t,
                            hipStream_t)
{
    reached("launch_quant_blockwise");
}
void launch_quant_transpose(const void*, int, int64_t, int64_t, int64_t, uint8_t*, int64_t, float*, int64_t, uint8_t*,
                            int64_t, float*, int64_t, hipStream_t)
{
    reached("launch_quant_transpose");
}
void launch_quant_blockwise_e8m0(const void*, int, int64_t, int64_t, int64_t, int, uint8_t*, int64_t, uint8_t*,
                                 int64_t, hipStream_t)
{
    reached("launch_quant_blockwise_e8m0");
}
void launch_quant_transpose_e8m0(const void*, int, int64_t, int64_t, int64_t, uint8_t*, int64_t, uint8_t*, int64_t,
                                 uint8_t*, int64_t, uint8_t*, int64_t, hipStream_t)
{
    reached("launch_quant_transpose_e8m0");
}
bool launch_gemm(int64_t, int64_t, int64_t, const uint8_t*, int64_t, const float*, int64_t, int, const uint8_t*,
                 int64_t, int, const float*, int64_t, int, void*, int64_t, int, hipStream_t)
{
    reached("launch_gemm");
}
bool launch_grouped_gemm_dgrad(int64_t, int64_t, int64_t, int64_t, const uint8_t*, int64_t, const float*, int64_t,
                               const int32_t*, const uint8_t*, const float*, void*, int64_t, int, hipStream_t)
{
    reached("launch_grouped_gemm_dgrad");
}
bool launch_grouped_gemm_wgrad(int64_t, int64_t, int64_t, int64_t, const uint8_t*, int64_t, const float*, int64_t,
                               const uint8_t*, int64_t, const float*, int64_t, const int32_t*, float*, int64_t,
                               hipStream_t)
{
    reached("launch_grouped_gemm_wgrad");
}
bool launch_gemm_e4m3(int64_t, int64_t, int64_t, const uint8_t*, int64_t, const float*, int64_t, int, const uint8_t*,
                      int64_t, int, const float*, int64_t, int, uint8_t*, int64_t, float*, int64_t, hipStream_t)
{
    reached("launch_gemm_e4m3");
}
bool launch_gemm_e8m0(int64_t, int64_t, int64_t, const uint8_t*, int64_t, const uint8_t*, int64_t, const uint8_t*,
                      int64_t, int, const uint8_t*, int64_t, int, void*, int64_t, int, hipStream_t)
{
    reached("launch_gemm_e8m0");
}
bool launch_grouped_gemm(int64_t, int64_t, int64_t, int64_t, const uint8_t*, int64_t, const float*, int64_t,
                         const int32_t*, const uint8_t*, const float*, void*, int64_t, int, hipStream_t)
{
    reached("launch_grouped_gemm");
}
bool launch_grouped_gemm_e4m3(int64_t, int64_t, int64_t, int64_t, const uint8_t*, int64_t, const float*, int64_t,
                              const int32_t*, const uint8_t*, const float*, uint8_t*, int64_t, float*, int64_t,
                              hipStream_t)
{
    reached("launch_grouped_gemm_e4m3");
}
void launch_adam_fp8(int64_t, float*, const void*, int, uint8_t*, float*, uint8_t*, float*, const AdamScalars&,
                     hipStream_t)
{
    reached("launch_adam_fp8");
}

}  // namespace fp8q
