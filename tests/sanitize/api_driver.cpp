// Calls every entry point of libfp8q with arguments that its host-side
// validation must reject, and checks the status each returns.  Built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code of the
// library (device code not compiled), it runs the validation logic, which is
// all host arithmetic on sizes, strides and pointers, under both sanitizers.
// Every call fails before the library touches a device, so the pointers
// below are never dereferenced.  Exit status 0 iff every status matches.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/fp8q.h"

namespace {

int failures = 0;

void expect(int got, int want, const char* what)
{
    if (got != want) {
        std::fprintf(stderr, "%s: got %d (%s), want %d\n", what, got, fp8q_status_string(got), want);
        ++failures;
    }
}

// aligned stand-ins for device buffers (never dereferenced)
uint8_t* const P = reinterpret_cast<uint8_t*>(uintptr_t(1) << 20);
uint8_t* const U = P + 1;   // misaligned by one byte
float* const F = reinterpret_cast<float*>(P);
int32_t* const O = reinterpret_cast<int32_t*>(P);

}  // namespace

int main()
{
    for (int s = -1; s <= 7; ++s)
        if (!fp8q_status_string(s) || !std::strlen(fp8q_status_string(s))) ++failures;

    // fp8_quant_blockwise
    expect(fp8_quant_blockwise(P, 7, 4, 128, 128, FP8Q_ROW_1x128, P, 128, F, 1, nullptr), FP8Q_ERR_UNSUPPORTED, "qb dtype");
    expect(fp8_quant_blockwise(P, FP8Q_BF16, 4, 128, 128, 9, P, 128, F, 1, nullptr), FP8Q_ERR_UNSUPPORTED, "qb kind");
    expect(fp8_quant_blockwise(P, FP8Q_BF16, -1, 128, 128, FP8Q_ROW_1x128, P, 128, F, 1, nullptr), FP8Q_ERR_SHAPE, "qb rows<0");
    expect(fp8_quant_blockwise(P, FP8Q_BF16, 0, 128, 128, FP8Q_ROW_1x128, P, 128, F, 1, nullptr), FP8Q_OK, "qb empty");
    expect(fp8_quant_blockwise(nullptr, FP8Q_BF16, 4, 128, 128, FP8Q_ROW_1x128, P, 128, F, 1, nullptr), FP8Q_ERR_NULL, "qb null x");
    expect(fp8_quant_blockwise(P, FP8Q_BF16, 4, 128, 120, FP8Q_ROW_1x128, P, 128, F, 1, nullptr), FP8Q_ERR_SHAPE, "qb ldx");
    expect(fp8_quant_blockwise(P, FP8Q_BF16, 4, 300, 304, FP8Q_ROW_1x128, P, 304, F, 2, nullptr), FP8Q_ERR_SHAPE, "qb lds");
    expect(fp8_quant_blockwise(P, FP8Q_BF16, int64_t(1) << 40, 1 << 20, 1 << 20, FP8Q_ROW_1x128, P, 1 << 20, F, 8192, nullptr),
           FP8Q_ERR_SHAPE, "qb too many tiles");
    expect(fp8_quant_blockwise(U, FP8Q_BF16, 4, 128, 128, FP8Q_ROW_1x128, P, 128, F, 1, nullptr), FP8Q_ERR_ALIGN, "qb align x");
    expect(fp8_quant_blockwise(P, FP8Q_BF16, 4, 100, 100, FP8Q_ROW_1x128, P, 112, F, 1, nullptr), FP8Q_ERR_ALIGN, "qb ldx bytes");
    expect(fp8_quant_blockwise(P, FP8Q_F32, 4, 128, 128, FP8Q_TENSOR, P, 128, reinterpret_cast<float*>(U), 1, nullptr),
           FP8Q_ERR_ALIGN, "qb tensor scale align");

    // fp8_quant_transpose
    expect(fp8_quant_transpose(P, 3, 4, 128, 128, P, 128, F, 1, P, 16, F, 1, nullptr), FP8Q_ERR_UNSUPPORTED, "qt dtype");
    expect(fp8_quant_transpose(P, FP8Q_BF16, 4, -2, 128, P, 128, F, 1, P, 16, F, 1, nullptr), FP8Q_ERR_SHAPE, "qt cols<0");
    expect(fp8_quant_transpose(P, FP8Q_BF16, 4, 128, 128, P, 128, nullptr, 1, P, 16, F, 1, nullptr), FP8Q_ERR_NULL, "qt half row");
    expect(fp8_quant_transpose(P, FP8Q_BF16, 4, 128, 128, nullptr, 0, nullptr, 0, nullptr, 0, nullptr, 0, nullptr), FP8Q_OK,
           "qt nothing wanted");
    expect(fp8_quant_transpose(P, FP8Q_BF16, 130, 128, 128, P, 128, F, 1, P, 128, F, 1, nullptr), FP8Q_ERR_SHAPE, "qt ldq_colT");
    expect(fp8_quant_transpose(P, FP8Q_BF16, 4, 128, 128, P, 128, F, 1, U, 16, F, 1, nullptr), FP8Q_ERR_ALIGN, "qt align colT");
    expect(fp8_quant_transpose_e8m0(P, FP8Q_BF16, 4, 128, 128, P, 128, P, 0, P, 16, P, 1, nullptr), FP8Q_ERR_SHAPE,
           "qt e8m0 lde");

    // fp8_gemm_blockscaled
    expect(fp8_gemm_blockscaled(4, 128, 128, P, 128, F, 1, FP8Q_ROW_1x128, P, 128, FP8Q_B_NK, F, 1, FP8Q_BLOCK_128x128,
                                P, 128, 5, nullptr), FP8Q_ERR_UNSUPPORTED, "gemm c dtype");
    expect(fp8_gemm_blockscaled(4, 128, 128, P, 128, F, 1, FP8Q_ROW_1x128, P, 128, 2, F, 1, FP8Q_BLOCK_128x128,
                                P, 128, FP8Q_BF16, nullptr), FP8Q_ERR_UNSUPPORTED, "gemm layout");
    expect(fp8_gemm_blockscaled(4, 128, 128, P, 128, F, 1, FP8Q_BLOCK_128x128, P, 128, FP8Q_B_NK, F, 1, FP8Q_BLOCK_128x128,
                                P, 128, FP8Q_BF16, nullptr), FP8Q_ERR_UNSUPPORTED, "gemm sa kind");
    expect(fp8_gemm_blockscaled(4, 128, 128, P, 128, F, 1, FP8Q_ROW_1x128, P, 128, FP8Q_B_KN, F, 1, FP8Q_ROW_1x128,
                                P, 128, FP8Q_BF16, nullptr), FP8Q_ERR_UNSUPPORTED, "gemm row B as KN");
    expect(fp8_gemm_blockscaled(4, 128, -1, P, 128, F, 1, FP8Q_ROW_1x128, P, 128, FP8Q_B_NK, F, 1, FP8Q_BLOCK_128x128,
                                P, 128, FP8Q_BF16, nullptr), FP8Q_ERR_SHAPE, "gemm K<0");
    expect(fp8_gemm_blockscaled(4, 0, 128, P, 128, F, 1, FP8Q_ROW_1x128, P, 128, FP8Q_B_NK, F, 1, FP8Q_BLOCK_128x128,
                                P, 128, FP8Q_BF16, nullptr), FP8Q_OK, "gemm empty");
    expect(fp8_gemm_blockscaled(4, 128, 128, nullptr, 128, F, 1, FP8Q_ROW_1x128, P, 128, FP8Q_B_NK, F, 1,
                                FP8Q_BLOCK_128x128, P, 128, FP8Q_BF16, nullptr), FP8Q_ERR_NULL, "gemm null a");
    expect(fp8_gemm_blockscaled(4, 128, 256, P, 256, F, 1, FP8Q_ROW_1x128, P, 256, FP8Q_B_NK, F, 2, FP8Q_BLOCK_128x128,
                                P, 128, FP8Q_BF16, nullptr), FP8Q_ERR_SHAPE, "gemm ldsa");
    expect(fp8_gemm_blockscaled(4, 300, 256, P, 256, F, 2, FP8Q_ROW_1x128, P, 304, FP8Q_B_KN, F, 2, FP8Q_BLOCK_128x128,
                                P, 304, FP8Q_BF16, nullptr), FP8Q_ERR_SHAPE, "gemm KN ldsb");
    expect(fp8_gemm_blockscaled(4, 128, 128, P, 128, F, 1, FP8Q_ROW_1x128, P, 128, FP8Q_B_NK, F, 1, FP8Q_BLOCK_128x128,
                                U, 128, FP8Q_BF16, nullptr), FP8Q_ERR_ALIGN, "gemm align c");
    expect(fp8_gemm_blockscaled(4, 128, 100, P, 100, F, 1, FP8Q_ROW_1x128, P, 112, FP8Q_B_NK, F, 1, FP8Q_BLOCK_128x128,
                                P, 128, FP8Q_BF16, nullptr), FP8Q_ERR_ALIGN, "gemm lda");
    expect(fp8_gemm_blockscaled_e4m3(4, 128, 128, P, 128, F, 1, FP8Q_ROW_1x128, P, 128, FP8Q_B_NK, F, 1, FP8Q_ROW_1x128,
                                     P, 128, F, 1, nullptr), FP8Q_ERR_UNSUPPORTED, "e4m3 row B");
    expect(fp8_gemm_blockscaled_e4m3(4, 300, 128, P, 128, F, 1, FP8Q_ROW_1x128, P, 128, FP8Q_B_NK, F, 1,
                                     FP8Q_BLOCK_128x128, P, 304, F, 2, nullptr), FP8Q_ERR_SHAPE, "e4m3 lds");
    expect(fp8_gemm_e8m0(4, 128, 128, P, 128, P, 1, P, 128, FP8Q_B_NK, P, 1, FP8Q_TENSOR, P, 128, FP8Q_BF16, nullptr),
           FP8Q_ERR_UNSUPPORTED, "e8m0 tensor");
    expect(fp8_gemm_e8m0(4, 128, 128, P, 128, U, 4, P, 128, FP8Q_B_NK, P, 4, FP8Q_BLOCK_128x128, P, 128, FP8Q_BF16, nullptr),
           FP8Q_ERR_ALIGN, "e8m0 scale align");

    // grouped
    expect(fp8_grouped_gemm(0, 128, 128, 128, P, 128, F, 1, O, P, F, P, 128, FP8Q_BF16, nullptr), FP8Q_ERR_SHAPE, "grouped G");
    expect(fp8_grouped_gemm(2, 100, 128, 128, P, 128, F, 1, O, P, F, P, 128, FP8Q_BF16, nullptr), FP8Q_ERR_SHAPE,
           "grouped M_pad");
    expect(fp8_grouped_gemm(1025, 128, 128, 128, P, 128, F, 1, O, P, F, P, 128, FP8Q_BF16, nullptr), FP8Q_ERR_UNSUPPORTED,
           "grouped G>1024");
    expect(fp8_grouped_gemm(2, 128, 128, 128, P, 128, F, 1, nullptr, P, F, P, 128, FP8Q_BF16, nullptr), FP8Q_ERR_NULL,
           "grouped null offsets");
    expect(fp8_grouped_gemm(2, 128, 128, 120, P, 128, F, 1, O, P, F, P, 128, FP8Q_BF16, nullptr), FP8Q_ERR_ALIGN,
           "grouped K%16");
    expect(fp8_grouped_gemm(2, 128, 128, 128, P, 128, F, 1, reinterpret_cast<int32_t*>(U), P, F, P, 128, FP8Q_BF16,
                            nullptr), FP8Q_ERR_ALIGN, "grouped offsets align");
    expect(fp8_grouped_gemm_e4m3(2, 128, 128, 200, P, 208, F, 2, O, P, F, P, 128, F, 1, nullptr), FP8Q_ERR_UNSUPPORTED,
           "grouped e4m3 K%128");
    expect(fp8_grouped_gemm_e4m3(2, 128, 300, 128, P, 128, F, 1, O, P, F, P, 304, F, 2, nullptr), FP8Q_ERR_SHAPE,
           "grouped e4m3 lds");
    expect(fp8_grouped_gemm_e4m3(2, 128, 128, 128, P, 128, F, 1, O, P, F, U, 128, F, 1, nullptr), FP8Q_ERR_ALIGN,
           "grouped e4m3 q align");
    expect(fp8_grouped_gemm_dgrad(2, 128, 128, 128, P, 128, F, 0, O, P, F, P, 128, FP8Q_BF16, nullptr), FP8Q_ERR_SHAPE,
           "dgrad ldsa");
    expect(fp8_grouped_gemm_wgrad(2, 256, 128, 128, P, 256, F, 1, P, 256, F, 2, O, F, 128, nullptr), FP8Q_ERR_SHAPE,
           "wgrad ldsa");
    expect(fp8_grouped_gemm_wgrad(2, 256, 128, 128, P, 256, F, 2, P, 256, F, 2, O, reinterpret_cast<float*>(U), 128,
                                  nullptr), FP8Q_ERR_ALIGN, "wgrad align c");

    // adam
    expect(fp8_adam_step(256, F, F, FP8Q_F32, P, F, P, F, 1e-3, 1.0, 0.999, 1e-8, 0.0, 1, nullptr), FP8Q_ERR_UNSUPPORTED,
           "adam beta1");
    expect(fp8_adam_step(256, F, F, FP8Q_F32, P, F, P, F, 1e-3, 0.9, 0.999, 1e-8, 0.0, 0, nullptr), FP8Q_ERR_UNSUPPORTED,
           "adam step 0");
    expect(fp8_adam_step(-5, F, F, FP8Q_F32, P, F, P, F, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, nullptr), FP8Q_ERR_SHAPE, "adam n");
    expect(fp8_adam_step(256, F, F, FP8Q_F32, U, F, P, F, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, nullptr), FP8Q_ERR_ALIGN,
           "adam align");

    if (failures) {
        std::fprintf(stderr, "%d case(s) failed\n", failures);
        return 1;
    }
    std::printf("api driver: all validation cases passed\n");
    return 0;
}
