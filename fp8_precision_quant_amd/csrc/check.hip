// Debug validation (environment variable FP8Q_CHECK=1): the device-side
// contract on the grouped GEMMs' group offsets (off[0] = 0, off[G] <= M_pad,
// non-decreasing, every offset a multiple of 128; the padding routing map of
// the Ling 2.0 FP8 blog, "FP8 padding routing map") is checked on the device
// before the GEMM is enqueued, and the caller's stream is synchronized to
// read the verdict back.
#include <cstdlib>

#include "fp8q_internal.h"

namespace fp8q {

namespace {

constexpr int kCheckThreads = 256;

// the verdict of the last check on this device (0 = valid); one word per
// device, no allocation
__device__ int g_offsets_verdict;

__global__ __launch_bounds__(kCheckThreads) void check_offsets_kernel(const int32_t* __restrict__ off, int G,
                                                                      int64_t M_pad, int* verdict)
{
    int bad = 0;
    for (int i = threadIdx.x; i <= G; i += kCheckThreads) {
        const int v = off[i];
        if (v < 0 || (int64_t)v > M_pad || v % 128 != 0) bad = 1;
        if (i < G && off[i + 1] < v) bad = 1;
    }
    if (threadIdx.x == 0 && off[0] != 0) bad = 1;
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) *verdict = bad;
}

}  // namespace

bool debug_checks_enabled()
{
    const char* v = std::getenv("FP8Q_CHECK");
    return v != nullptr && v[0] == '1' && v[1] == '\0';
}

int check_group_offsets(const int32_t* offsets, int64_t G, int64_t M_pad, hipStream_t st)
{
    int* verdict = nullptr;
    if (hipGetSymbolAddress(reinterpret_cast<void**>(&verdict), HIP_SYMBOL(g_offsets_verdict)) != hipSuccess) {
        (void)hipGetLastError();
        return FP8Q_ERR_DEVICE;
    }
    hipLaunchKernelGGL(check_offsets_kernel, dim3(1), dim3(kCheckThreads), 0, st, offsets, (int)G, M_pad,
                       verdict);
    int host = 1;
    if (hipGetLastError() != hipSuccess ||
        hipMemcpyAsync(&host, verdict, sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess) {
        (void)hipGetLastError();
        return FP8Q_ERR_LAUNCH;
    }
    return host == 0 ? FP8Q_OK : FP8Q_ERR_SHAPE;
}

}  // namespace fp8q
