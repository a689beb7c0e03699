// Block-scaled FP8 GEMM for gfx950 (CDNA4 FP8 MFMA).
//
//   C[m][n] = sum_kb SA(m,kb) * SB(n,kb) * sum_{k in chunk kb} dec(A[m][k]) * dec(B^[n][k])
//
// The FP8 Linear of the Ling 2.0 FP8 blog (BF16 Linear -> FP8 tensor + scale
// tensor -> FP8 GEMM with an FP32 accumulator, "where is error introduced"),
// with the fine-grained scales of its "fine-grained quantization" section:
// activations / gradients 1x128, weights 128x128 ("FP8-RL" article, 一).
//
// Mapping to gfx950: one v_mfma_f32_16x16x128_f8f6f4 covers exactly one
// 128-wide K chunk of a 16x16 output block, so every MFMA produces the fresh
// fp32 partial sum of one scale chunk; the VALU then adds partial * SA * SB
// into the fp32 accumulator.  Workgroup tile 256x128x128, 8 waves of 64x64,
// A and B chunks double-buffered in LDS (16-byte slots XOR-swizzled by row),
// the next chunk prefetched into registers while the current one computes.
//
// B layouts: NK ([N][K], forward and wgrad) is staged as is; KN ([K][N],
// dgrad reading the weight in its stored layout, Ling 2.0 FP8 blog "FP8
// on-demand transpose weight") is transposed in registers (4x4 byte blocks)
// on its way into LDS, so LDS always holds K-contiguous rows for both
// operands.
#include <atomic>

#include "fp8q_device.h"
#include "fp8q_internal.h"
#include "gemm_common.h"

namespace fp8q {

constexpr int BN = 128;
constexpr int BK = 128;
constexpr int kGemmThreads = 512;
constexpr int WM = 64;       // wave tile rows
constexpr int MI = WM / 16;  // 16x16 blocks per wave along M

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 4); }

// Loads of one K-contiguous ([rows][K]) ROWSx128 operand tile: ROWS/64 chunks
// of 16 bytes per thread.  Rows >= `rows_valid` and bytes >= K read as zero.
template <int ROWS>
struct NKLoad {
    static constexpr int kPer = ROWS * 8 / kGemmThreads;
    uint4 v[kPer];
    __device__ __forceinline__ void load(const uint8_t* base, int64_t ld, int64_t row0,
                                         int64_t rows_valid, int64_t k0, int64_t K, int tid)
    {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            int ci = tid + kGemmThreads * i;
            int r = ci >> 3, ch = ci & 7;
            int64_t kk = k0 + ch * 16;
            if (row0 + r < rows_valid && kk < K) {
                uint4 x = *reinterpret_cast<const uint4*>(base + (row0 + r) * ld + kk);
                v[i] = mask_bytes(x, (int)(K - kk));
            } else {
                v[i] = make_uint4(0, 0, 0, 0);
            }
        }
    }
    __device__ __forceinline__ void store(uint8_t* lds, int tid) const
    {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            int ci = tid + kGemmThreads * i;
            int r = ci >> 3, ch = ci & 7;
            *reinterpret_cast<uint4*>(lds + swz(r, ch)) = v[i];
        }
    }
};

// Loads of a [K][N]-stored operand tile (128 k-rows x BN n-columns): a
// thread takes 4 consecutive k-rows x 16 consecutive n (threads beyond
// 32 * BN/16 idle), transposes the 4x4 byte blocks in registers and writes
// K-contiguous 4-byte groups to LDS.
struct KNLoad {
    static constexpr int kUnits = 32 * (BN / 16);
    uint4 v[4];
    __device__ __forceinline__ void load(const uint8_t* base, int64_t ld, int64_t n0, int64_t N,
                                         int64_t k0, int64_t K, int tid)
    {
        int kq = tid / (BN / 16);   // k-rows 4kq..4kq+3
        int nc = tid % (BN / 16);   // n 16nc..16nc+15
        int64_t n = n0 + nc * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int64_t k = k0 + 4 * kq + i;
            if (tid < kUnits && k < K && n < N)
                v[i] = *reinterpret_cast<const uint4*>(base + k * ld + n);
            else
                v[i] = make_uint4(0, 0, 0, 0);
        }
    }
    __device__ __forceinline__ void store(uint8_t* lds, int tid) const
    {
        if (tid >= kUnits) return;
        int kq = tid / (BN / 16);
        int nc = tid % (BN / 16);
        const uint32_t r0[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
        const uint32_t r1[4] = {v[1].x, v[1].y, v[1].z, v[1].w};
        const uint32_t r2[4] = {v[2].x, v[2].y, v[2].z, v[2].w};
        const uint32_t r3[4] = {v[3].x, v[3].y, v[3].z, v[3].w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            // rows k..k+3 hold bytes n = 16nc + 4d + {0..3}; produce one dword per n
            uint32_t t0 = __builtin_amdgcn_perm(r1[d], r0[d], 0x05010400u);
            uint32_t t1 = __builtin_amdgcn_perm(r1[d], r0[d], 0x07030602u);
            uint32_t t2 = __builtin_amdgcn_perm(r3[d], r2[d], 0x05010400u);
            uint32_t t3 = __builtin_amdgcn_perm(r3[d], r2[d], 0x07030602u);
            uint32_t col[4];
            col[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
            col[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
            col[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
            col[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                int n = nc * 16 + 4 * d + e;
                int kbyte = 4 * kq;
                *reinterpret_cast<uint32_t*>(lds + swz(n, kbyte >> 4) + (kbyte & 15)) = col[e];
            }
        }
    }
};

// BM_ = 256: dense GEMM, waves 4 (M) x 2 (N), wave tile 64x64.
// BM_ = 128: grouped GEMM (a 128-row tile never straddles two 128-aligned
//            groups), waves 2 (M) x 4 (N), wave tile 64x32.
template <int BM_, int SA_MODE, int SB_MODE, bool B_KN, bool OUT_BF16, bool GROUPED>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(GemmArgs p)
{
    constexpr int WAVES_M = BM_ / WM;
    constexpr int WAVES_N = (kGemmThreads / 64) / WAVES_M;
    constexpr int WN = BN / WAVES_N;
    constexpr int NI = WN / 16;

    __shared__ __attribute__((aligned(16))) uint8_t As[2][BM_ * BK];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * BK];
    __shared__ __attribute__((aligned(16))) float SAs[2][BM_];
    __shared__ __attribute__((aligned(16))) float SBs[2][BN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_m = wave / WAVES_N;
    const int wave_n = wave % WAVES_N;

    // tile order: consecutive workgroups walk down M inside a panel of up to
    // 8 N-tiles, so the set of B panels being read at once stays small
    const int tiles_m = p.tiles_m, tiles_n = p.tiles_n;
    const int bid = blockIdx.x;
    const int group_n = 8;
    const int group = bid / (group_n * tiles_m);
    const int first_n = group * group_n;
    const int gsize = min(tiles_n - first_n, group_n);
    const int in_group = bid - group * group_n * tiles_m;
    const int tile_m = in_group / gsize;
    const int tile_n = first_n + in_group % gsize;

    const int64_t m0 = (int64_t)tile_m * BM_;
    const int64_t n0 = (int64_t)tile_n * BN;
    const int64_t M = p.M, N = p.N, K = p.K;

    const uint8_t* bbase = p.b;
    const float* sbbase = p.sb;
    if (GROUPED) {
        // group e with off[e] <= m0 < off[e+1]: the largest e with off[e] <= m0
        const int32_t* off = p.offsets;
        if (m0 >= off[p.G]) return;            // rows past the last group are not written
        int lo = 0, hi = p.G - 1;
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if ((int64_t)off[mid] <= m0) lo = mid; else hi = mid - 1;
        }
        bbase += (int64_t)lo * p.b_group_stride;
        sbbase += (int64_t)lo * p.sb_group_stride;
    }

    const int KB = p.KB;

    NKLoad<BM_> la;
    NKLoad<BN> lbn;
    KNLoad lbk;
    float sa_pre = 0.0f, sb_pre = 0.0f;

    auto prefetch = [&](int kb) {
        int64_t k0 = (int64_t)kb * BK;
        la.load(p.a, p.lda, m0, M, k0, K, tid);
        if (B_KN)
            lbk.load(bbase, p.ldb, n0, N, k0, K, tid);
        else
            lbn.load(bbase, p.ldb, n0, N, k0, K, tid);
        if (SA_MODE == SA_ROW && tid < BM_) {
            int64_t m = m0 + tid;
            sa_pre = m < M ? p.sa[m * p.ldsa + kb] : 0.0f;
        }
        if (SB_MODE == SB_ROW && tid >= kGemmThreads - BN) {
            int64_t n = n0 + (tid - (kGemmThreads - BN));
            sb_pre = n < N ? sbbase[n * p.ldsb + kb] : 0.0f;
        }
    };
    auto commit = [&](int buf) {
        la.store(As[buf], tid);
        if (B_KN)
            lbk.store(Bs[buf], tid);
        else
            lbn.store(Bs[buf], tid);
        if (SA_MODE == SA_ROW && tid < BM_) SAs[buf][tid] = sa_pre;
        if (SB_MODE == SB_ROW && tid >= kGemmThreads - BN) SBs[buf][tid - (kGemmThreads - BN)] = sb_pre;
    };

    v4f acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    const int lrow = lane & 15;            // A row / B column inside a 16x16 block
    const int kgrp = lane >> 4;            // which 32-byte K slice of the chunk
    const int wm0 = wave_m * WM;
    const int wn0 = wave_n * WN;
    // the wave's columns lie inside one 128-wide block of B's scale grid
    const int64_t nblk = (n0 + wn0) / 128;
    const int64_t nblocks_valid = (N + 127) / 128;

    const float sa_t = (SA_MODE == SA_TENSOR && KB > 0) ? p.sa[0] : 0.0f;
    const float sb_t = (SB_MODE == SB_TENSOR && KB > 0) ? sbbase[0] : 0.0f;

    if (KB > 0) {
        prefetch(0);
        commit(0);
    }
    __syncthreads();

    for (int kb = 0; kb < KB; ++kb) {
        const int buf = kb & 1;
        if (kb + 1 < KB) prefetch(kb + 1);

        // per-lane scale of each accumulator row for this chunk
        float sb_blk = 0.0f;
        if (SB_MODE == SB_BLOCK) {
            if (nblk < nblocks_valid)
                sb_blk = B_KN ? sbbase[(int64_t)kb * p.ldsb + nblk] : sbbase[nblk * p.ldsb + kb];
        } else if (SB_MODE == SB_TENSOR) {
            sb_blk = sb_t;
        }
        float rs[MI][4];
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            if (SA_MODE == SA_ROW) {
                float4 s4 = *reinterpret_cast<const float4*>(&SAs[buf][wm0 + 16 * i + 4 * kgrp]);
                rs[i][0] = s4.x; rs[i][1] = s4.y; rs[i][2] = s4.z; rs[i][3] = s4.w;
            } else {
                rs[i][0] = rs[i][1] = rs[i][2] = rs[i][3] = sa_t;
            }
            if (SB_MODE != SB_ROW) {
#pragma unroll
                for (int r = 0; r < 4; ++r) rs[i][r] *= sb_blk;
            }
        }

        v8i af[MI];
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            int row = wm0 + 16 * i + lrow;
            uint4 lo = *reinterpret_cast<const uint4*>(&As[buf][swz(row, 2 * kgrp)]);
            uint4 hi = *reinterpret_cast<const uint4*>(&As[buf][swz(row, 2 * kgrp + 1)]);
            af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            int col = wn0 + 16 * j + lrow;
            uint4 lo = *reinterpret_cast<const uint4*>(&Bs[buf][swz(col, 2 * kgrp)]);
            uint4 hi = *reinterpret_cast<const uint4*>(&Bs[buf][swz(col, 2 * kgrp + 1)]);
            v8i bfr = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            float cs = 1.0f;
            if (SB_MODE == SB_ROW) cs = SBs[buf][wn0 + 16 * j + lrow];
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bfr, zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float t = SB_MODE == SB_ROW ? rs[i][r] * cs : rs[i][r];
                    acc[i][j][r] = __builtin_fmaf(part[r], t, acc[i][j][r]);
                }
            }
            // keep the next fragment's MFMAs from being hoisted over these
            // FMAs: bounds the live partial sums to one fragment's worth
            __builtin_amdgcn_sched_barrier(0);
        }

        if (kb + 1 < KB) commit(buf ^ 1);
        __syncthreads();
    }

    // epilogue: the lane holds rows 4*kgrp + r of each 16x16 block, column lrow
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            int64_t n = n0 + wn0 + 16 * j + lrow;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                int64_t m = m0 + wm0 + 16 * i + 4 * kgrp + r;
                if (m < M && n < N) {
                    if (OUT_BF16)
                        reinterpret_cast<uint16_t*>(p.c)[m * p.ldc + n] = (uint16_t)bf16_rne(acc[i][j][r]);
                    else
                        reinterpret_cast<float*>(p.c)[m * p.ldc + n] = acc[i][j][r];
                }
            }
        }
    }
}

template <int SA_MODE, int SB_MODE, bool B_KN>
static void launch_typed(const GemmArgs& a, bool out_bf16, hipStream_t st)
{
    dim3 grid((uint32_t)(a.tiles_m * a.tiles_n));
    if (out_bf16)
        hipLaunchKernelGGL((gemm_kernel<256, SA_MODE, SB_MODE, B_KN, true, false>), grid,
                           dim3(kGemmThreads), 0, st, a);
    else
        hipLaunchKernelGGL((gemm_kernel<256, SA_MODE, SB_MODE, B_KN, false, false>), grid,
                           dim3(kGemmThreads), 0, st, a);
}

// Compute-unit count of the current device, cached per device (the query
// is not free).  Falls back to 256 (MI355X) if the query fails.
int device_cu_count()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        n = 256;
    }
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

void launch_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const float* sa,
                 int64_t ldsa, int sa_kind, const uint8_t* b, int64_t ldb, int b_layout,
                 const float* sb, int64_t ldsb, int sb_kind, void* c, int64_t ldc, int c_dtype,
                 hipStream_t st)
{
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.a = a; g.lda = lda; g.sa = sa; g.ldsa = ldsa;
    g.b = b; g.ldb = ldb; g.sb = sb; g.ldsb = ldsb;
    g.c = c; g.ldc = ldc;
    g.KB = (int)((K + BK - 1) / BK);
    g.tiles_m = (int)((M + 255) / 256);
    g.tiles_n = (int)((N + BN - 1) / BN);
    g.num_cus = device_cu_count();
    const bool bf = c_dtype == FP8Q_BF16;
    const bool kn = b_layout == FP8Q_B_KN;
    {
        const int sa_mode = sa_kind == FP8Q_ROW_1x128 ? SA_ROW : SA_TENSOR;
        const int sb_mode = sb_kind == FP8Q_ROW_1x128 ? SB_ROW
                          : (sb_kind == FP8Q_BLOCK_128x128 ? SB_BLOCK : SB_TENSOR);
        if (launch_gemm_nk(g, sa_mode, sb_mode, kn, bf ? OUT_BF16 : OUT_F32, st)) return;
    }
    if (sa_kind == FP8Q_ROW_1x128) {
        if (sb_kind == FP8Q_BLOCK_128x128) {
            if (kn) launch_typed<SA_ROW, SB_BLOCK, true>(g, bf, st);
            else launch_typed<SA_ROW, SB_BLOCK, false>(g, bf, st);
        } else if (sb_kind == FP8Q_ROW_1x128) {
            launch_typed<SA_ROW, SB_ROW, false>(g, bf, st);
        } else {
            if (kn) launch_typed<SA_ROW, SB_TENSOR, true>(g, bf, st);
            else launch_typed<SA_ROW, SB_TENSOR, false>(g, bf, st);
        }
    } else {
        if (sb_kind == FP8Q_BLOCK_128x128) {
            if (kn) launch_typed<SA_TENSOR, SB_BLOCK, true>(g, bf, st);
            else launch_typed<SA_TENSOR, SB_BLOCK, false>(g, bf, st);
        } else if (sb_kind == FP8Q_ROW_1x128) {
            launch_typed<SA_TENSOR, SB_ROW, false>(g, bf, st);
        } else {
            if (kn) launch_typed<SA_TENSOR, SB_TENSOR, true>(g, bf, st);
            else launch_typed<SA_TENSOR, SB_TENSOR, false>(g, bf, st);
        }
    }
}

bool launch_gemm_e4m3(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const float* sa,
                      int64_t ldsa, int sa_kind, const uint8_t* b, int64_t ldb, int b_layout,
                      const float* sb, int64_t ldsb, int sb_kind, uint8_t* q, int64_t ldq, float* s,
                      int64_t lds, hipStream_t st)
{
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.a = a; g.lda = lda; g.sa = sa; g.ldsa = ldsa;
    g.b = b; g.ldb = ldb; g.sb = sb; g.ldsb = ldsb;
    g.c = q; g.ldc = ldq;
    g.cs = s; g.ldcs = lds;
    g.KB = (int)((K + BK - 1) / BK);
    g.num_cus = device_cu_count();
    const int sa_mode = sa_kind == FP8Q_ROW_1x128 ? SA_ROW : SA_TENSOR;
    if (sb_kind == FP8Q_ROW_1x128) return false;   // row-scaled B: fp32/bf16 output only
    const int sb_mode = sb_kind == FP8Q_BLOCK_128x128 ? SB_BLOCK : SB_TENSOR;
    return launch_gemm_nk(g, sa_mode, sb_mode, b_layout == FP8Q_B_KN, OUT_E4M3, st);
}

bool launch_gemm_e8m0(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const uint8_t* ea,
                      int64_t ldea, const uint8_t* b, int64_t ldb, int b_layout, const uint8_t* eb,
                      int64_t ldeb, int eb_kind, void* c, int64_t ldc, int c_dtype, hipStream_t st)
{
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.a = a; g.lda = lda; g.sa = reinterpret_cast<const float*>(ea); g.ldsa = ldea;
    g.b = b; g.ldb = ldb; g.sb = reinterpret_cast<const float*>(eb); g.ldsb = ldeb;
    g.c = c; g.ldc = ldc;
    g.KB = (int)((K + BK - 1) / BK);
    g.num_cus = device_cu_count();
    return launch_gemm_nk_e8m0(g, eb_kind == FP8Q_ROW_1x128 ? SB_ROW : SB_BLOCK, b_layout == FP8Q_B_KN,
                               c_dtype == FP8Q_BF16, st);
}

void launch_grouped_gemm(int64_t G, int64_t M_pad, int64_t N, int64_t K, const uint8_t* a,
                         int64_t lda, const float* sa, int64_t ldsa, const int32_t* offsets,
                         const uint8_t* b, const float* sb, void* c, int64_t ldc, int c_dtype,
                         hipStream_t st)
{
    GemmArgs g{};
    g.M = M_pad; g.N = N; g.K = K;
    g.a = a; g.lda = lda; g.sa = sa; g.ldsa = ldsa;
    g.b = b; g.ldb = K; g.sb = sb;
    g.KB = (int)((K + BK - 1) / BK);
    g.ldsb = g.KB;
    g.c = c; g.ldc = ldc;
    g.tiles_m = (int)(M_pad / 128);
    g.tiles_n = (int)((N + BN - 1) / BN);
    g.offsets = offsets;
    g.G = (int)G;
    g.b_group_stride = N * K;
    g.sb_group_stride = ((N + 127) / 128) * (int64_t)g.KB;
    g.num_cus = device_cu_count();
    if (launch_grouped_gemm_nk(g, c_dtype == FP8Q_BF16, false, st)) return;
    dim3 grid((uint32_t)(g.tiles_m * g.tiles_n));
    if (c_dtype == FP8Q_BF16)
        hipLaunchKernelGGL((gemm_kernel<128, SA_ROW, SB_BLOCK, false, true, true>), grid,
                           dim3(kGemmThreads), 0, st, g);
    else
        hipLaunchKernelGGL((gemm_kernel<128, SA_ROW, SB_BLOCK, false, false, true>), grid,
                           dim3(kGemmThreads), 0, st, g);
}

bool launch_grouped_gemm_dgrad(int64_t G, int64_t M_pad, int64_t N, int64_t K, const uint8_t* a,
                               int64_t lda, const float* sa, int64_t ldsa, const int32_t* offsets,
                               const uint8_t* w, const float* sw, void* c, int64_t ldc, int c_dtype,
                               hipStream_t st)
{
    // dX[m][k] = sum_n dY[m][n] W_e[n][k]: contraction over W's rows, so in
    // GEMM terms M = M_pad, N = K, K = N and B is W_e read as stored ([K][N])
    GemmArgs g{};
    g.M = M_pad; g.N = K; g.K = N;
    g.a = a; g.lda = lda; g.sa = sa; g.ldsa = ldsa;
    g.b = w; g.ldb = K; g.sb = sw;
    g.KB = (int)((N + BK - 1) / BK);
    g.ldsb = (K + 127) / 128;
    g.c = c; g.ldc = ldc;
    g.offsets = offsets;
    g.G = (int)G;
    g.b_group_stride = N * K;
    g.sb_group_stride = (int64_t)g.KB * g.ldsb;
    g.num_cus = device_cu_count();
    return launch_grouped_gemm_nk(g, c_dtype == FP8Q_BF16, true, st);
}

bool launch_grouped_gemm_wgrad(int64_t G, int64_t M_pad, int64_t N, int64_t K, const uint8_t* a,
                               int64_t lda, const float* sa, int64_t ldsa, const uint8_t* b,
                               int64_t ldb, const float* sb, int64_t ldsb, const int32_t* offsets,
                               float* c, int64_t ldc, hipStream_t st)
{
    // dW_e[n][k] = sum over the group's tokens t of dYT[n][t] XT[k][t]: rows
    // of A and B are N and K, the contraction runs over the group's tokens
    GemmArgs g{};
    g.M = N; g.N = K; g.K = M_pad;
    g.a = a; g.lda = lda; g.sa = sa; g.ldsa = ldsa;
    g.b = b; g.ldb = ldb; g.sb = sb; g.ldsb = ldsb;
    g.KB = (int)(M_pad / BK);
    g.c = c; g.ldc = ldc;
    g.offsets = offsets;
    g.G = (int)G;
    g.c_group_stride = N * ldc;
    g.num_cus = device_cu_count();
    return launch_grouped_wgrad_nk(g, st);
}

}  // namespace fp8q
