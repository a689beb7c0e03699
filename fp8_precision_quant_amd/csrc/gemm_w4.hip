// Block-scaled FP8 GEMM on gfx950, four-wave form: one wave per SIMD.
//
//   C[m][n] = sum_kb SA(m,kb) * SB(n,kb) * sum_{k in chunk kb} dec(A[m][k]) * dec(B[n][k])
//
// (FP8 Linear with an FP32 accumulator: Ling 2.0 FP8 blog, "where does the
// worry come from" and "where is error introduced"; per-tile activation and
// 128x128 weight-block scales: same blog, "fine-grained quantization", and
// "FP8-RL" article, 一; the weight read as stored for dgrad: "FP8 on-demand
// transpose weight".)
//
// The same 128 x 256 x 128 tile, LDS layout and direct global -> LDS loads
// as gemm_nk.hip, with a different division of work:
//  * four waves per workgroup, one per SIMD, each owning all 128 rows of 64
//    columns for every K chunk, so no partial tiles are exchanged;
//  * one wave per SIMD may hold 512 registers: the operand fragments of two
//    chunks live in fixed accumulation registers a0..a191 (the chunk being
//    multiplied and the next one, read from LDS while the current one runs),
//    the fp32 accumulators, chunk partials and scales in ordinary registers;
//  * each chunk is 32 steps; a step issues one MFMA, one or two LDS reads of
//    the next chunk or one direct load of the chunk three ahead, and the
//    scale FMAs of the block whose MFMA was issued three steps earlier (so
//    the FMAs never wait on their own MFMA and need no hazard padding);
//  * one barrier per chunk: before it every wave has its own loads of the
//    next chunk in LDS and has finished reading the current one, whose stage
//    then takes the chunk three ahead.  The loads run on across tiles, so the
//    next tile's first chunks arrive while the current tile is stored.
// Fragment registers are named in the instructions (the compiler cannot be
// made to place a fragment's two 16-byte halves in adjacent registers), so
// every fragment read declares them clobbered and the compiler allocates no
// accumulation registers of its own in this kernel.
#include <type_traits>

#include "fp8q_device.h"
#include "fp8q_internal.h"
#include "gemm_common.h"
#include "gemm_lds.h"

namespace fp8q {

namespace {

constexpr int kW4Threads = 256;

// fragment F (0..23) lives in a[8F .. 8F+7]: set s, A fragment i -> F = 12 s + i;
// B fragment j -> F = 12 s + 8 + j.  Columns: F, low and high 16-byte halves.
#define W4_FRAGS(X) \
    X(0, "a[0:3]", "a[4:7]") \
    X(1, "a[8:11]", "a[12:15]") \
    X(2, "a[16:19]", "a[20:23]") \
    X(3, "a[24:27]", "a[28:31]") \
    X(4, "a[32:35]", "a[36:39]") \
    X(5, "a[40:43]", "a[44:47]") \
    X(6, "a[48:51]", "a[52:55]") \
    X(7, "a[56:59]", "a[60:63]") \
    X(8, "a[64:67]", "a[68:71]") \
    X(9, "a[72:75]", "a[76:79]") \
    X(10, "a[80:83]", "a[84:87]") \
    X(11, "a[88:91]", "a[92:95]") \
    X(12, "a[96:99]", "a[100:103]") \
    X(13, "a[104:107]", "a[108:111]") \
    X(14, "a[112:115]", "a[116:119]") \
    X(15, "a[120:123]", "a[124:127]") \
    X(16, "a[128:131]", "a[132:135]") \
    X(17, "a[136:139]", "a[140:143]") \
    X(18, "a[144:147]", "a[148:151]") \
    X(19, "a[152:155]", "a[156:159]") \
    X(20, "a[160:163]", "a[164:167]") \
    X(21, "a[168:171]", "a[172:175]") \
    X(22, "a[176:179]", "a[180:183]") \
    X(23, "a[184:187]", "a[188:191]")

// the four 8-byte quarters of fragment F (transposing reads of B read as stored)
#define W4_QUARTERS(X) \
    X(0, "a[0:1]", "a[2:3]", "a[4:5]", "a[6:7]") \
    X(1, "a[8:9]", "a[10:11]", "a[12:13]", "a[14:15]") \
    X(2, "a[16:17]", "a[18:19]", "a[20:21]", "a[22:23]") \
    X(3, "a[24:25]", "a[26:27]", "a[28:29]", "a[30:31]") \
    X(4, "a[32:33]", "a[34:35]", "a[36:37]", "a[38:39]") \
    X(5, "a[40:41]", "a[42:43]", "a[44:45]", "a[46:47]") \
    X(6, "a[48:49]", "a[50:51]", "a[52:53]", "a[54:55]") \
    X(7, "a[56:57]", "a[58:59]", "a[60:61]", "a[62:63]") \
    X(8, "a[64:65]", "a[66:67]", "a[68:69]", "a[70:71]") \
    X(9, "a[72:73]", "a[74:75]", "a[76:77]", "a[78:79]") \
    X(10, "a[80:81]", "a[82:83]", "a[84:85]", "a[86:87]") \
    X(11, "a[88:89]", "a[90:91]", "a[92:93]", "a[94:95]") \
    X(12, "a[96:97]", "a[98:99]", "a[100:101]", "a[102:103]") \
    X(13, "a[104:105]", "a[106:107]", "a[108:109]", "a[110:111]") \
    X(14, "a[112:113]", "a[114:115]", "a[116:117]", "a[118:119]") \
    X(15, "a[120:121]", "a[122:123]", "a[124:125]", "a[126:127]") \
    X(16, "a[128:129]", "a[130:131]", "a[132:133]", "a[134:135]") \
    X(17, "a[136:137]", "a[138:139]", "a[140:141]", "a[142:143]") \
    X(18, "a[144:145]", "a[146:147]", "a[148:149]", "a[150:151]") \
    X(19, "a[152:153]", "a[154:155]", "a[156:157]", "a[158:159]") \
    X(20, "a[160:161]", "a[162:163]", "a[164:165]", "a[166:167]") \
    X(21, "a[168:169]", "a[170:171]", "a[172:173]", "a[174:175]") \
    X(22, "a[176:177]", "a[178:179]", "a[180:181]", "a[182:183]") \
    X(23, "a[184:185]", "a[186:187]", "a[188:189]", "a[190:191]")

#define W4_AGPRS "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", "a10", "a11", "a12", "a13", "a14", "a15", "a16", "a17", "a18", "a19", "a20", "a21", "a22", "a23", "a24", "a25", "a26", "a27", "a28", "a29", "a30", "a31", "a32", "a33", "a34", "a35", "a36", "a37", "a38", "a39", "a40", "a41", "a42", "a43", "a44", "a45", "a46", "a47", "a48", "a49", "a50", "a51", "a52", "a53", "a54", "a55", "a56", "a57", "a58", "a59", "a60", "a61", "a62", "a63", "a64", "a65", "a66", "a67", "a68", "a69", "a70", "a71", "a72", "a73", "a74", "a75", "a76", "a77", "a78", "a79", "a80", "a81", "a82", "a83", "a84", "a85", "a86", "a87", "a88", "a89", "a90", "a91", "a92", "a93", "a94", "a95", "a96", "a97", "a98", "a99", "a100", "a101", "a102", "a103", "a104", "a105", "a106", "a107", "a108", "a109", "a110", "a111", "a112", "a113", "a114", "a115", "a116", "a117", "a118", "a119", "a120", "a121", "a122", "a123", "a124", "a125", "a126", "a127", "a128", "a129", "a130", "a131", "a132", "a133", "a134", "a135", "a136", "a137", "a138", "a139", "a140", "a141", "a142", "a143", "a144", "a145", "a146", "a147", "a148", "a149", "a150", "a151", "a152", "a153", "a154", "a155", "a156", "a157", "a158", "a159", "a160", "a161", "a162", "a163", "a164", "a165", "a166", "a167", "a168", "a169", "a170", "a171", "a172", "a173", "a174", "a175", "a176", "a177", "a178", "a179", "a180", "a181", "a182", "a183", "a184", "a185", "a186", "a187", "a188", "a189", "a190", "a191"

// A fragments (multiplicand rows) and B fragments by number, for the MFMA
#define W4_A_LIST(X, B) \
    X(B, 0, "a[0:7]") \
    X(B, 1, "a[8:15]") \
    X(B, 2, "a[16:23]") \
    X(B, 3, "a[24:31]") \
    X(B, 4, "a[32:39]") \
    X(B, 5, "a[40:47]") \
    X(B, 6, "a[48:55]") \
    X(B, 7, "a[56:63]") \
    X(B, 12, "a[96:103]") \
    X(B, 13, "a[104:111]") \
    X(B, 14, "a[112:119]") \
    X(B, 15, "a[120:127]") \
    X(B, 16, "a[128:135]") \
    X(B, 17, "a[136:143]") \
    X(B, 18, "a[144:151]") \
    X(B, 19, "a[152:159]")
#define W4_B_LIST(X) \
    X(8, "a[64:71]") \
    X(9, "a[72:79]") \
    X(10, "a[80:87]") \
    X(11, "a[88:95]") \
    X(20, "a[160:167]") \
    X(21, "a[168:175]") \
    X(22, "a[176:183]") \
    X(23, "a[184:191]")

// 16-byte LDS read into half H (0 low, 1 high) of fragment F
template <int F, int H, int OFF>
__device__ __forceinline__ void w4_read_half(uint32_t addr)
{
#define X(FI, LO, HI) \
    if constexpr (F == FI) { \
        if constexpr (H == 0) asm volatile("ds_read_b128 " LO ", %0 offset:%1" ::"v"(addr), "i"(OFF) : "memory", W4_AGPRS); \
        else asm volatile("ds_read_b128 " HI ", %0 offset:%1" ::"v"(addr), "i"(OFF) : "memory", W4_AGPRS); \
    }
    W4_FRAGS(X)
#undef X
}

// transposing 8-byte LDS read into quarter Q of fragment F
template <int F, int Q, int OFF>
__device__ __forceinline__ void w4_read_quarter(uint32_t addr)
{
#define X(FI, Q0, Q1, Q2, Q3) \
    if constexpr (F == FI) { \
        if constexpr (Q == 0) asm volatile("ds_read_b64_tr_b8 " Q0 ", %0 offset:%1" ::"v"(addr), "i"(OFF) : "memory", W4_AGPRS); \
        else if constexpr (Q == 1) asm volatile("ds_read_b64_tr_b8 " Q1 ", %0 offset:%1" ::"v"(addr), "i"(OFF) : "memory", W4_AGPRS); \
        else if constexpr (Q == 2) asm volatile("ds_read_b64_tr_b8 " Q2 ", %0 offset:%1" ::"v"(addr), "i"(OFF) : "memory", W4_AGPRS); \
        else asm volatile("ds_read_b64_tr_b8 " Q3 ", %0 offset:%1" ::"v"(addr), "i"(OFF) : "memory", W4_AGPRS); \
    }
    W4_QUARTERS(X)
#undef X
}

// the chunk's fp32 partial of one 16 x 16 block: fragment FB (B rows) times FA (A rows)
template <int FB, int FA>
__device__ __forceinline__ void w4_mfma(v4f& d)
{
#define W4_MF_A(BFULL, FAI, AFULL) \
    if constexpr (FA == FAI) asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, " BFULL ", " AFULL ", 0" : "=v"(d) : : "memory");
#define W4_MF_B(FBI, BFULL) \
    if constexpr (FB == FBI) { W4_A_LIST(W4_MF_A, BFULL) }
    W4_B_LIST(W4_MF_B)
#undef W4_MF_B
#undef W4_MF_A
}

// the same with power-of-two scales applied by the matrix core (E8M0 bytes
// in bits 0-7 of sb for the B rows, of sa for the A rows), accumulating in d
template <int FB, int FA>
__device__ __forceinline__ void w4_mfma_scaled(v4f& d, int sb, int sa)
{
#define W4_MS_A(BFULL, FAI, AFULL) \
    if constexpr (FA == FAI) asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, " BFULL ", " AFULL ", %0, %1, %2" : "+v"(d) : "v"(sb), "v"(sa) : "memory");
#define W4_MS_B(FBI, BFULL) \
    if constexpr (FB == FBI) { W4_A_LIST(W4_MS_A, BFULL) }
    W4_B_LIST(W4_MS_B)
#undef W4_MS_B
#undef W4_MS_A
}

template <int OFF>
__device__ __forceinline__ int w4_ds8(uint32_t addr)
{
    int v;
    asm volatile("ds_read_u8 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
    return v;
}

__device__ __forceinline__ void w4_fmac(float& acc, float p, float s)
{
    asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(acc) : "v"(p), "v"(s) : "memory");
}

// max(m, |a|, |b|) for m >= 0 and finite a, b (exact; no NaN quieting, which
// the compiler would otherwise add for values it cannot see the origin of)
__device__ __forceinline__ float w4_max3_abs(float m, float a, float b)
{
    float d;
    asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(d) : "v"(m), "v"(a), "v"(b));
    return d;
}

__device__ __forceinline__ void w4_mul(float& d, float a, float b)
{
    asm volatile("v_mul_f32_e32 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b) : "memory");
}

// one lane's fp32 scale from LDS (a load: its result is used only after the
// chunk's closing wait, which names it)
template <int OFF>
__device__ __forceinline__ float w4_ds32(uint32_t addr)
{
    float v;
    asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
    return v;
}

template <int OFF>
__device__ __forceinline__ v4f w4_ds128(uint32_t addr)
{
    v4f v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
    return v;
}

}  // namespace

namespace {

template <int I, int N, typename F>
__device__ __forceinline__ void w4_for(F&& f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        w4_for<I + 1, N>(f);
    }
}

template <int N>
__device__ __forceinline__ void w4_wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// the scales of one chunk as a lane uses them
template <int SB_MODE>
struct W4Scales {
    float sa[PMI];                            // SA of the lane's row in 16-row block i
    float sb;                                 // SB of the wave's 128-column block
    v4f sc[SB_MODE == SB_ROW ? NNI : 1];      // SB of the lane's 4 columns in 16-column block j
    float comb[PMI];                          // SA * SB (uniform B scale)
    int e[PMI];                               // power-of-two scales: E8M0 byte of the lane's A row in block i
    int eb[SB_MODE == SB_ROW ? NNI : 1];      // ... of its B row (column of block j, or the wave's block)
};

}  // namespace

// GMODE 0: one dense product.
// GMODE 1 (MoE forward, groups of rows): row tile m0 belongs to group e with
//   off[e] <= m0 < off[e+1] (offsets held in LDS), whose expert's B and block
//   scales it multiplies; rows at or past off[G] are not stored.
// GMODE 2 (MoE weight gradient, groups of K): the tiles of output block e
//   (dW[e] = p.c + e * c_group_stride) contract over the chunks
//   [off[e], off[e+1]) / 128 of the token axis only.  Non-empty groups are
//   ranked by size and dealt to the XCDs in snake order (ranks 0..7 to XCDs
//   0..7, 8..15 to 7..0, ...); each XCD's workgroups walk its groups' tiles,
//   largest group first, so a group's operands share one L2 and the K loops
//   balance across XCDs.  Empty groups get dW[e] = 0, their tiles stored by
//   all workgroups before the chunk stream.
// B_KN: B read as stored [K][N] (dgrad: the weight, or the MoE experts'
// weights, without a transposed copy): the load stages 32 K rows x 256
// columns per wave and the fragment reads transpose 8-byte quarters
// (ds_read_b64_tr_b8), twice the reads of [N][K] B.
// P2: power-of-two scales as E8M0 bytes (p.sa / p.sb point at bytes; the
// micro-scaling form of block scaling), applied by the scaled MFMA, which
// accumulates straight into the tile: no chunk partials, no scale FMAs.
// Each chunk loads the 4-byte word of a scale row that holds its byte (the
// grids' row strides are multiples of 4) and the reads select the byte.
template <int SA_MODE, int SB_MODE, int OUT, int GMODE, bool B_KN = false, bool P2 = false>
__global__ __launch_bounds__(kW4Threads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_w4_kernel(GemmArgs p)
{
    static_assert(!P2 || (GMODE == 0 && SA_MODE == SA_ROW && SB_MODE != SB_TENSOR && OUT != OUT_E4M3),
                  "power-of-two scales: dense, row-scaled A, row- or block-scaled B, fp32 or bf16 out");
    static_assert(!B_KN || (GMODE <= 1 && SB_MODE != SB_ROW), "[K][N] B: block or tensor scales, no groups of K");
    static_assert(GMODE != 1 || (SA_MODE == SA_ROW && SB_MODE == SB_BLOCK && (OUT != OUT_E4M3 || !B_KN)),
                  "groups of rows: row-scaled A, block-scaled B; E4M3 out for [N][K] B (the forward)");
    static_assert(GMODE != 2 || (SA_MODE == SA_ROW && SB_MODE == SB_ROW && OUT == OUT_F32),
                  "groups of K: row-scaled A and B, fp32 out");
    static_assert(OUT != OUT_E4M3 || SB_MODE != SB_ROW, "quantize-on-store: uniform B scales");
    // direct loads per chunk and wave: 4 of A, 8 of B, one of A's and one of
    // B's scales where they are per row / per block
    constexpr int ND = 12 + (SA_MODE == SA_ROW ? 1 : 0) + (SB_MODE != SB_TENSOR ? 1 : 0);
    __shared__ __attribute__((aligned(16))) uint8_t Stg[kStages][kStageBytes];
    __shared__ __attribute__((aligned(16))) float SAs[kStages][TBM];
    __shared__ __attribute__((aligned(16))) float SBs[kStages][SB_MODE == SB_ROW ? TBN : 4];
    // quantize-on-store: each wave's row maxima over its 64 columns
    __shared__ float RowMax[OUT == OUT_E4M3 ? kW4Threads / 64 : 1][OUT == OUT_E4M3 ? TBM : 1];
    __shared__ int32_t goff[GMODE != 0 ? kMaxLdsGroups + 1 : 1];
    // groups of K: this XCD's groups, largest first
    __shared__ int32_t xlist[GMODE == 2 ? kMaxLdsGroups / 8 + 1 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wq = __builtin_amdgcn_readfirstlane(tid >> 6);   // columns [64 wq, 64 wq + 64) of the tile

    if (GMODE != 0) {
        for (int i = tid; i <= p.G; i += kW4Threads) goff[i] = p.offsets[i];
        __syncthreads();
    }

    // Persistent workgroups dealt to the 8 XCDs round-robin; XCD x owns a
    // contiguous range of tile ids, walked by its workgroups in lockstep in
    // groups of kGM M-tiles (neighbouring workgroups share A and B panels
    // in that XCD's L2).
    const int T = p.tiles_m * p.tiles_n;
    const int xcd = blockIdx.x & 7;
    const int local = blockIdx.x >> 3;
    const int nwg = (gridDim.x >> 3) + (xcd < (int)(gridDim.x & 7) ? 1 : 0);
    const int range_start = xcd * (T >> 3) + min(xcd, T & 7);
    int tiles_here = (T >> 3) + (xcd < (T & 7) ? 1 : 0);
    // (row-scaled B, the weight gradient: groups of 8 M-tiles measured 2%
    // faster than 16; the other layouts keep 16)
    constexpr int kGM = (GMODE == 0 && SB_MODE == SB_ROW) ? 8 : kGroupM;
    const int span = kGM * p.tiles_n;
    const int64_t M = p.M, N = p.N, K = p.K;
    if constexpr (GMODE == 2) {
        int gn = 0;   // non-empty groups
        for (int f = 0; f < p.G; ++f) gn += goff[f + 1] > goff[f] ? 1 : 0;
        for (int e = tid; e < p.G; e += kW4Threads) {
            const int size = goff[e + 1] - goff[e];
            if (size == 0) continue;
            int rank = 0;
            for (int f = 0; f < p.G; ++f) {
                const int sf = goff[f + 1] - goff[f];
                rank += (sf > size || (sf == size && f < e)) ? 1 : 0;
            }
            const int x = ((rank >> 3) & 1) ? 7 - (rank & 7) : (rank & 7);
            if (x == xcd) xlist[rank >> 3] = e;
        }
        __syncthreads();
        const int q = gn >> 3, rem = gn & 7;
        const int nx = q + ((q & 1) ? (xcd >= 8 - rem ? 1 : 0) : (xcd < rem ? 1 : 0));
        tiles_here = nx * T;
        // dW[e] = 0 for the empty groups: (empty group, tile) pairs dealt to
        // all workgroups, 128 x 256 fp32 zeros per tile
        const int ne = p.G - gn;
        for (int j = blockIdx.x; j < ne * T; j += gridDim.x) {
            int e = -1;
            for (int f = 0, k = j / T; f < p.G; ++f) {
                if (goff[f + 1] == goff[f] && k-- == 0) {
                    e = f;
                    break;
                }
            }
            if (e < 0) break;   // (not reached: j < ne * T)
            const int t = j % T;
            const int64_t zm0 = (int64_t)(t % p.tiles_m) * TBM, zn0 = (int64_t)(t / p.tiles_m) * TBN;
            float* cz = reinterpret_cast<float*>(p.c) + (int64_t)e * p.c_group_stride;
            for (int i = tid; i < TBM * (TBN / 4); i += kW4Threads) {
                const int64_t m = zm0 + i / (TBN / 4), n = zn0 + 4 * (i % (TBN / 4));
                if (m >= M) continue;
                if (n + 3 < N) {
                    *reinterpret_cast<v4f*>(cz + m * p.ldc + n) = v4f{0.f, 0.f, 0.f, 0.f};
                } else {
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N) cz[m * p.ldc + n + r] = 0.0f;
                }
            }
        }
    }
    if (local >= tiles_here) return;
    // group of row tile m0 (wave-uniform): the last e with off[e] <= m0
    auto group_of = [&](int64_t m0) __attribute__((always_inline)) {
        int lo = 0, hi = p.G - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((int64_t)goff[mid] <= m0) lo = mid; else hi = mid - 1;
        }
        return __builtin_amdgcn_readfirstlane(lo);
    };
    // Tile `ordinal` of this workgroup: origin, group, and its chunks
    // [kb0, kb0 + kbn) of the K axis.
    struct Tile {
        int64_t m0, n0;
        int e, kb0, kbn;
    };
    auto tile_at = [&](int ordinal) __attribute__((always_inline)) {
        Tile t;
        t.e = 0;
        t.kb0 = 0;
        t.kbn = p.KB;
        if constexpr (GMODE == 2) {
            const int i = local + ordinal * nwg;
            t.e = __builtin_amdgcn_readfirstlane(xlist[i / T]);
            const int r = i % T;
            t.m0 = (int64_t)(r % p.tiles_m) * TBM;
            t.n0 = (int64_t)(r / p.tiles_m) * TBN;
            t.kb0 = __builtin_amdgcn_readfirstlane(goff[t.e]) / TBK;
            t.kbn = __builtin_amdgcn_readfirstlane(goff[t.e + 1]) / TBK - t.kb0;
        } else {
            const int pid = range_start + local + ordinal * nwg;
            const int group = pid / span;
            const int first_m = group * kGM;
            const int gsz = min(p.tiles_m - first_m, kGM);
            const int idx = pid - group * span;
            t.m0 = (int64_t)(first_m + idx % gsz) * TBM;
            t.n0 = (int64_t)(idx / gsz) * TBN;
            if constexpr (GMODE == 1) t.e = group_of(t.m0);
        }
        return t;
    };
    const int my_tiles = (tiles_here - local + nwg - 1) / nwg;
    const int KB = p.KB;

    // Buffer resources bound every load to its operand; rows past M or N
    // start past the bound and read as zero (they feed outputs not stored).
    const int64_t nblocks = (N + 127) / 128;
    const __amdgpu_buffer_rsrc_t ra = rsrc(p.a, (M - 1) * p.lda + K);
    const int64_t b_ext = B_KN ? (K - 1) * p.ldb + ((N + 15) & ~(int64_t)15) : (N - 1) * p.ldb + K;
    __amdgpu_buffer_rsrc_t rb = rsrc(p.b, b_ext);
    // (E8M0 grids: byte extents, each row's last word included)
    const int64_t kb_words = (KB + 3) & ~3, nb_words = (nblocks + 3) & ~3;
    const __amdgpu_buffer_rsrc_t rsa =
        rsrc(p.sa, SA_MODE != SA_ROW ? 4 : P2 ? (M - 1) * p.ldsa + kb_words : ((M - 1) * p.ldsa + KB) * 4);
    __amdgpu_buffer_rsrc_t rsb =
        rsrc(p.sb, SB_MODE == SB_ROW     ? (P2 ? (N - 1) * p.ldsb + kb_words : ((N - 1) * p.ldsb + KB) * 4)
                   : SB_MODE == SB_BLOCK ? (P2 ? (B_KN ? (int64_t)(KB - 1) * p.ldsb + nb_words
                                                       : (nblocks - 1) * p.ldsb + kb_words)
                                               : B_KN ? ((int64_t)(KB - 1) * p.ldsb + nblocks) * 4
                                                      : ((nblocks - 1) * p.ldsb + KB) * 4)
                                         : 4);
    const float sa_t = SA_MODE == SA_TENSOR ? p.sa[0] : 0.0f;
    const float sb_t = SB_MODE == SB_TENSOR ? p.sb[0] : 0.0f;

    // ---- loads (the load cursor runs three chunks ahead of the MFMAs) ----
    // This wave loads A rows [32 wq, 32 wq + 32) (4 loads of 8 rows), B rows
    // [64 wq, 64 wq + 64) (8 loads of 8 rows), A's row scales of rows
    // [32 wq, 32 wq + 32), and its own B scales.  Load t differs from
    // load 0 by t row steps (scalar offset) and, for odd t, by the swizzle key.
    int ld_ord = 0, ld_k = 0;
    Tile lt = tile_at(0);
    uint32_t va0, va1, vb0, vb1, vsa = 0, vsb = 0;
    auto load_offsets = [&]() __attribute__((always_inline)) {
        const int l = lane;
        const int64_t lm0 = lt.m0, ln0 = lt.n0;
        const int64_t arow = lm0 + 32 * wq + (l >> 3);
        va0 = (uint32_t)(arow * p.lda) + 16u * (uint32_t)((l & 7) ^ (l >> 3));
        va1 = (uint32_t)(arow * p.lda) + 16u * (uint32_t)((l & 7) ^ (l >> 3) ^ 1);
        if (B_KN) {
            // K rows [32 wq, 32 wq + 32) of the chunk, 4 per load, each 256
            // columns; the 16-byte slot of column group (l & 15) is xor-ed
            // with the row's key
            const int r = 32 * wq + (l >> 4);
            const int k0 = (l >> 4) ^ (8 * (wq & 1)), k1 = (4 + (l >> 4)) ^ (8 * (wq & 1));
            vb0 = (uint32_t)(r * p.ldb + ln0) + 16u * (uint32_t)((l & 15) ^ k0);
            vb1 = (uint32_t)(r * p.ldb + ln0) + 16u * (uint32_t)((l & 15) ^ k1);
        } else {
            const int64_t brow = ln0 + 64 * wq + (l >> 3);
            vb0 = (uint32_t)(brow * p.ldb) + 16u * (uint32_t)((l & 7) ^ (l >> 3));
            vb1 = (uint32_t)(brow * p.ldb) + 16u * (uint32_t)((l & 7) ^ (l >> 3) ^ 1);
        }
        constexpr int se = P2 ? 1 : 4;   // bytes per scale
        if (SA_MODE == SA_ROW) vsa = (uint32_t)((lm0 + 32 * wq + l) * p.ldsa * se);
        if (SB_MODE == SB_ROW) vsb = (uint32_t)((ln0 + 64 * wq + l) * p.ldsb * se);
        if (SB_MODE == SB_BLOCK) {
            const int64_t nb = ln0 / 128 + (wq >> 1);
            vsb = P2 ? (uint32_t)(B_KN ? (nb & ~(int64_t)3) : nb * p.ldsb) : (uint32_t)(nb * (B_KN ? 4 : p.ldsb * 4));
        }
        if (GMODE == 1) {
            // the expert of the load cursor's tile: its B and block scales
            rb = rsrc(p.b + (int64_t)lt.e * p.b_group_stride, b_ext);
            rsb = rsrc(p.sb + (int64_t)lt.e * p.sb_group_stride, p.sb_group_stride * 4);
        }
    };
    load_offsets();
    // load d (0 .. ND-1) of the cursor's chunk into stage st
    auto load_item = [&](auto dt, int st) __attribute__((always_inline)) {
        constexpr int d = decltype(dt)::value;
        const uint32_t kg = (uint32_t)(lt.kb0 + ld_k);
        if constexpr (d < 4) {
            dma16_at(ra, lds_addr(&Stg[st][0]) + (uint32_t)((32 * wq + 8 * d) * TBK), (d & 1) ? va1 : va0,
                     kg * TBK + (uint32_t)(8 * d) * (uint32_t)p.lda);
        } else if constexpr (d < 12) {
            constexpr int t = d - 4;
            if constexpr (B_KN)
                dma16_at(rb, lds_addr(&Stg[st][kAStage]) + (uint32_t)((32 * wq + 4 * t) * TBN), (t & 1) ? vb1 : vb0,
                         (kg * TBK + 4u * t) * (uint32_t)p.ldb);
            else
                dma16_at(rb, lds_addr(&Stg[st][kAStage]) + (uint32_t)((64 * wq + 8 * t) * TBK), (t & 1) ? vb1 : vb0,
                         kg * TBK + 8u * t * (uint32_t)p.ldb);
        } else if constexpr (SA_MODE == SA_ROW && d == 12) {
            // (E8M0: the word of the row that holds the chunk's byte)
            if (lane < 32) dma4(rsa, &SAs[st][32 * wq], vsa, P2 ? (kg & ~3u) : kg * 4);
        } else {
            if constexpr (SB_MODE == SB_ROW) dma4(rsb, &SBs[st][64 * wq], vsb, P2 ? (kg & ~3u) : kg * 4);
            if constexpr (SB_MODE == SB_BLOCK) {
                if (lane == 0)
                    dma4(rsb, &SBs[st][wq], vsb,
                         B_KN ? kg * (uint32_t)p.ldsb * (P2 ? 1u : 4u) : (P2 ? (kg & ~3u) : kg * 4));
            }
        }
    };
    // (past the last tile the cursor stays on it: the loads it then issues
    // read valid memory into a free stage and are never used, which keeps
    // the loads per chunk, and so the wait counts, the same for every chunk)
    auto load_advance = [&]() __attribute__((always_inline)) {
        if (++ld_k == lt.kbn) {
            ld_k = 0;
            if (ld_ord + 1 < my_tiles) {
                ++ld_ord;
                lt = tile_at(ld_ord);
                load_offsets();
            }
        }
    };

    // ---- LDS reads of a chunk into fragment set NS (fixed registers) ----
    const int lrow = lane & 15, kgrp = lane >> 4;
    const uint32_t stg0 = lds_addr(&Stg[0][0]);
    const uint32_t a_rel0 = (uint32_t)sw(lrow, 2 * kgrp), a_rel1 = (uint32_t)sw(lrow, 2 * kgrp + 1);
    const uint32_t b_rel0 = (uint32_t)(kAStage + sw(64 * wq + lrow, 2 * kgrp));
    const uint32_t b_rel1 = (uint32_t)(kAStage + sw(64 * wq + lrow, 2 * kgrp + 1));
    // [K][N] B: lane (kgrp, lrow) addresses K row 32 kgrp + lrow / 2 at column
    // 64 wq + 16 j + 8 (lrow & 1); fragment j is fragment 0 with the 16-byte
    // slot index xor j
    uint32_t kn_rel[NNI] = {};
    if (B_KN) {
        const int r = 32 * kgrp + (lrow >> 1);
        const uint32_t rel = (uint32_t)(kAStage + r * TBN + (((4 * wq) ^ kn_key(r)) << 4) + 8 * (lrow & 1));
#pragma unroll
        for (int j = 0; j < NNI; ++j) kn_rel[j] = rel ^ (uint32_t)(j << 4);
    }
    const uint32_t sa_rel = lds_addr(&SAs[0][0]) + (uint32_t)lrow * 4;
    // E8M0 B row scales: the lane's B row 64 wq + 16 j + lrow
    const uint32_t sbp_rel = lds_addr(&SBs[0][0]) + (uint32_t)(64 * wq + lrow) * 4;
    // E8M0: the read cursor (chunk being read into registers) and the byte
    // of the staged scale words that belongs to it: byte kb & 3 of a row's
    // word; for [K][N] B's block scales byte (n0 / 128 + wave block) & 3
    int rd_k = 0, rd_ord = 0;
    int64_t rd_n0 = P2 ? tile_at(0).n0 : 0;
    uint32_t rsel = 0, bsel = 0;
    auto read_cursor_set = [&]() __attribute__((always_inline)) {
        rsel = (uint32_t)(rd_k & 3);
        bsel = B_KN ? (uint32_t)((rd_n0 / 128 + (wq >> 1)) & 3) : rsel;
    };
    auto read_advance = [&]() __attribute__((always_inline)) {
        if (++rd_k == p.KB) {
            rd_k = 0;
            if (++rd_ord < my_tiles) rd_n0 = tile_at(rd_ord).n0;
        }
        read_cursor_set();
    };
    const uint32_t sb_rel = SB_MODE == SB_ROW ? lds_addr(&SBs[0][0]) + (uint32_t)(64 * wq + 4 * kgrp) * 4
                                              : lds_addr(&SBs[0][0]) + (uint32_t)wq * 4;

    W4Scales<SB_MODE> scl[2];
    // read item k (0 .. 31) of the chunk in stage st into fragment set NS and
    // scale set NS: 0-1 B0, 2-17 A0..A7 (two halves each), 18-23 B1..B3
    // (with [K][N] B as two transposing quarters each), 24-31 the scales.
    auto read_item = [&](auto kt, auto nst, int st) __attribute__((always_inline)) {
        constexpr int k = decltype(kt)::value;
        constexpr int NS = decltype(nst)::value;
        const uint32_t base = stg0 + (uint32_t)st * kStageBytes;
        if constexpr (k >= 2 && k < 18) {
            constexpr int i = (k - 2) / 2, h = (k - 2) % 2;
            w4_read_half<12 * NS + i, h, i * 16 * TBK>(base + (h ? a_rel1 : a_rel0));
        } else if constexpr (k < 24) {
            constexpr int j = k < 2 ? 0 : 1 + (k - 18) / 2;
            constexpr int h = k < 2 ? k : (k - 18) % 2;
            constexpr int F = 12 * NS + 8 + j;
            if constexpr (B_KN) {
                w4_read_quarter<F, 2 * h, (2 * h) * 8 * TBN>(base + kn_rel[j]);
                w4_read_quarter<F, 2 * h + 1, (2 * h + 1) * 8 * TBN>(base + kn_rel[j]);
            } else {
                w4_read_half<F, h, j * 16 * TBK>(base + (h ? b_rel1 : b_rel0));
            }
        } else {
            constexpr int i = k - 24;
            if constexpr (P2) {
                scl[NS].e[i] = w4_ds8<i * 64>(sa_rel + (uint32_t)(st * TBM * 4) + rsel);
                if constexpr (SB_MODE == SB_BLOCK && i == 0) scl[NS].eb[0] = w4_ds8<0>(sb_rel + (uint32_t)(st * 16) + bsel);
                if constexpr (SB_MODE == SB_ROW && i < NNI)
                    scl[NS].eb[i] = w4_ds8<i * 64>(sbp_rel + (uint32_t)(st * TBN * 4) + rsel);
            } else {
            if constexpr (SA_MODE == SA_ROW) scl[NS].sa[i] = w4_ds32<i * 64>(sa_rel + (uint32_t)(st * TBM * 4));
            if constexpr (SB_MODE == SB_BLOCK && i == 0) scl[NS].sb = w4_ds32<0>(sb_rel + (uint32_t)(st * 16));
            if constexpr (SB_MODE == SB_ROW && (i & 1) == 0)
                scl[NS].sc[i / 2] = w4_ds128<(i / 2) * 64>(sb_rel + (uint32_t)(st * TBN * 4));
            }
        }
    };
    // the closing wait of a chunk's reads; it names the scale registers so
    // that nothing reads them earlier
    auto reads_done = [&](auto nst) __attribute__((always_inline)) {
        constexpr int NS = decltype(nst)::value;
        W4Scales<SB_MODE>& s = scl[NS];
        if constexpr (P2) {
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(s.e[0]), "+v"(s.e[1]), "+v"(s.e[2]), "+v"(s.e[3]), "+v"(s.e[4]),
                           "+v"(s.e[5]), "+v"(s.e[6]), "+v"(s.e[7]), "+v"(s.eb[0])
                         :
                         : "memory");
            if constexpr (SB_MODE == SB_ROW) asm volatile("" : "+v"(s.eb[1]), "+v"(s.eb[2]), "+v"(s.eb[3]));
            return;
        }
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(s.sa[0]), "+v"(s.sa[1]), "+v"(s.sa[2]), "+v"(s.sa[3]), "+v"(s.sa[4]),
                       "+v"(s.sa[5]), "+v"(s.sa[6]), "+v"(s.sa[7]), "+v"(s.sb)
                     :
                     : "memory");
        if constexpr (SB_MODE == SB_ROW)
            asm volatile("" : "+v"(s.sc[0]), "+v"(s.sc[1]), "+v"(s.sc[2]), "+v"(s.sc[3]));
    };

    v4f acc[PMI][NNI];
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < PMI; ++i)
#pragma unroll
        for (int j = 0; j < NNI; ++j) acc[i][j] = zero;
    v4f P[4] = {zero, zero, zero, zero};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int i = 0; i < PMI; ++i) {
            scl[s].sa[i] = scl[s].comb[i] = 0.0f;
            scl[s].e[i] = 0;
        }
#pragma unroll
        for (int j = 0; j < (SB_MODE == SB_ROW ? NNI : 1); ++j) scl[s].eb[j] = 0;
        scl[s].sb = 0.0f;
#pragma unroll
        for (int j = 0; j < (SB_MODE == SB_ROW ? NNI : 1); ++j) scl[s].sc[j] = zero;
    }

    // scale FMAs of 16 x 16 block v (MFMA order: j = v / 8, i = v % 8) from
    // partial slot v & 3 with the scales of set S
    auto block_fma = [&](auto vt, auto st_) __attribute__((always_inline)) {
        constexpr int v = decltype(vt)::value;
        constexpr int S = decltype(st_)::value;
        constexpr int i = v % PMI, j = v / PMI;
        const v4f pp = P[v & 3];
        if constexpr (SB_MODE == SB_ROW) {
            const float ra = SA_MODE == SA_ROW ? scl[S].sa[i] : sa_t;
            float t[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) w4_mul(t[r], ra, scl[S].sc[j][r]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float a = acc[i][j][r];
                w4_fmac(a, pp[r], t[r]);
                acc[i][j][r] = a;
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float a = acc[i][j][r];
                w4_fmac(a, pp[r], scl[S].comb[i]);
                acc[i][j][r] = a;
            }
        }
    };

    // ---- output of a finished tile ----
    int c_ord = 0;
    Tile ct = tile_at(0);
    // rows stored: [0, M), or [0, off[G]) for groups of rows
    const int64_t m_end = GMODE == 1 ? min(M, (int64_t)__builtin_amdgcn_readfirstlane(goff[p.G])) : M;
    auto store_tile = [&]() __attribute__((always_inline)) {
        const int64_t cm0 = ct.m0, cn0 = ct.n0;
        // the output block of the tile's group (groups of K)
        void* const cbase = GMODE == 2 ? (void*)(reinterpret_cast<float*>(p.c) + (int64_t)ct.e * p.c_group_stride)
                                       : p.c;
        if constexpr (OUT == OUT_E4M3) {
            // The output's 1x128 tiles along N: a tile is the 64 columns of
            // this wave and those of wave wq ^ 1 (same rows).  Columns past N
            // are left out of the amax.
            float mx[PMI];
            const int64_t ncol0 = cn0 + 64 * wq + 4 * kgrp;
            if (cn0 + 64 * wq + 64 <= N) {
                // all 64 columns inside: |x| maxima three operands at a time
#pragma unroll
                for (int i = 0; i < PMI; ++i) {
                    float v = 0.0f;
#pragma unroll
                    for (int j = 0; j < NNI; ++j) {
                        v = w4_max3_abs(v, acc[i][j][0], acc[i][j][1]);
                        v = w4_max3_abs(v, acc[i][j][2], acc[i][j][3]);
                    }
                    mx[i] = v;
                }
            } else {
#pragma unroll
                for (int i = 0; i < PMI; ++i) {
                    float v = 0.0f;
#pragma unroll
                    for (int j = 0; j < NNI; ++j)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (ncol0 + 16 * j + r < N) v = fmaxf(v, fabsf(acc[i][j][r]));
                    mx[i] = v;
                }
            }
            // over the row's four lanes: each swap leaves a lane its own
            // value and its partner's (in either order), so the max of the
            // pair needs no select (maxima of non-negative floats compared
            // as their bit patterns)
#pragma unroll
            for (int i = 0; i < PMI; ++i) {
                const uint32_t b = __float_as_uint(mx[i]);
                const auto h = __builtin_amdgcn_permlane32_swap(b, b, false, false);
                const uint32_t v = h[0] > h[1] ? h[0] : h[1];
                const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
                mx[i] = __uint_as_float(r[0] > r[1] ? r[0] : r[1]);
                if (kgrp == 0) RowMax[wq][16 * i + lrow] = mx[i];
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < PMI; ++i) {
                const float other = RowMax[wq ^ 1][16 * i + lrow];
                const TileScale ts = make_scale(fmaxf(mx[i], other));
                uint32_t code[NNI];
                float v[8];
#pragma unroll
                for (int jp = 0; jp < NNI / 2; ++jp) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        v[r] = acc[i][2 * jp][r];
                        v[4 + r] = acc[i][2 * jp + 1][r];
                    }
                    quant8(v, ts, code[2 * jp], code[2 * jp + 1]);
                }
                const int64_t m = cm0 + 16 * i + lrow;
                uint8_t* qrow = reinterpret_cast<uint8_t*>(cbase) + m * p.ldc;
                if (cn0 + 64 * wq + 64 <= N) {
                    // one 16-byte store per lane: the four lanes of a row
                    // (kgrp L holds the codes of columns 16j + 4L .. + 3,
                    // j = 0..3) transpose their 4 x 4 dwords with the
                    // half-wave and row swaps (no lane selects): after
                    // swap 1 (lanes 0-31 <-> 32-63) lane L holds blocks 2h and
                    // 2h + 1 (h = L >> 1), each as the dwords of lanes
                    // L & 1 and (L & 1) + 2; after swap 2 (16-lane rows
                    // 0 <-> 1, 2 <-> 3) it holds block L from lanes 0..3 in
                    // order, i.e. columns 16L .. 16L + 15
                    const auto s02 = __builtin_amdgcn_permlane32_swap(code[0], code[2], false, false);
                    const auto s13 = __builtin_amdgcn_permlane32_swap(code[1], code[3], false, false);
                    const auto w0 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
                    const auto w1 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
                    if (m < m_end)
                        *reinterpret_cast<uint4*>(qrow + cn0 + 64 * wq + 16 * kgrp) =
                            make_uint4(w0[0], w0[1], w1[0], w1[1]);
                } else if (m < m_end) {
#pragma unroll
                for (int j = 0; j < NNI; ++j) {
                    const int64_t n = ncol0 + 16 * j;
                    if (n + 3 < N) {
                        *reinterpret_cast<uint32_t*>(qrow + n) = code[j];
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (n + r < N) qrow[n + r] = (uint8_t)(code[j] >> (8 * r));
                    }
                }
                }
                const int64_t n_tile = cn0 + 64 * wq;
                if (m < m_end && kgrp == 0 && (wq & 1) == 0 && n_tile < N) p.cs[m * p.ldcs + n_tile / 128] = ts.s;
            }
            return;
        }
        if constexpr (OUT == OUT_BF16) {
            if (cn0 + 64 * wq + 64 <= N) {
                // 16-byte stores: for each pair of 16-column blocks (2p, 2p+1)
                // the four lanes of a row (kgrp k, four columns of each block)
                // exchange halves with the half-wave and row swaps (no lane
                // selects), after which lane k holds columns 32p + 8k .. + 7:
                // half the store instructions of one 8-byte store per block
#pragma unroll
                for (int i = 0; i < PMI; ++i) {
                    const int64_t m = cm0 + 16 * i + lrow;
#pragma unroll
                    for (int pq = 0; pq < NNI / 2; ++pq) {
                        const v4f A = acc[i][2 * pq], B = acc[i][2 * pq + 1];
                        // swap 1 (lanes 0-31 <-> 32-63): lanes of kgrp 0, 1
                        // keep block 2p, kgrp 2, 3 block 2p + 1; each then
                        // holds that block's columns 4(k & 1) (first) and
                        // 4(k & 1) + 8 (second), two per dword
                        const auto s0 = __builtin_amdgcn_permlane32_swap(bf16x2_rne(A[0], A[1]),
                                                                         bf16x2_rne(B[0], B[1]), false, false);
                        const auto s1 = __builtin_amdgcn_permlane32_swap(bf16x2_rne(A[2], A[3]),
                                                                         bf16x2_rne(B[2], B[3]), false, false);
                        // swap 2 (16-lane rows 0 <-> 1, 2 <-> 3): even k end
                        // with columns 0-3 and 4-7 of the block half they
                        // keep, odd k with columns 8-11 and 12-15
                        const auto t0 = __builtin_amdgcn_permlane16_swap(s0[0], s0[1], false, false);
                        const auto t1 = __builtin_amdgcn_permlane16_swap(s1[0], s1[1], false, false);
                        if (m >= m_end) continue;
                        const uint4 w = make_uint4(t0[0], t1[0], t0[1], t1[1]);
                        const int64_t n = cn0 + 64 * wq + 32 * pq + 8 * kgrp;
                        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(cbase) + m * p.ldc + n) = w;
                    }
                }
                return;
            }
        }
        if constexpr (OUT == OUT_F32) {
            if (cn0 + 64 * wq + 64 <= N) {
                // whole 128-byte lines per store instruction: for each pair
                // of 16-column blocks (2p, 2p+1) lanes l and l ^ 8 (rows r and
                // r ^ 8) swap one block (DPP rotate by 8 within each row of
                // 16 lanes); the first store then covers rows 0-7 of the pair's
                // 32 columns, the second rows 8-15
                const bool top = lrow < 8;
#pragma unroll
                for (int i = 0; i < PMI; ++i) {
#pragma unroll
                    for (int pq = 0; pq < NNI / 2; ++pq) {
                        const v4f A = acc[i][2 * pq], B = acc[i][2 * pq + 1];
                        v4f R;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            R[r] = __int_as_float(__builtin_amdgcn_update_dpp(
                                0, __float_as_int(top ? B[r] : A[r]), 0x128, 0xF, 0xF, false));
                        // store 1: rows 16i .. 16i+7; store 2: rows 16i+8 .. 16i+15
                        const int64_t m1 = cm0 + 16 * i + (lrow & 7), m2 = m1 + 8;
                        // top lanes store block 2p, the others block 2p + 1
                        const int64_t n = cn0 + 64 * wq + 32 * pq + 4 * kgrp + (top ? 0 : 16);
                        const v4f w1 = top ? A : R, w2 = top ? R : B;
                        float* const c0 = reinterpret_cast<float*>(cbase);
                        if (m1 < m_end) {
                            if constexpr (GMODE == 2) __builtin_nontemporal_store(w1, reinterpret_cast<v4f*>(c0 + m1 * p.ldc + n));
                            else *reinterpret_cast<v4f*>(c0 + m1 * p.ldc + n) = w1;
                        }
                        if (m2 < m_end) {
                            if constexpr (GMODE == 2) __builtin_nontemporal_store(w2, reinterpret_cast<v4f*>(c0 + m2 * p.ldc + n));
                            else *reinterpret_cast<v4f*>(c0 + m2 * p.ldc + n) = w2;
                        }
                    }
                }
                return;
            }
        }
#pragma unroll
        for (int i = 0; i < PMI; ++i) {
            const int64_t m = cm0 + 16 * i + lrow;
            if (m >= m_end) continue;
#pragma unroll
            for (int j = 0; j < NNI; ++j) {
                const int64_t n = cn0 + 64 * wq + 16 * j + 4 * kgrp;
                const v4f v = acc[i][j];
                if (n + 3 < N) {
                    if (OUT == OUT_BF16) {
                        const uint32_t lo = bf16x2_rne(v[0], v[1]);
                        const uint32_t hi = bf16x2_rne(v[2], v[3]);
                        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(cbase) + m * p.ldc + n) = make_uint2(lo, hi);
                    } else if (GMODE == 2) {
                        // the MoE weight gradient streams its fp32 output
                        // (1.6 GB for 128 experts of 1536 x 2048) past the
                        // caches, which keep the operands (measured 19-33%
                        // faster than cached stores; no gain on dense outputs)
                        __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(reinterpret_cast<float*>(cbase) + m * p.ldc + n));
                    } else {
                        *reinterpret_cast<v4f*>(reinterpret_cast<float*>(cbase) + m * p.ldc + n) = v;
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (n + r < N) {
                            if (OUT == OUT_BF16)
                                reinterpret_cast<uint16_t*>(cbase)[m * p.ldc + n + r] = (uint16_t)bf16_rne(v[r]);
                            else
                                reinterpret_cast<float*>(cbase)[m * p.ldc + n + r] = v[r];
                        }
                    }
                }
            }
        }
    };

    // ---- prologue: chunks 0..2 to LDS, chunk 0 to registers ----
    for (int c = 0; c < 3; ++c) {
        w4_for<0, ND>([&](auto dt) __attribute__((always_inline)) { load_item(dt, c); });
        load_advance();
    }
    w4_wait_vm<2 * ND>();
    __builtin_amdgcn_s_barrier();
    if constexpr (P2) read_cursor_set();
    w4_for<0, 32>([&](auto kt) __attribute__((always_inline)) { read_item(kt, std::integral_constant<int, 0>{}, 0); });
    reads_done(std::integral_constant<int, 0>{});
    if constexpr (P2) read_advance();

    // ---- the chunk stream ----
    int ck = 0;
    int st_w = 0;          // stage of chunk g (takes chunk g + 3)
    auto iteration = [&](auto s_tag) __attribute__((always_inline)) {
        constexpr int S = decltype(s_tag)::value;
        constexpr int NS = 1 - S;
        // own loads of chunk g + 1 have landed; after the barrier every
        // wave's have, and every wave is done reading chunk g's stage
        w4_wait_vm<ND>();
        __builtin_amdgcn_s_barrier();
        if constexpr (!P2 && SB_MODE != SB_ROW) {
            const float sbv = SB_MODE == SB_BLOCK ? scl[S].sb : SB_MODE == SB_TENSOR ? sb_t : 1.0f;
#pragma unroll
            for (int i = 0; i < PMI; ++i) scl[S].comb[i] = (SA_MODE == SA_ROW ? scl[S].sa[i] : sa_t) * sbv;
            // formed here, once per chunk, not next to each use
            asm volatile("" : "+v"(scl[S].comb[0]), "+v"(scl[S].comb[1]), "+v"(scl[S].comb[2]), "+v"(scl[S].comb[3]),
                              "+v"(scl[S].comb[4]), "+v"(scl[S].comb[5]), "+v"(scl[S].comb[6]), "+v"(scl[S].comb[7]));
        }
        const int st_r = st_w == 2 ? 0 : st_w + 1;
        w4_for<0, 32>([&](auto ut) __attribute__((always_inline)) {
            constexpr int u = decltype(ut)::value;
            if constexpr (P2)
                w4_mfma_scaled<12 * S + 8 + u / PMI, 12 * S + u % PMI>(
                    acc[u % PMI][u / PMI], scl[S].eb[SB_MODE == SB_ROW ? u / PMI : 0], scl[S].e[u % PMI]);
            else
                w4_mfma<12 * S + 8 + u / PMI, 12 * S + u % PMI>(P[u & 3]);
            read_item(ut, std::integral_constant<int, NS>{}, st_r);
            if constexpr (u >= 4 && (u - 4) % 2 == 0 && (u - 4) / 2 < ND)
                load_item(std::integral_constant<int, (u - 4) / 2>{}, st_w);
            // blocks 29..31 of the previous chunk (zero partials after a
            // tile's last chunk, whose blocks were scaled before its output)
            if constexpr (!P2) {
                if constexpr (u >= 3) block_fma(std::integral_constant<int, u - 3>{}, std::integral_constant<int, S>{});
                else block_fma(std::integral_constant<int, 29 + u>{}, std::integral_constant<int, NS>{});
            }
        });
        load_advance();
        reads_done(std::integral_constant<int, NS>{});
        if constexpr (P2) read_advance();
        if (ck == ct.kbn - 1 && P2) {
            // the output reads accumulators the last MFMAs wrote (an 8-pass
            // MFMA result needs 11 wait states before a vector read)
            asm volatile("s_nop 7\n s_nop 7" ::: "memory");
            store_tile();
#pragma unroll
            for (int i = 0; i < PMI; ++i)
#pragma unroll
                for (int j = 0; j < NNI; ++j) acc[i][j] = zero;
            if (++c_ord < my_tiles) ct = tile_at(c_ord);
            ck = 0;
        } else if (ck == ct.kbn - 1) {
            // last chunk of the tile: blocks 29..31 (their MFMAs are more
            // than 12 instructions back after this padding), then the output
            asm volatile("s_nop 7" ::: "memory");
            block_fma(std::integral_constant<int, 29>{}, std::integral_constant<int, S>{});
            block_fma(std::integral_constant<int, 30>{}, std::integral_constant<int, S>{});
            block_fma(std::integral_constant<int, 31>{}, std::integral_constant<int, S>{});
            P[1] = zero;
            P[2] = zero;
            P[3] = zero;
            store_tile();
#pragma unroll
            for (int i = 0; i < PMI; ++i)
#pragma unroll
                for (int j = 0; j < NNI; ++j) acc[i][j] = zero;
            if (++c_ord < my_tiles) ct = tile_at(c_ord);
            ck = 0;
        } else {
            ++ck;
        }
        st_w = st_r;
    };
    for (;;) {
        iteration(std::integral_constant<int, 0>{});
        if (c_ord == my_tiles) break;
        iteration(std::integral_constant<int, 1>{});
        if (c_ord == my_tiles) break;
    }
    w4_wait_vm<0>();
}

template <int SA_MODE, int SB_MODE, int GMODE = 0, bool B_KN = false, bool P2 = false>
static void w4_launch_out(const GemmArgs& g, int out, hipStream_t st)
{
    GemmArgs a = g;
    a.tiles_m = (int)((g.M + TBM - 1) / TBM);
    a.tiles_n = (int)((g.N + TBN - 1) / TBN);
    // groups of K: every workgroup derives its tiles from the offsets
    const int64_t tiles = GMODE == 2 ? g.num_cus : (int64_t)a.tiles_m * a.tiles_n;
    dim3 grid((uint32_t)(tiles < g.num_cus ? tiles : g.num_cus));
    if (out == OUT_BF16) {
        if constexpr (GMODE != 2)
            hipLaunchKernelGGL((gemm_w4_kernel<SA_MODE, SB_MODE, OUT_BF16, GMODE, B_KN, P2>), grid, dim3(kW4Threads), 0, st, a);
    } else if (out == OUT_F32) {
        hipLaunchKernelGGL((gemm_w4_kernel<SA_MODE, SB_MODE, OUT_F32, GMODE, B_KN, P2>), grid, dim3(kW4Threads), 0, st, a);
    } else if constexpr (SB_MODE != SB_ROW && (GMODE == 0 || (GMODE == 1 && !B_KN)) && !P2) {
        hipLaunchKernelGGL((gemm_w4_kernel<SA_MODE, SB_MODE, OUT_E4M3, GMODE, B_KN>), grid, dim3(kW4Threads), 0, st, a);
    }
}

// Every dense call with K a multiple of 128: B stored [N][K] (forward,
// wgrad) or read as stored [K][N] (dgrad; not with row-scaled B).  Returns
// false otherwise.
bool launch_gemm_w4(const GemmArgs& g, int sa_mode, int sb_mode, bool b_kn, int out, hipStream_t st)
{
    if (g.K <= 0 || g.K % 128 != 0) return false;
    if (out == OUT_E4M3 && sb_mode == SB_ROW) return false;
    if (b_kn) {
        if (sb_mode == SB_ROW) return false;
        if (sa_mode == SA_ROW) {
            if (sb_mode == SB_BLOCK) w4_launch_out<SA_ROW, SB_BLOCK, 0, true>(g, out, st);
            else w4_launch_out<SA_ROW, SB_TENSOR, 0, true>(g, out, st);
        } else {
            if (sb_mode == SB_BLOCK) w4_launch_out<SA_TENSOR, SB_BLOCK, 0, true>(g, out, st);
            else w4_launch_out<SA_TENSOR, SB_TENSOR, 0, true>(g, out, st);
        }
        return true;
    }
    if (sa_mode == SA_ROW) {
        if (sb_mode == SB_BLOCK) w4_launch_out<SA_ROW, SB_BLOCK>(g, out, st);
        else if (sb_mode == SB_ROW) w4_launch_out<SA_ROW, SB_ROW>(g, out, st);
        else w4_launch_out<SA_ROW, SB_TENSOR>(g, out, st);
    } else {
        if (sb_mode == SB_BLOCK) w4_launch_out<SA_TENSOR, SB_BLOCK>(g, out, st);
        else if (sb_mode == SB_ROW) w4_launch_out<SA_TENSOR, SB_ROW>(g, out, st);
        else w4_launch_out<SA_TENSOR, SB_TENSOR>(g, out, st);
    }
    return true;
}

// Dense calls with power-of-two scales (E8M0 bytes; row-scaled A, block-
// scaled B [N][K] or [K][N], or row-scaled [N][K] B) and K a multiple of
// 128; false otherwise.
bool launch_gemm_w4_e8m0(const GemmArgs& g, int sb_mode, bool b_kn, bool out_bf16, hipStream_t st)
{
    if (g.K <= 0 || g.K % 128 != 0) return false;
    if (b_kn && sb_mode != SB_BLOCK) return false;
    const int out = out_bf16 ? OUT_BF16 : OUT_F32;
    if (b_kn) w4_launch_out<SA_ROW, SB_BLOCK, 0, true, true>(g, out, st);
    else if (sb_mode == SB_BLOCK) w4_launch_out<SA_ROW, SB_BLOCK, 0, false, true>(g, out, st);
    else w4_launch_out<SA_ROW, SB_ROW, 0, false, true>(g, out, st);
    return true;
}

// The MoE forward (groups of rows, expert B stored [N][K]) and dgrad (expert
// weight read as stored, [K][N]) with K a multiple of 128; false if it does
// not cover the call.  Every operand must span less than 2 GiB (32-bit buffer
// offsets; A's loads run up to a tile past M, B's up to a chunk past K).
bool launch_grouped_gemm_w4(const GemmArgs& g, bool out_bf16, bool b_kn, hipStream_t st)
{
    const int64_t lim = (int64_t)1 << 31;
    if (g.K <= 0 || g.K % 128 != 0 || g.G < 1 || g.G > kMaxLdsGroups) return false;
    const int64_t b_span = b_kn ? (g.K + TBK) * g.ldb : g.N * g.ldb;
    if ((g.M + TBM) * g.lda >= lim || b_span >= lim || (g.M + TBM) * g.ldsa * 4 >= lim ||
        g.sb_group_stride * 4 >= lim)
        return false;
    const int out = out_bf16 ? OUT_BF16 : OUT_F32;
    if (b_kn) w4_launch_out<SA_ROW, SB_BLOCK, 1, true>(g, out, st);
    else w4_launch_out<SA_ROW, SB_BLOCK, 1>(g, out, st);
    return true;
}

// The MoE forward stored quantized (E4M3 codes in p.c, 1x128 scales in
// p.cs); K a multiple of 128, the operand limits of launch_grouped_gemm_w4;
// false otherwise.
bool launch_grouped_gemm_w4_e4m3(const GemmArgs& g, hipStream_t st)
{
    const int64_t lim = (int64_t)1 << 31;
    if (g.K <= 0 || g.K % 128 != 0 || g.G < 1 || g.G > kMaxLdsGroups) return false;
    if ((g.M + TBM) * g.lda >= lim || g.N * g.ldb >= lim || (g.M + TBM) * g.ldsa * 4 >= lim ||
        g.sb_group_stride * 4 >= lim)
        return false;
    w4_launch_out<SA_ROW, SB_BLOCK, 1>(g, OUT_E4M3, st);
    return true;
}

// The MoE weight gradient (groups of K over the token axis, row-scaled
// operands, fp32 out); false if it does not cover the call.  The token
// extent M_pad (the GEMM's K) is a multiple of 128 by contract; with
// M_pad = 0 every group is empty and the kernel only stores zeros.
bool launch_grouped_wgrad_w4(const GemmArgs& g, hipStream_t st)
{
    const int64_t lim = (int64_t)1 << 31;
    if (g.K < 0 || g.K % 128 != 0 || g.G < 1 || g.G > kMaxLdsGroups) return false;
    if ((g.M + TBM) * g.lda >= lim || (g.N + TBN) * g.ldb >= lim || (g.M + TBM) * g.ldsa * 4 >= lim ||
        (g.N + TBN) * g.ldsb * 4 >= lim || (int64_t)g.G * g.c_group_stride * 4 >= ((int64_t)1 << 62))
        return false;
    w4_launch_out<SA_ROW, SB_ROW, 2>(g, OUT_F32, st);
    return true;
}

}  // namespace fp8q
