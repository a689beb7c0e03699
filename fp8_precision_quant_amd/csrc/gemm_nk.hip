// Block-scaled FP8 GEMM on gfx950, eight-wave form.  The four-wave kernel
// (gemm_w4.hip) runs every dense and grouped call whose K (the contraction
// axis) is a multiple of 128, with fp32 or power-of-two scales; this kernel
// takes the calls with a ragged last chunk (K % 128 != 0), whose fragment
// bytes at or past K it zeroes in registers (a code past K may be anything):
// the forward y = x W^T (B = W stored [N][K]), dgrad dx = dy W (B = W read as
// stored, [K][N], no transposed copy: Ling 2.0 FP8 blog, "FP8 on-demand
// transpose weight"), the weight gradient dW = dy^T x on transposed
// re-quantized operands (row-scaled B), per-tensor scaling, E8M0 scales, and
// the grouped (MoE) forward and dgrad.
//
//   C[m][n] = sum_kb SA(m,kb) * SB(n,kb) * sum_{k in chunk kb} dec(A[m][k]) * dec(B[n][k])
//
// (FP8 Linear with an FP32 accumulator: Ling 2.0 FP8 blog, "where does the
// worry come from" and "where is error introduced"; tile scales: same blog,
// "fine-grained quantization"; 128x128 weight blocks: "FP8-RL" article, 一.)
//
// gfx950 mapping:
//  * persistent workgroups (one per CU) with a tile of 128 (M) x 256 (N);
//    K chunk 128 = one scale chunk = one v_mfma_f32_16x16x128_f8f6f4 per
//    16x16 block, which gives the chunk's fp32 partial; VALU FMAs scale it
//    into the fp32 accumulator, each behind the next block's MFMA;
//  * 8 waves, each owning all 128 rows of 64 columns (8 A and 4 B fragments,
//    32 MFMAs per chunk); the two groups of four waves (one wave of each per
//    SIMD) take alternate K chunks in ping-pong phases, so one wave of every
//    SIMD runs MFMAs from registers while its partner loads and reads the
//    next chunk; the two partial tiles are added through LDS at the end;
//  * operands and per-chunk scales go global -> LDS with buffer loads that
//    write LDS directly (no VGPR staging), through a ring of 3 LDS stages of
//    48 KB, two chunks ahead.  Buffer resources bound every load to its
//    operand;
//  * 16-byte LDS slots are XOR-swizzled per row so fragment reads are free
//    of bank conflicts; a [K][N] operand is staged as stored (K rows of 256
//    bytes) and read with ds_read_b64_tr_b8, which returns each lane 8
//    consecutive K values of its own column -- the MFMA operand layout;
//  * tile order: workgroups are dealt to the 8 XCDs round-robin, so each XCD
//    gets a contiguous range of tiles, walked in groups of 16 M-tiles so
//    neighbouring workgroups share A and B panels in that XCD's L2.
#include <type_traits>

#include "fp8q_device.h"
#include "fp8q_internal.h"
#include "gemm_common.h"
#include "gemm_lds.h"

namespace fp8q {

namespace {

constexpr int kThreads = 512;

}  // namespace


// ---------------------------------------------------------------------------
// The kernel.  Each wave owns all 128 rows of its 64 columns (32 MFMAs per
// chunk from 8 A and 4 B fragments: 768 LDS bytes per MFMA, against 1024
// for a 64 x 64 wave tile), and the two wave groups (one wave of each per
// SIMD) take alternate K chunks.  Phase q (one barrier each): group q % 2
// loads chunk q+2 and reads chunk q from LDS into registers while the other
// group runs the MFMAs of chunk q-1 from registers, so each SIMD has one
// wave on the matrix core while its partner waits for memory.  A group
// loads exactly the chunks it reads, two phases ahead, so waiting for a
// chunk is vmcnt(0) in its waves.  With [N][K] B each wave loads the B rows
// of its own columns, so it reads those right after its compute phase and
// only the shared A rows after the barrier.
// At the end of a tile each group holds the sum over its chunks; the halves
// are added through LDS (the ring is idle by then), each group finishing and
// storing 64 of the 128 rows.
struct Frags {
    v8i a[PMI], b[NNI];
    float s[PMI];    // combined scale of the lane's row in block i for the chunk
    float sbk;       // SB of the wave's 128-column block (block-scaled B)
    // power-of-two scales: E8M0 bytes of the lane's A row in block i, of its
    // B row in block j (row-scaled B), of the wave's column block
    int e[PMI], eb[NNI], ebk;
};

template <int OFF>
__device__ __forceinline__ void ds_write128(uint32_t addr, v4f v)
{
    asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(addr), "v"(v), "i"(OFF) : "memory");
}

// max(m, |a|, |b|) for m >= 0 and finite a, b (exact; no NaN quieting)
__device__ __forceinline__ float nk_max3_abs(float m, float a, float b)
{
    float d;
    asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(d) : "v"(m), "v"(a), "v"(b));
    return d;
}

template <int I>
__device__ __forceinline__ v8i frag_nk(uint32_t r0, uint32_t r1)
{
    return cat(ds128<I * 16 * TBK>(r0), ds128<I * 16 * TBK>(r1));
}

// the 4 column scales of a lane in 16-column block j (row-scaled B)
__device__ __forceinline__ v4f col_scales(uint32_t a, int j)
{
    switch (j) {
    case 0: return (v4f)ds128<0>(a);
    case 1: return (v4f)ds128<64>(a);
    case 2: return (v4f)ds128<128>(a);
    default: return (v4f)ds128<192>(a);
    }
}

// GMODE: 0 dense; 1 groups of A rows (MoE forward and dgrad: the row tile's
// group selects the expert's B and B scales).  (The MoE weight gradient,
// groups of K, runs on gemm_w4.hip.)
// P2: power-of-two scales given as E8M0 bytes (p.sa / p.sb point at bytes),
// applied by the scaled MFMA itself: the chunk's product is accumulated in
// place, with no partial sum and no scale FMA.  A scale grid's rows are read
// as 4-byte words, each holding the bytes of four consecutive chunks.
template <int SA_MODE, int SB_MODE, bool B_KN, int OUT, int GMODE, bool P2>
__global__ __launch_bounds__(kThreads) void gemm_nk_kernel(GemmArgs p)
{
    constexpr int kSbStages = SB_MODE == SB_ROW ? 4 : kStages;
    static_assert(!(B_KN && SB_MODE == SB_ROW), "row-scaled B is [N][K] only");
    static_assert(!P2 || (GMODE == 0 && SA_MODE == SA_ROW && SB_MODE != SB_TENSOR && OUT != OUT_E4M3),
                  "power-of-two scales: dense, row-scaled A, block- or row-scaled B, fp32/bf16 out");
    static_assert(GMODE == 0 || GMODE == 1, "dense or groups of rows");
    __shared__ int32_t goff[GMODE != 0 ? kMaxLdsGroups + 1 : 1];
    __shared__ __attribute__((aligned(16))) uint8_t Stg[kStages][kStageBytes];
    __shared__ __attribute__((aligned(16))) float SAs[kStages][TBM];
    // B scales of a chunk: its two 128-column blocks (block-scaled B), or its
    // 256 column scales (row-scaled B), which the computing group reads one
    // phase after the chunk's operands, hence a ring one deeper
    __shared__ __attribute__((aligned(16))) float SBs[kSbStages][SB_MODE == SB_ROW ? TBN : 64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;   // chunk parity of this wave
    const int wq = wave & 3;     // wave within its group: columns [64 wq, 64 wq + 64)

    // Persistent workgroups.  Workgroups are dealt to the 8 XCDs
    // round-robin; XCD x owns a contiguous range of tile ids, walked by its
    // workgroups in lockstep (tile id = start + local + i * count), in
    // groups of kGroupM M-tiles so that concurrently running tiles share A
    // and B panels in that XCD's L2.
    const int T = p.tiles_m * p.tiles_n;
    const int xcd = blockIdx.x & 7;
    const int local = blockIdx.x >> 3;
    const int G = gridDim.x;
    const int nwg = (G >> 3) + (xcd < (G & 7) ? 1 : 0);
    const int range_start = xcd * (T >> 3) + min(xcd, T & 7);
    const int range_len = (T >> 3) + (xcd < (T & 7) ? 1 : 0);
    const int span = kGroupM * p.tiles_n;
    const int tiles_here = range_len;
    auto tile_origin = [&](int i, int64_t& tm0, int64_t& tn0) {
        const int pid = range_start + i;
        const int group = pid / span;
        const int first_m = group * kGroupM;
        const int gsz = min(p.tiles_m - first_m, kGroupM);
        const int idx = pid - group * span;
        tm0 = (int64_t)(first_m + idx % gsz) * TBM;
        tn0 = (int64_t)(idx / gsz) * TBN;
    };
    int ti = local;
    if (ti >= tiles_here) return;
    if (GMODE != 0) {
        for (int i = tid; i <= p.G; i += kThreads) goff[i] = p.offsets[i];
        __syncthreads();
    }
    int64_t m0, n0;
    tile_origin(ti, m0, n0);

    const int64_t M = p.M, N = p.N, K = p.K;
    const int KB = p.KB;                  // chunks of the K loop
    const int k_tail = (int)(K - (int64_t)(KB - 1) * TBK);

    const int64_t ext_a = (M - 1) * p.lda + ((K + 15) & ~(int64_t)15);
    const int64_t ext_b = B_KN ? (K - 1) * p.ldb + ((N + 15) & ~(int64_t)15)
                               : (N - 1) * p.ldb + ((K + 15) & ~(int64_t)15);
    const __amdgpu_buffer_rsrc_t ra = rsrc(p.a, ext_a);
    __amdgpu_buffer_rsrc_t rb = rsrc(p.b, ext_b);
    int grp_e = 0;
    bool tile_live = true;
    // groups of rows: the tile's group e (off[e] <= m0 < off[e+1]) selects
    // expert e's B and block scales; tiles at or past off[G] are computed
    // from group G-1 but not stored.  (values read from LDS are made
    // wave-uniform explicitly, so that addresses derived from them stay
    // scalar)
    auto set_group = [&](int64_t& tm0) {
        if (GMODE == 1) {
            int lo = 0, hi = p.G - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if ((int64_t)goff[mid] <= tm0) lo = mid; else hi = mid - 1;
            }
            grp_e = __builtin_amdgcn_readfirstlane(lo);
            tile_live = tm0 < (int64_t)__builtin_amdgcn_readfirstlane(goff[p.G]);
            rb = rsrc(p.b + (int64_t)grp_e * p.b_group_stride, ext_b);
        }
    };
    set_group(m0);

    // scale loads: waves 0-1 of a group the SA of the tile's 128 rows
    // (row-scaled A); wave 2 the block scales of the tile's two 128-column
    // blocks (block-scaled B), or every wave the scales of its 64 columns
    // (row-scaled B)
    const int64_t nblocks = (N + 127) / 128;
    const bool load_sa = SA_MODE == SA_ROW && wq < 2;
    const bool load_sb = SB_MODE == SB_ROW || (SB_MODE == SB_BLOCK && wq == 2);
    // (E8M0 grids: byte extents, each row's last word included)
    const int64_t kb_words = (KB + 3) & ~3, nb_words = (nblocks + 3) & ~3;
    const __amdgpu_buffer_rsrc_t rsa = rsrc(p.sa, SA_MODE != SA_ROW ? 4
                                                  : P2 ? (M - 1) * p.ldsa + kb_words
                                                       : ((M - 1) * p.ldsa + KB) * 4);
    auto sb_rsrc = [&]() {
        if (SB_MODE == SB_ROW) return rsrc(p.sb, P2 ? (N - 1) * p.ldsb + kb_words : ((N - 1) * p.ldsb + KB) * 4);
        if (SB_MODE == SB_BLOCK) {
            const float* sbg = p.sb + (GMODE == 1 ? (int64_t)grp_e * p.sb_group_stride : 0);
            if (P2) return rsrc(sbg, B_KN ? (int64_t)(KB - 1) * p.ldsb + nb_words : (nblocks - 1) * p.ldsb + kb_words);
            if (B_KN) return rsrc(sbg, ((int64_t)(KB - 1) * p.ldsb + nblocks) * 4);
            return rsrc(sbg, ((nblocks - 1) * p.ldsb + KB) * 4);
        }
        return rsrc(p.sb, 4);
    };
    __amdgpu_buffer_rsrc_t rsb = sb_rsrc();

    // Loads of chunk kb by this wave: A rows [32 wq, 32 wq + 32) (4 DMAs of
    // 8 rows), B rows [64 wq, 64 wq + 64) of [N][K] B (8 DMAs of 8 rows) or K
    // rows [32 wq, 32 wq + 32) of [K][N] B (8 DMAs of 4 rows), and its scale
    // words.  DMA t of an operand differs from DMA 0 by t row steps (a scalar
    // offset) and, for odd t, by the row's swizzle key (bit 0 of the 8-row
    // group index, resp. bit 2 of the [K][N] key): two per-lane offsets per
    // operand.  Rows past M or N are not clamped: lda and ldb are multiples
    // of 16 and at least K, so such rows start past the buffer resource's
    // bound and read as zero (they feed only outputs that are not stored);
    // scale rows past M and a missing second column block read as zero too.
    // (rebuilt from the lane id for each chunk, so that they do not occupy
    // registers through the compute phase)
    struct DmaOffs { uint32_t va[2], vb[2], vsa, vsb; };
    auto dma_offsets = [&]() {
        DmaOffs o;
        int l = lane;
        asm volatile("" : "+v"(l));
        const int ra_row = 32 * wq + (l >> 3);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            o.va[h] = (uint32_t)((m0 + ra_row) * p.lda) + 16u * (uint32_t)((l & 7) ^ (l >> 3) ^ h);
            if (B_KN) {
                const int r = 32 * wq + (l >> 4);
                const int key = (4 * h + (l >> 4)) ^ (8 * (wq & 1));
                o.vb[h] = (uint32_t)(r * p.ldb + n0) + 16u * (uint32_t)((l & 15) ^ key);
            } else {
                o.vb[h] = (uint32_t)((n0 + 64 * wq + (l >> 3)) * p.ldb) + 16u * (uint32_t)((l & 7) ^ (l >> 3) ^ h);
            }
        }
        constexpr int se = P2 ? 1 : 4;   // bytes per scale
        o.vsa = (uint32_t)((m0 + 64 * wq + l) * p.ldsa * se);
        if (SB_MODE == SB_ROW)
            o.vsb = (uint32_t)((n0 + 64 * wq + l) * p.ldsb * se);
        else if (P2 && B_KN)   // one word holds both column blocks (n0 / 128 is even)
            o.vsb = (uint32_t)((n0 / 128) & ~(int64_t)3);
        else
            o.vsb = (uint32_t)((n0 / 128 + (l < 1 ? l : 1)) * (B_KN ? 4 : p.ldsb * se));
        return o;
    };
    auto issue = [&](int kb) {
        const DmaOffs o = dma_offsets();
        const int st = kb % kStages;
        // per-chunk scalars, opaque so that the per-DMA sums below are formed
        // here rather than hoisted out of the loop into spilled registers
        uint32_t a_lds = lds_addr(&Stg[st][0]) + (uint32_t)(32 * wq * TBK);
        uint32_t b_lds = lds_addr(&Stg[st][kAStage]) + (uint32_t)(B_KN ? 32 * wq * TBN : 64 * wq * TBK);
        const uint32_t kg = (uint32_t)kb;
        uint32_t a_soff = kg * TBK, a_step = 8u * (uint32_t)p.lda;
        uint32_t b_soff = B_KN ? kg * TBK * (uint32_t)p.ldb : kg * TBK;
        uint32_t b_step = (B_KN ? 4u : 8u) * (uint32_t)p.ldb;
        asm volatile("" : "+s"(a_lds), "+s"(b_lds), "+s"(a_soff), "+s"(a_step), "+s"(b_soff), "+s"(b_step));
#pragma unroll
        for (int t = 0; t < 4; ++t) dma16_at(ra, a_lds + (uint32_t)(8 * t * TBK), o.va[t & 1], a_soff + t * a_step);
#pragma unroll
        for (int t = 0; t < 8; ++t)
            dma16_at(rb, b_lds + (uint32_t)(B_KN ? 4 * t * TBN : 8 * t * TBK), o.vb[t & 1], b_soff + t * b_step);
        const uint32_t s_soff = P2 ? (kg & ~3u) : kg * 4;   // the chunk's word of a scale row
        if (load_sa) dma4(rsa, &SAs[st][64 * wq], o.vsa, s_soff);
        if (SB_MODE == SB_ROW)
            dma4(rsb, &SBs[kb % kSbStages][64 * wq], o.vsb, s_soff);
        else if (load_sb)
            dma4(rsb, &SBs[st][0], o.vsb, B_KN ? kg * (uint32_t)p.ldsb * (P2 ? 1 : 4) : s_soff);
    };

    v4f acc[PMI][NNI];
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    const float sa_t = (SA_MODE == SA_TENSOR && KB > 0) ? p.sa[0] : 0.0f;
    const float sb_t = (SB_MODE == SB_TENSOR && KB > 0) ? p.sb[0] : 0.0f;

    // the LDS reads of one chunk (addresses rebuilt from the lane id)
    // B fragments of the chunk in stage st: the wave's own 64 columns.  For
    // [N][K] B those are exactly the B rows this wave loaded, so they may be
    // read as soon as its own loads have landed, right after the wave's
    // compute phase; that pays only where the compute phase is short (scaled
    // MFMAs, no scale FMAs).  Otherwise, and for [K][N] B (rows loaded
    // across all columns by every wave of the group), B is read after the
    // phase barrier like A.  (Per-wave s_memtime stamps, forward shape: the
    // compute phase with fp32 scales is ~1360 cycles and the early read
    // ~350 more, both on the phase's critical path.)  Which order wins was
    // measured per mode: the quantize-on-store output keeps the early read
    // (+19% without it), and the scaled-MFMA dgrad keeps issuing the loads
    // before the reads (+4% for it otherwise).
    constexpr bool kEarlyB = !B_KN && (P2 || OUT == OUT_E4M3);
    constexpr bool kReadsFirst = !(P2 && B_KN);
    // Wave priority between the two groups on a SIMD (each SIMD holds one
    // wave of each).  The instruction arbiter otherwise favours the older
    // waves (group 0), so group 1's read phase ran ~300 cycles longer than
    // group 0's.  With a uniform B scale the read phase is the longer one
    // and the reading wave is raised (forward -6%, dgrad -4%); with row
    // scales the two scale operations per output make the compute phase
    // the longer one and the computing wave is raised (wgrad -2%).  The
    // scaled-MFMA and quantize-on-store kernels measured no difference.
    constexpr int kPrio = (P2 || OUT == OUT_E4M3) ? 0 : (SB_MODE == SB_ROW ? 2 : 1);
    auto read_b = [&](int st, Frags& f) {
        int l = lane;
        asm volatile("" : "+v"(l));
        const int lrow = l & 15, kgrp = l >> 4;
        const uint32_t so = lds_addr(Stg) + (uint32_t)st * kStageBytes;
        if (B_KN) {
            // lane (kgrp, lrow) addresses K row 32 kgrp + lrow / 2 at column
            // 64 wq + 16 j + 8 (lrow & 1); fragment j is fragment 0 with the
            // 16-byte slot index xor j
            const int r = 32 * kgrp + (lrow >> 1);
            const uint32_t rel = (uint32_t)(r * TBN + (((4 * wq) ^ kn_key(r)) << 4) + 8 * (lrow & 1));
#pragma unroll
            for (int j = 0; j < NNI; ++j) {
                const uint32_t ad = so + kAStage + (rel ^ (uint32_t)(j << 4));
                f.b[j] = cat4(ds64tr<0>(ad), ds64tr<8 * TBN>(ad), ds64tr<16 * TBN>(ad), ds64tr<24 * TBN>(ad));
            }
        } else {
            const uint32_t b0 = so + kAStage + sw(64 * wq + lrow, 2 * kgrp);
            const uint32_t b1 = so + kAStage + sw(64 * wq + lrow, 2 * kgrp + 1);
            f.b[0] = frag_nk<0>(b0, b1);
            f.b[1] = frag_nk<1>(b0, b1);
            f.b[2] = frag_nk<2>(b0, b1);
            f.b[3] = frag_nk<3>(b0, b1);
        }
    };
    // A fragments and scales of the chunk in stage st (A rows are loaded by
    // all four waves of the group: read after the phase barrier)
    auto read_a = [&](int st, Frags& f, int c) {
        int l = lane;
        asm volatile("" : "+v"(l));
        const int lrow = l & 15, kgrp = l >> 4;
        const uint32_t so = lds_addr(Stg) + (uint32_t)st * kStageBytes;
        if (P2) {
            // byte c & 3 of the scale words (dense: the chunk index is kg)
            const uint32_t sel = (uint32_t)(c & 3);
            const uint32_t sa = lds_addr(SAs) + (uint32_t)(st * TBM + lrow) * 4 + sel;
            f.e[0] = ds_u8<0>(sa);
            f.e[1] = ds_u8<64>(sa);
            f.e[2] = ds_u8<128>(sa);
            f.e[3] = ds_u8<192>(sa);
            f.e[4] = ds_u8<256>(sa);
            f.e[5] = ds_u8<320>(sa);
            f.e[6] = ds_u8<384>(sa);
            f.e[7] = ds_u8<448>(sa);
            if (SB_MODE == SB_BLOCK) {
                const uint32_t byte = B_KN ? (uint32_t)((n0 >> 7) & 3) + (uint32_t)(wq >> 1)
                                           : (uint32_t)(wq >> 1) * 4 + sel;
                f.ebk = ds_u8<0>(lds_addr(SBs) + (uint32_t)(st * 64) * 4 + byte);
            }
            if (SB_MODE == SB_ROW) {
                const uint32_t sb = lds_addr(SBs) + (uint32_t)((c % kSbStages) * TBN + 64 * wq + lrow) * 4 + sel;
                f.eb[0] = ds_u8<0>(sb);
                f.eb[1] = ds_u8<64>(sb);
                f.eb[2] = ds_u8<128>(sb);
                f.eb[3] = ds_u8<192>(sb);
            }
        } else if (SA_MODE == SA_ROW) {
            const uint32_t sa = lds_addr(SAs) + (uint32_t)(st * TBM + lrow) * 4;
            f.s[0] = ds32<0>(sa);
            f.s[1] = ds32<64>(sa);
            f.s[2] = ds32<128>(sa);
            f.s[3] = ds32<192>(sa);
            f.s[4] = ds32<256>(sa);
            f.s[5] = ds32<320>(sa);
            f.s[6] = ds32<384>(sa);
            f.s[7] = ds32<448>(sa);
        }
        if (!P2 && SB_MODE == SB_BLOCK) f.sbk = ds32<0>(lds_addr(SBs) + (uint32_t)(st * 64 + (wq >> 1)) * 4);
        const uint32_t a0 = so + sw(lrow, 2 * kgrp), a1 = so + sw(lrow, 2 * kgrp + 1);
        f.a[0] = frag_nk<0>(a0, a1);
        f.a[1] = frag_nk<1>(a0, a1);
        f.a[2] = frag_nk<2>(a0, a1);
        f.a[3] = frag_nk<3>(a0, a1);
        f.a[4] = frag_nk<4>(a0, a1);
        f.a[5] = frag_nk<5>(a0, a1);
        f.a[6] = frag_nk<6>(a0, a1);
        f.a[7] = frag_nk<7>(a0, a1);
    };
    // all reads of f have landed; fold the chunk's B scale into the row scales
    auto reads_wait = [&](Frags& f) {
        lgkm_wait<0>(f.a[7]);
        pin4(f.a[0], f.a[1], f.a[2], f.a[3]);
        asm volatile("" : "+v"(f.a[4]), "+v"(f.a[5]), "+v"(f.a[6]));
        pin4(f.b[0], f.b[1], f.b[2], f.b[3]);
        if (P2) {
            asm volatile("" : "+v"(f.e[0]), "+v"(f.e[1]), "+v"(f.e[2]), "+v"(f.e[3]),
                              "+v"(f.e[4]), "+v"(f.e[5]), "+v"(f.e[6]), "+v"(f.e[7]));
            if (SB_MODE == SB_ROW) asm volatile("" : "+v"(f.eb[0]), "+v"(f.eb[1]), "+v"(f.eb[2]), "+v"(f.eb[3]));
            if (SB_MODE == SB_BLOCK) asm volatile("" : "+v"(f.ebk));
            return;
        }
        if (SA_MODE == SA_ROW)
            asm volatile("" : "+v"(f.s[0]), "+v"(f.s[1]), "+v"(f.s[2]), "+v"(f.s[3]),
                              "+v"(f.s[4]), "+v"(f.s[5]), "+v"(f.s[6]), "+v"(f.s[7]));
        if (SB_MODE == SB_BLOCK) asm volatile("" : "+v"(f.sbk));
        const float sbv = SB_MODE == SB_BLOCK ? f.sbk : SB_MODE == SB_TENSOR ? sb_t : 1.0f;
#pragma unroll
        for (int i = 0; i < PMI; ++i)
            f.s[i] = SB_MODE == SB_ROW ? (SA_MODE == SA_ROW ? f.s[i] : sa_t) : (SA_MODE == SA_ROW ? f.s[i] : sa_t) * sbv;
    };
    // Partial last chunk: every fragment of a lane (A, B as [N][K] or, through
    // the transposing reads, as [K][N]) holds the chunk's K bytes
    // [32 kgrp, 32 kgrp + 32) in order, so one mask per dword clears the bytes
    // at or past K in both operands (a code past K may be anything, NaN too).
    auto mask_k_tail = [&](Frags& f) {
        const int kgrp = lane >> 4;
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            const int keep = k_tail - (32 * kgrp + 4 * d);
            const int mk = keep >= 4 ? -1 : (keep <= 0 ? 0 : (int)((1u << (8 * keep)) - 1u));
#pragma unroll
            for (int i = 0; i < PMI; ++i) f.a[i][d] &= mk;
#pragma unroll
            for (int j = 0; j < NNI; ++j) f.b[j][d] &= mk;
        }
    };
    // the 32 MFMAs of chunk c in f; the FMAs of block u run behind the MFMA
    // of block u+1.  Row-scaled B: the lane's 4 column scales of block j are
    // read from LDS while the MFMAs of block j-1 run, and each FMA takes
    // the product of its row and column scale.
    auto compute = [&](Frags& f, int c) {
        if constexpr (P2) {
            // the scaled MFMA: first scale for the first operand (B rows,
            // lane l: row l % 16), second for A rows; each lane gives the
            // byte of the row it holds, the same for its four 32-wide K groups
#pragma unroll
            for (int u = 0; u < PMI * NNI; ++u) {
                const int j = u / PMI, i = u % PMI;
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    f.b[j], f.a[i], acc[i][j], 0, 0, 0, SB_MODE == SB_ROW ? f.eb[j] : f.ebk, 0, f.e[i]);
            }
#pragma unroll
            for (int i = 0; i < PMI; ++i)
#pragma unroll
                for (int j = 0; j < NNI; ++j) asm volatile("" : "+v"(acc[i][j]));
            return;
        }
        uint32_t sbp = 0;
        v4f sc[NNI];
        if (SB_MODE == SB_ROW) {
            int l = lane;
            asm volatile("" : "+v"(l));
            sbp = lds_addr(SBs) + (uint32_t)((c % kSbStages) * TBN + 64 * wq + 4 * (l >> 4)) * 4;
            sc[0] = col_scales(sbp, 0);
        }
        auto scale_fma = [&](const v4f& pv, int pi, int pj) {
            if (SB_MODE == SB_ROW) {
                if (pi == 0) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(sc[pj]));
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[pi][pj][r] = __builtin_fmaf(pv[r], f.s[pi] * sc[pj][r], acc[pi][pj][r]);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[pi][pj][r] = __builtin_fmaf(pv[r], f.s[pi], acc[pi][pj][r]);
            }
        };
        v4f prev = zero;
#pragma unroll
        for (int u = 0; u < PMI * NNI; ++u) {
            const int j = u / PMI, i = u % PMI;
            const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.b[j], f.a[i], zero, 0, 0, 0, 0, 0, 0);
            if (SB_MODE == SB_ROW && i == 1 && j + 1 < NNI) sc[j + 1] = col_scales(sbp, j + 1);
            if (u > 0) scale_fma(prev, (u - 1) % PMI, (u - 1) / PMI);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, SB_MODE == SB_ROW ? 8 : 4, 0);
            __builtin_amdgcn_sched_barrier(0);
            prev = part;
        }
        scale_fma(prev, PMI - 1, NNI - 1);
#pragma unroll
        for (int i = 0; i < PMI; ++i)
#pragma unroll
            for (int j = 0; j < NNI; ++j) asm volatile("" : "+v"(acc[i][j]));
    };
    auto bar = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    // group g loads chunk g of the first tile
    if (grp < KB) issue(grp);
    for (;;) {
#pragma unroll
        for (int i = 0; i < PMI; ++i)
#pragma unroll
            for (int j = 0; j < NNI; ++j) acc[i][j] = zero;
        if (KB > 0) {
            // KB + 1 phases, each a barrier in every wave.  Phase c: chunk c's
            // loads (issued by this group two phases ago) landed, and chunk
            // c-1's stage, read in phase c-1, takes chunk c+2.
            // A group reads the B fragments of its next chunk right after its
            // compute phase (its own loads, two phases old by then), so its
            // read phase holds only the A fragments and scales.
            Frags f;
            int q = 0;
            if (grp == 1) {
                bar();
                q = 1;
            }
            if (kEarlyB && grp < KB) {
                wait_vm<0>();
                read_b(grp % kStages, f);
            }
            for (int c = grp; c < KB; c += 2) {
                if (!kEarlyB) wait_vm<0>();
                bar();
                if (kPrio == 1) __builtin_amdgcn_s_setprio(1);
                if (kPrio == 2) __builtin_amdgcn_s_setprio(0);
                // the fragment reads go first: they complete while the loads
                // of chunk c + 2 are being issued (issuing them waits on the
                // CU's vector-memory queue, ~850 cycles per chunk per wave)
                if (!kReadsFirst && c + 2 < KB) issue(c + 2);
                if (!kEarlyB) read_b(c % kStages, f);
                read_a(c % kStages, f, c);
                __builtin_amdgcn_sched_barrier(0);
                if (kReadsFirst && c + 2 < KB) issue(c + 2);
                __builtin_amdgcn_sched_barrier(0);
                reads_wait(f);
                if (c == KB - 1 && k_tail < TBK) mask_k_tail(f);
                if (kPrio == 1) __builtin_amdgcn_s_setprio(0);
                if (kPrio == 2) __builtin_amdgcn_s_setprio(1);
                bar();
                compute(f, c);
                if (kEarlyB && c + 2 < KB) {
                    wait_vm<0>();
                    read_b((c + 2) % kStages, f);
                }
                q = c + 2;
            }
            if (q == KB) bar();
        }
        if (kPrio == 2) __builtin_amdgcn_s_setprio(0);
        // Add the two groups' halves: group 0 finishes rows [0, 64), group 1
        // rows [64, 128).  Each wave sends the other half to its partner (the
        // wave of the other group with the same columns) through a 16 KB slot
        // of the LDS ring, which no wave reads or loads into any more.
        const int64_t cm0 = m0, cn0 = n0;
        const bool store_tile = tile_live;
        ti += nwg;
        const bool more = ti < tiles_here;
        const uint32_t slot_out = lds_addr(Stg) + (uint32_t)(wave * 16384 + lane * 16);
        const uint32_t slot_in = lds_addr(Stg) + (uint32_t)(((wave + 4) & 7) * 16384 + lane * 16);
        auto finish = [&](auto half) {
            constexpr int h = decltype(half)::value;   // rows kept: [64h, 64h+64)
            constexpr int o = (1 - h) * 4;            // first block sent
#pragma unroll
            for (int q2 = 0; q2 < 16; ++q2) {
                const v4f v = acc[o + q2 / 4][q2 % 4];
                switch (q2) {
#define FP8Q_W(Q) case Q: ds_write128<Q * 1024>(slot_out, v); break;
                    FP8Q_W(0) FP8Q_W(1) FP8Q_W(2) FP8Q_W(3) FP8Q_W(4) FP8Q_W(5) FP8Q_W(6) FP8Q_W(7)
                    FP8Q_W(8) FP8Q_W(9) FP8Q_W(10) FP8Q_W(11) FP8Q_W(12) FP8Q_W(13) FP8Q_W(14) FP8Q_W(15)
#undef FP8Q_W
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            v4f in[16];
#pragma unroll
            for (int q2 = 0; q2 < 16; ++q2) {
                switch (q2) {
#define FP8Q_R(Q) case Q: in[Q] = (v4f)ds128<Q * 1024>(slot_in); break;
                    FP8Q_R(0) FP8Q_R(1) FP8Q_R(2) FP8Q_R(3) FP8Q_R(4) FP8Q_R(5) FP8Q_R(6) FP8Q_R(7)
                    FP8Q_R(8) FP8Q_R(9) FP8Q_R(10) FP8Q_R(11) FP8Q_R(12) FP8Q_R(13) FP8Q_R(14) FP8Q_R(15)
#undef FP8Q_R
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            const int lrow = lane & 15, kgrp = lane >> 4;
#pragma unroll
            for (int q2 = 0; q2 < 16; ++q2) {
                asm volatile("" : "+v"(in[q2]));
                acc[h * 4 + q2 / 4][q2 % 4] += in[q2];
            }
            if (OUT == OUT_E4M3) {
                // Quantize-on-store: the output's 1x128 tiles along N.  A
                // tile is the 64 columns of this wave and those of wave ^ 1
                // (same rows).  Columns past N are left out of the amax (with
                // [K][N] B they are computed from bytes past the row's end).
                float mx[4];
                const int64_t ncol0 = cn0 + 64 * wq + 4 * kgrp;
                if (cn0 + 64 * wq + 64 <= N) {
                    // all 64 columns inside: |x| maxima three operands at a time
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float v = 0.0f;
#pragma unroll
                        for (int j = 0; j < NNI; ++j) {
                            v = nk_max3_abs(v, acc[h * 4 + i][j][0], acc[h * 4 + i][j][1]);
                            v = nk_max3_abs(v, acc[h * 4 + i][j][2], acc[h * 4 + i][j][3]);
                        }
                        mx[i] = v;
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float v = 0.0f;
#pragma unroll
                        for (int j = 0; j < NNI; ++j)
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (ncol0 + 16 * j + r < N) v = fmaxf(v, fabsf(acc[h * 4 + i][j][r]));
                        mx[i] = v;
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = fmaxf(mx[i], __shfl_xor(mx[i], 16));
                    mx[i] = fmaxf(v, __shfl_xor(v, 32));
                }
                // row maxima of the two waves of a tile meet past the
                // exchange slots in the ring
                const uint32_t am = lds_addr(Stg) + 8u * 16384u;
                if (kgrp == 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        *reinterpret_cast<__attribute__((address_space(3))) float*>(
                            (uintptr_t)(am + (uint32_t)(wave * 64 + 16 * i + lrow) * 4)) = mx[i];
                }
                __syncthreads();
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    mx[i] = fmaxf(mx[i], *reinterpret_cast<__attribute__((address_space(3))) const float*>(
                                             (uintptr_t)(am + (uint32_t)((wave ^ 1) * 64 + 16 * i + lrow) * 4)));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const TileScale ts = make_scale(mx[i]);
                    uint32_t code[NNI];
                    float v[8];
#pragma unroll
                    for (int jp = 0; jp < NNI / 2; ++jp) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            v[r] = acc[h * 4 + i][2 * jp][r];
                            v[4 + r] = acc[h * 4 + i][2 * jp + 1][r];
                        }
                        quant8(v, ts, code[2 * jp], code[2 * jp + 1]);
                    }
                    const int64_t m = cm0 + 64 * h + 16 * i + lrow;
                    if (m >= M || !store_tile) continue;
                    uint8_t* qrow = reinterpret_cast<uint8_t*>(p.c) + m * p.ldc;
#pragma unroll
                    for (int j = 0; j < NNI; ++j) {
                        const int64_t n = cn0 + 64 * wq + 16 * j + 4 * kgrp;
                        if (n + 3 < N) {
                            *reinterpret_cast<uint32_t*>(qrow + n) = code[j];
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (n + r < N) qrow[n + r] = (uint8_t)(code[j] >> (8 * r));
                        }
                    }
                    const int64_t n_tile = cn0 + 64 * wq;
                    if (kgrp == 0 && (wq & 1) == 0 && n_tile < N) p.cs[m * p.ldcs + n_tile / 128] = ts.s;
                }
                return;
            }
            // lane l holds C[m][n .. n+3] of each kept block
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t m = cm0 + 64 * h + 16 * i + lrow;
                if (m >= M || !store_tile) continue;
#pragma unroll
                for (int j = 0; j < NNI; ++j) {
                    const int64_t n = cn0 + 64 * wq + 16 * j + 4 * kgrp;
                    const v4f v = acc[h * 4 + i][j];
                    if (n + 3 < N) {
                        if (OUT == OUT_BF16) {
                            const uint32_t lo = bf16x2_rne(v[0], v[1]);
                            const uint32_t hi = bf16x2_rne(v[2], v[3]);
                            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.c) + m * p.ldc + n) = make_uint2(lo, hi);
                        } else {
                            *reinterpret_cast<v4f*>(reinterpret_cast<float*>(p.c) + m * p.ldc + n) = v;
                        }
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            if (n + r < N) {
                                if (OUT == OUT_BF16)
                                    reinterpret_cast<uint16_t*>(p.c)[m * p.ldc + n + r] = (uint16_t)bf16_rne(v[r]);
                                else
                                    reinterpret_cast<float*>(p.c)[m * p.ldc + n + r] = v[r];
                            }
                        }
                    }
                }
            }
        };
        if (grp == 0) finish(std::integral_constant<int, 0>{});
        else finish(std::integral_constant<int, 1>{});
        if (!more) break;
        tile_origin(ti, m0, n0);
        set_group(m0);
        rsb = sb_rsrc();
        // every wave is done with the exchange slots before they are loaded into
        __builtin_amdgcn_s_barrier();
        if (grp < KB) issue(grp);
    }
    wait_vm<0>();
}

template <int SA_MODE, int SB_MODE, bool B_KN, int OUT, int GMODE = 0, bool P2 = false>
static void launch_out(const GemmArgs& g, hipStream_t st)
{
    GemmArgs a = g;
    a.tiles_m = (int)((g.M + TBM - 1) / TBM);
    a.tiles_n = (int)((g.N + TBN - 1) / TBN);
    const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
    dim3 grid((uint32_t)(tiles < g.num_cus ? tiles : g.num_cus));
    hipLaunchKernelGGL((gemm_nk_kernel<SA_MODE, SB_MODE, B_KN, OUT, GMODE, P2>), grid, dim3(kThreads), 0, st, a);
}

template <int SA_MODE, int SB_MODE, bool B_KN, int GMODE = 0>
static void launch_tiles(const GemmArgs& g, int out, hipStream_t st)
{
    if (out == OUT_BF16) launch_out<SA_MODE, SB_MODE, B_KN, OUT_BF16, GMODE>(g, st);
    else if (out == OUT_F32) launch_out<SA_MODE, SB_MODE, B_KN, OUT_F32, GMODE>(g, st);
    else if constexpr (GMODE == 0 && SB_MODE != SB_ROW) launch_out<SA_MODE, SB_MODE, B_KN, OUT_E4M3, GMODE>(g, st);
}

bool launch_grouped_gemm_nk(const GemmArgs& g, bool out_bf16, bool b_kn, hipStream_t st)
{
    const int64_t lim = (int64_t)1 << 31;
    const int64_t b_rows = b_kn ? g.K : g.N;
    if (g.G > kMaxLdsGroups || g.M * g.lda >= lim || (b_rows + TBK) * g.ldb >= lim ||
        g.M * g.ldsa * 4 >= lim || g.sb_group_stride * 4 >= lim || (int64_t)g.KB * TBK >= lim)
        return false;
    const int out = out_bf16 ? OUT_BF16 : OUT_F32;
    if (b_kn) launch_tiles<SA_ROW, SB_BLOCK, true, 1>(g, out, st);
    else launch_tiles<SA_ROW, SB_BLOCK, false, 1>(g, out, st);
    return true;
}

// Every operand of one dense launch must span less than 2 GiB: the kernel
// addresses them through 32-bit buffer offsets, and reads up to a tile of
// rows past the end of A, B and the scale grids (clamped to zero by the
// buffer bounds).  `sbytes` is the size of one scale (4 fp32, 1 E8M0).
static bool dense_fits(const GemmArgs& g, int sa_mode, int sb_mode, bool b_kn, int sbytes)
{
    const int64_t lim = (int64_t)1 << 31;
    const int64_t pad = 256;
    const int64_t b_rows = b_kn ? g.K : g.N;
    const int64_t nblocks = (g.N + 127) / 128;
    int64_t sb_ext = 4;
    if (sb_mode == SB_ROW) sb_ext = (g.N + pad) * g.ldsb * sbytes;
    else if (sb_mode == SB_BLOCK) sb_ext = (b_kn ? (int64_t)g.KB + 1 : nblocks + 2) * g.ldsb * sbytes;
    const int64_t sa_ext = sa_mode == SA_ROW ? (g.M + pad) * g.ldsa * sbytes : 4;
    return (g.M + pad) * g.lda < lim && (b_rows + pad) * g.ldb < lim && sa_ext < lim && sb_ext < lim &&
           (int64_t)g.KB * TBK < lim;
}

bool launch_gemm_nk_e8m0(const GemmArgs& g, int sb_mode, bool b_kn, bool out_bf16, hipStream_t st)
{
    if (!dense_fits(g, SA_ROW, sb_mode, b_kn, 1)) return false;
    if (b_kn && sb_mode != SB_BLOCK) return false;
    if (launch_gemm_w4_e8m0(g, sb_mode, b_kn, out_bf16, st)) return true;
    if (b_kn) {
        if (out_bf16) launch_out<SA_ROW, SB_BLOCK, true, OUT_BF16, 0, true>(g, st);
        else launch_out<SA_ROW, SB_BLOCK, true, OUT_F32, 0, true>(g, st);
    } else if (sb_mode == SB_BLOCK) {
        if (out_bf16) launch_out<SA_ROW, SB_BLOCK, false, OUT_BF16, 0, true>(g, st);
        else launch_out<SA_ROW, SB_BLOCK, false, OUT_F32, 0, true>(g, st);
    } else {
        if (out_bf16) launch_out<SA_ROW, SB_ROW, false, OUT_BF16, 0, true>(g, st);
        else launch_out<SA_ROW, SB_ROW, false, OUT_F32, 0, true>(g, st);
    }
    return true;
}

bool launch_gemm_nk(const GemmArgs& g, int sa_mode, int sb_mode, bool b_kn, int out, hipStream_t st)
{
    if (!dense_fits(g, sa_mode, sb_mode, b_kn, 4)) return false;
    if (launch_gemm_w4(g, sa_mode, sb_mode, b_kn, out, st)) return true;
    if (b_kn) {
        if (sb_mode == SB_ROW) return false;
        if (sa_mode == SA_ROW) {
            if (sb_mode == SB_BLOCK) launch_tiles<SA_ROW, SB_BLOCK, true>(g, out, st);
            else launch_tiles<SA_ROW, SB_TENSOR, true>(g, out, st);
        } else {
            if (sb_mode == SB_BLOCK) launch_tiles<SA_TENSOR, SB_BLOCK, true>(g, out, st);
            else launch_tiles<SA_TENSOR, SB_TENSOR, true>(g, out, st);
        }
        return true;
    }
    if (sa_mode == SA_ROW) {
        if (sb_mode == SB_BLOCK) launch_tiles<SA_ROW, SB_BLOCK, false>(g, out, st);
        else if (sb_mode == SB_ROW) launch_tiles<SA_ROW, SB_ROW, false>(g, out, st);
        else launch_tiles<SA_ROW, SB_TENSOR, false>(g, out, st);
    } else {
        if (sb_mode == SB_BLOCK) launch_tiles<SA_TENSOR, SB_BLOCK, false>(g, out, st);
        else if (sb_mode == SB_ROW) launch_tiles<SA_TENSOR, SB_ROW, false>(g, out, st);
        else launch_tiles<SA_TENSOR, SB_TENSOR, false>(g, out, st);
    }
    return true;
}

}  // namespace fp8q
