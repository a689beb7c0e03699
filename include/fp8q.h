/*
 * fp8q.h -- block-scaled FP8 (E4M3) quantization and FP8 GEMM for AMD
 * Instinct MI355X (gfx950).  C ABI of libfp8q.so.
 *
 * What is computed (the web pages on FP8 training):
 *  - A high-precision tensor becomes an FP8 tensor plus a much smaller,
 *    wider-range scale tensor ("quantization"); dequantization is the inverse
 *    (Ling 2.0 FP8 blog, "where does the precision worry come from").
 *  - The rule is x_fp8 = Cast_FP8(x / s) (FP8-LM review, section 三, tensor
 *    scaling).  E4M3 has 4 exponent bits and 3 mantissa bits and covers
 *    [-448, 448] ("FP8-RL" article, section 一; FP8-LM review, section 三).
 *  - Scales are kept per tile / per block so that outliers only affect their
 *    own tile (Ling 2.0 FP8 blog, "fine-grained quantization"); weights use
 *    128x128 blocks ("FP8-RL" article, section 一); activations and gradients
 *    are quantized dynamically (same section) with 1x128 tiles.
 *  - The FP8 GEMM accumulates in FP32 (Ling 2.0 FP8 blog, "where is error
 *    introduced").  dgrad reads the weight in its stored layout instead of a
 *    cached transposed copy, and wgrad consumes a transposed re-quantization
 *    of the gradient (Ling 2.0 FP8 blog, "FP8 on-demand transpose weight" and
 *    the underflow monitor of "grad (transpose)").  MoE experts run as one
 *    grouped GEMM over groups padded to the kernel's row multiple (Ling 2.0
 *    FP8 blog, "FP8 padding routing map").
 *
 * Numerics (exact contract; the CPU oracle implements the same definitions):
 *  - Codes are OCP E4M3FN bytes (bias 7, subnormals, no infinities, NaN =
 *    S.1111.111), the same bytes as torch.float8_e4m3fn.
 *  - Per tile: amax = max |x| (fp32; bf16 inputs widen exactly),
 *    s = amax / 448 (IEEE fp32 division), code = E4M3(RN_fp32(x / s)) with
 *    round-to-nearest-even and saturation at +-448; the code's sign bit is the
 *    sign bit of x.  If s == 0 (zero tile, or amax so small that amax/448
 *    underflows) every code is a signed zero.  s is stored as-is: it is the
 *    dequantization multiplier (x ~= dec(code) * s).
 *  - GEMM: C[m][n] = sum over K-chunks kb of 128 (the last may be shorter) of
 *    SA(m,kb) * SB(n,kb) * sum_{k in kb} dec(A[m][k]) * dec(B^[n][k]),
 *    products exact, fp32 partial sums, fp32 accumulator; the summation
 *    order inside a chunk is the hardware's, and the order in which the
 *    chunk terms are added is unspecified (the library adds the even and the
 *    odd chunks separately, then the two sums).  BF16 output is the fp32
 *    result rounded to nearest even.
 *  - Inputs must be finite; NaN/Inf inputs give unspecified codes.
 *
 * Conventions for every entry point:
 *  - All data pointers are DEVICE pointers to memory on the current HIP
 *    device.  The library never allocates, frees, synchronizes or keeps a
 *    pointer after returning; all work is enqueued on `stream` (a
 *    hipStream_t, or NULL for the default stream).  The caller keeps every
 *    buffer alive until the stream has finished the work.
 *  - Matrices are row-major with a leading dimension `ld*` in ELEMENTS.
 *    Every matrix pointer must be 16-byte aligned and ld * element_size must
 *    be a multiple of 16 bytes.  Inputs may be read up to the 16-byte
 *    boundary past the last column of a row (never past ld); outputs are
 *    written exactly in [0, rows) x [0, cols).  Scale grids have no alignment
 *    requirement (4-byte floats).
 *  - Shapes may be any size >= 0 (ragged edge tiles are clipped); a call with
 *    an empty output returns FP8Q_OK without launching anything.  A GEMM
 *    with K == 0 writes zeros; its operand and scale pointers may then be
 *    NULL (they are not read).  (fp8_grouped_gemm_e4m3 is the exception: it
 *    takes K as a positive multiple of 128 only.)
 *  - Arguments are validated on the host before any launch; a failing call
 *    returns its status and enqueues nothing.  After launching, a pending
 *    launch error is reported as FP8Q_ERR_LAUNCH.
 *  - Calls are stateless and thread-safe (the only state is a per-device
 *    architecture check cached at first use).
 *  - Debug mode: with the environment variable FP8Q_CHECK=1 (read at every
 *    call) each call synchronizes its stream after enqueueing and reports an
 *    error of the work as FP8Q_ERR_LAUNCH, and the grouped GEMMs first check
 *    the group-offset contract on the device (one small kernel and a
 *    synchronization; a violation returns FP8Q_ERR_SHAPE and enqueues no
 *    GEMM).  Without it the offsets are the caller's responsibility.
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A HIP stream (NULL: the default stream); the same type as the HIP
 * runtime's hipStream_t, declared here so that this header needs no HIP
 * header.  Data types, scale kinds and B layouts are passed as int, with the
 * values of the enums below: a value outside an enum's list, which a C or
 * foreign-function caller can pass, then reaches the validation as a defined
 * int and is rejected (FP8Q_ERR_UNSUPPORTED); as an enum-typed parameter it
 * would be undefined behaviour in the C++ implementation. */
typedef struct ihipStream_t* hipStream_t;

typedef enum {
    FP8Q_OK = 0,
    FP8Q_ERR_NULL = 1,        /* a required pointer is NULL */
    FP8Q_ERR_SHAPE = 2,       /* negative size, ld too small, or grid/offset size mismatch */
    FP8Q_ERR_ALIGN = 3,       /* pointer not 16-byte aligned or ld*elem not a multiple of 16 */
    FP8Q_ERR_UNSUPPORTED = 4, /* unsupported dtype / scale kind / layout combination */
    FP8Q_ERR_DEVICE = 5,      /* current device is not gfx950, or a HIP query failed */
    FP8Q_ERR_LAUNCH = 6       /* a kernel launch failed */
} fp8q_status;

typedef enum { FP8Q_F32 = 0, FP8Q_BF16 = 1 } fp8q_dtype;

typedef enum {
    FP8Q_ROW_1x128 = 0,     /* tile = 1 row x 128 columns; s[r * lds + c/128] */
    FP8Q_BLOCK_128x128 = 1, /* tile = 128 x 128;           s[(r/128) * lds + c/128] */
    FP8Q_TENSOR = 2         /* one tile = the whole matrix; s[0] */
} fp8q_scale_kind;

typedef enum {
    FP8Q_B_NK = 0, /* B stored [N][K]: B^[n][k] = b[n * ldb + k]  (y = x W^T, wgrad) */
    FP8Q_B_KN = 1  /* B stored [K][N]: B^[n][k] = b[k * ldb + n]  (dgrad: dx = dy W)  */
} fp8q_b_layout;

/*
 * fp8_quant_blockwise -- quantize X[rows][cols] to E4M3 codes + fp32 scales.
 *
 *  x       : input, x_dtype (FP8Q_F32 or FP8Q_BF16), row stride ldx >= cols.
 *  kind    : FP8Q_ROW_1x128 (activations, gradients), FP8Q_BLOCK_128x128
 *            (weights) or FP8Q_TENSOR (one scale; comparison baseline).
 *  q       : output codes [rows][cols], row stride ldq >= cols.
 *  s       : output scales.  ROW: [rows][ceil(cols/128)] with row stride
 *            lds >= ceil(cols/128).  BLOCK: [ceil(rows/128)][ceil(cols/128)]
 *            with row stride lds.  TENSOR: s[0] (lds ignored); s[0] is also
 *            used as the amax cell while the call runs.
 * Tiles start at row 0 / column 0 and are clipped at the matrix edge.
 */
int fp8_quant_blockwise(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                        int kind, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                        hipStream_t stream);

/*
 * fp8_quant_transpose -- one read of X[rows][cols] produces both
 *   (i)  row tiles along cols:   q_row[rows][cols],   s_row[rows][ceil(cols/128)]
 *   (ii) column tiles along rows, stored transposed, i.e. the 1x128 row tiles
 *        of X^T:                 q_colT[cols][rows],  s_colT[cols][ceil(rows/128)]
 * (ii) is the operand of the weight-gradient GEMM (contraction over tokens);
 * it is re-quantized from the high-precision input, never transposed codes.
 * Either output pair may be NULL (both pointers of the pair) to skip it.
 * Strides: ldq_row >= cols, lds_row >= ceil(cols/128), ldq_colT >= rows,
 * lds_colT >= ceil(rows/128).  x_dtype is FP8Q_F32 or FP8Q_BF16.
 */
int fp8_quant_transpose(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                        uint8_t* q_row, int64_t ldq_row, float* s_row, int64_t lds_row,
                        uint8_t* q_colT, int64_t ldq_colT, float* s_colT, int64_t lds_colT,
                        hipStream_t stream);

/*
 * fp8_gemm_blockscaled -- C[M][N] = block-scaled FP8 product (see Numerics).
 *
 *  a, lda        : A codes [M][K], contraction axis contiguous.
 *  sa, ldsa      : A scales. sa_kind FP8Q_ROW_1x128: SA(m,kb) = sa[m*ldsa + kb]
 *                  (ldsa >= ceil(K/128)); FP8Q_TENSOR: SA = sa[0].
 *  b, ldb        : B codes, b_layout FP8Q_B_NK ([N][K], ldb >= K) or
 *                  FP8Q_B_KN ([K][N], ldb >= N).
 *  sb, ldsb      : B scales. sb_kind
 *                  FP8Q_BLOCK_128x128, NK: SB(n,kb) = sb[(n/128)*ldsb + kb]
 *                  FP8Q_BLOCK_128x128, KN: SB(n,kb) = sb[kb*ldsb + n/128]
 *                     (the block grid follows B's storage, so the weight's
 *                      own scales serve dgrad without a transposed copy)
 *                  FP8Q_ROW_1x128, NK only: SB(n,kb) = sb[n*ldsb + kb] (wgrad)
 *                  FP8Q_TENSOR: SB = sb[0].
 *  c, ldc, c_dtype : output [M][N], FP8Q_F32 or FP8Q_BF16, ldc >= N.
 * Typical uses: forward y = x W^T (ROW x BLOCK, NK); dgrad dx = dy W
 * (ROW x BLOCK, KN); wgrad dW = dy^T x (ROW x ROW, NK, operands from
 * fp8_quant_transpose's column outputs).
 * Operands of 2 GiB or more are handled by several launches over slices of
 * M (and, for FP8Q_B_NK, of N).  Returns FP8Q_ERR_UNSUPPORTED (nothing
 * enqueued) if a FP8Q_B_KN operand spans 2 GiB or more, or a single 256-row
 * slice of an operand does.
 */
int fp8_gemm_blockscaled(int64_t M, int64_t N, int64_t K,
                         const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa, int sa_kind,
                         const uint8_t* b, int64_t ldb, int b_layout,
                         const float* sb, int64_t ldsb, int sb_kind,
                         void* c, int64_t ldc, int c_dtype, hipStream_t stream);

/*
 * fp8_gemm_blockscaled_e4m3 -- the same product, stored quantized: the
 * output's E4M3 codes and its 1x128 scales along N (the next layer's dynamic
 * activation quantization, Ling 2.0 FP8 blog "fine-grained quantization";
 * "FP8-RL" article, section 一, activations quantized on the fly), with no
 * fp32/bf16 round trip through memory.
 *
 * With C the fp32 result of fp8_gemm_blockscaled for the same arguments, the
 * codes and scales are exactly those fp8_quant_blockwise(FP8Q_ROW_1x128)
 * gives for C (see Numerics).
 *  a .. sb_kind : as fp8_gemm_blockscaled, except that sb_kind
 *                 FP8Q_ROW_1x128 (the weight-gradient operands, whose result
 *                 feeds the optimizer in fp32) is FP8Q_ERR_UNSUPPORTED.
 *  q, ldq       : codes [M][N], ldq >= N (multiple of 16, q 16-byte aligned).
 *  s, lds       : scales s[m*lds + n/128], lds >= ceil(N/128).
 * Large operands are sliced as for fp8_gemm_blockscaled, with the same
 * FP8Q_ERR_UNSUPPORTED cases.
 */
int fp8_gemm_blockscaled_e4m3(int64_t M, int64_t N, int64_t K,
                              const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa, int sa_kind,
                              const uint8_t* b, int64_t ldb, int b_layout,
                              const float* sb, int64_t ldsb, int sb_kind,
                              uint8_t* q, int64_t ldq, float* s, int64_t lds, hipStream_t stream);

/*
 * fp8_grouped_gemm -- MoE expert GEMM over padded groups.
 *
 * For each group e in [0, G): rows [off[e], off[e+1]) of A times expert
 * weights B[e]:  C[m][n] = block-scaled product of A[m][:] (1x128 scales) and
 * B[e][n][:] (128x128 block scales).
 *  a, lda, sa, ldsa : A codes [M_pad][K] (contiguous groups), scales
 *                     sa[m*ldsa + kb].
 *  group_offsets    : DEVICE int32[G+1]; off[0] = 0, off[G] <= M_pad,
 *                     non-decreasing, every off[e] a multiple of 128 (the
 *                     caller pads each group with zero rows; zero codes with
 *                     s = 0 give zero output rows).  This device-side
 *                     contract is the caller's: rows outside [0, off[G]) are
 *                     not written.
 *  b                : B codes [G][N][K] (each expert NK, row stride K; K % 16 == 0).
 *  sb               : B scales [G][ceil(N/128)][ceil(K/128)], contiguous.
 *  c, ldc, c_dtype  : output [M_pad][N].
 * M_pad must be a multiple of 128.  Returns FP8Q_ERR_UNSUPPORTED (nothing
 * enqueued) if G > 1024 or an operand spans 2 GiB or more.
 */
int fp8_grouped_gemm(int64_t G, int64_t M_pad, int64_t N, int64_t K,
                     const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                     const int32_t* group_offsets,
                     const uint8_t* b, const float* sb,
                     void* c, int64_t ldc, int c_dtype, hipStream_t stream);

/*
 * fp8_grouped_gemm_e4m3 -- the same MoE expert GEMM stored quantized: E4M3
 * codes of C and its 1x128 scales along N (the next layer's activation
 * quantization, as fp8_gemm_blockscaled_e4m3; Ling 2.0 FP8 blog, "FP8 padding
 * routing map" and "fine-grained quantization").
 *
 * With C the fp32 result of fp8_grouped_gemm for the same arguments, the
 * codes and scales of rows [0, off[G]) are exactly those
 * fp8_quant_blockwise(FP8Q_ROW_1x128) gives for C; rows at or past off[G]
 * are not written.
 *  a .. sb : as fp8_grouped_gemm.
 *  q, ldq  : codes [M_pad][N], ldq >= N (multiple of 16, q 16-byte aligned).
 *  s, lds  : scales s[m*lds + n/128], lds >= ceil(N/128).
 * K must be a positive multiple of 128 (FP8Q_ERR_UNSUPPORTED otherwise), as
 * must M_pad; FP8Q_ERR_UNSUPPORTED also for G > 1024 or an operand of 2 GiB
 * or more.
 */
int fp8_grouped_gemm_e4m3(int64_t G, int64_t M_pad, int64_t N, int64_t K,
                          const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                          const int32_t* group_offsets,
                          const uint8_t* b, const float* sb,
                          uint8_t* q, int64_t ldq, float* s, int64_t lds, hipStream_t stream);

/*
 * fp8_grouped_gemm_dgrad -- MoE expert dgrad over padded groups (Ling 2.0
 * FP8 blog, "FP8 padding routing map" and "FP8 on-demand transpose weight").
 *
 * For each group e, rows [off[e], off[e+1]) of dY times expert weight W[e]
 * read as stored (no transposed copy):
 *   dX[m][k] = sum over chunks nb of 128 along n of
 *              SA(m,nb) * SW_e(nb, k/128) * sum_{n in nb} dec(dY[m][n]) * dec(W[e][n][k])
 * with the Numerics above (W[e]'s 128x128 block grid used transposed).
 *  a, lda, sa, ldsa : dY codes [M_pad][N] (contiguous groups, lda >= N), 1x128
 *                     scales along N: SA(m,nb) = sa[m*ldsa + nb], ldsa >= ceil(N/128).
 *  group_offsets    : DEVICE int32[G+1] as for fp8_grouped_gemm.
 *  w                : W codes [G][N][K], the forward weights as stored (row
 *                     stride K, K % 16 == 0).
 *  sw               : W block scales [G][ceil(N/128)][ceil(K/128)], contiguous.
 *  c, ldc, c_dtype  : dX [M_pad][K], ldc >= K.
 * M_pad must be a multiple of 128.  Rows outside [0, off[G]) are not written.
 * Returns FP8Q_ERR_UNSUPPORTED (nothing enqueued) if G > 1024 or an operand
 * spans 2 GiB or more.
 */
int fp8_grouped_gemm_dgrad(int64_t G, int64_t M_pad, int64_t N, int64_t K,
                           const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                           const int32_t* group_offsets,
                           const uint8_t* w, const float* sw,
                           void* c, int64_t ldc, int c_dtype, hipStream_t stream);

/*
 * fp8_grouped_gemm_wgrad -- MoE expert weight gradient over padded groups
 * (Ling 2.0 FP8 blog, "FP8 padding routing map" and the transposed
 * re-quantization of "grad (transpose)").
 *
 * For each group e, the sum over its tokens t in [off[e], off[e+1]) only:
 *   dW[e][n][k] = sum over chunks tb of 128 tokens of
 *                 SA(n,tb) * SB(k,tb) * sum_{t in tb} dec(dYT[n][t]) * dec(XT[k][t])
 * with the Numerics above; a group with no rows gets dW[e] = 0.  The operands
 * are the column outputs of fp8_quant_transpose on the padded dY and X, whose
 * 1x128 tiles along tokens never straddle two groups because every off[e] is
 * a multiple of 128.
 *  a, lda, sa, ldsa : dYT codes [N][M_pad] (lda >= M_pad), SA(n,tb) = sa[n*ldsa + tb],
 *                     ldsa >= M_pad/128.
 *  b, ldb, sb, ldsb : XT codes [K][M_pad] (ldb >= M_pad), SB(k,tb) = sb[k*ldsb + tb],
 *                     ldsb >= M_pad/128.
 *  group_offsets    : DEVICE int32[G+1] as for fp8_grouped_gemm.
 *  c, ldc           : fp32 dW [G][N][ldc] (group stride N*ldc elements), ldc >= K.
 * M_pad must be a multiple of 128.  Returns FP8Q_ERR_UNSUPPORTED (nothing
 * enqueued) if G > 1024 or an operand spans 2 GiB or more.
 */
int fp8_grouped_gemm_wgrad(int64_t G, int64_t M_pad, int64_t N, int64_t K,
                           const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                           const uint8_t* b, int64_t ldb, const float* sb, int64_t ldsb,
                           const int32_t* group_offsets,
                           float* c, int64_t ldc, hipStream_t stream);

/*
 * Power-of-two (E8M0) scales -- the micro-scaling variant of block scaling.
 *
 * Blackwell's MXFP8 gives each block of a tensor its own scale factor and
 * applies it in hardware (Introl FP8 infrastructure guide, scaling strategies
 * and the Blackwell section).  Here the tiles stay 1x128 / 128x128 and the
 * scale is restricted to a power of two, s = 2^e, which gfx950's scaled MFMA
 * applies itself (no scale arithmetic on the accumulators).  Per tile:
 *   e = the smallest integer >= -126 with amax <= 448 * 2^e (exactly; amax
 *       = 0 gives -126), stored as the byte e + 127 (E8M0: 2^(byte - 127));
 *   code = E4M3(RN_fp32(x / 2^e)), the quotient exact in fp32 (or below
 *       2^-126, where the code is a signed zero).  No value saturates.
 * Compared with s = amax / 448 the scale is up to 2x larger, so small values
 * underflow more easily; the product needs no scale multiplication.
 * E8M0 grids are uint8 with row stride lde in bytes; the GEMM reads each row
 * as 4-byte words, so a grid it consumes needs a 4-byte aligned pointer and
 * lde % 4 == 0 (the quantizers accept any lde >= the grid width).
 */

/*
 * fp8_quant_blockwise_e8m0 -- fp8_quant_blockwise with power-of-two scales.
 *  kind : FP8Q_ROW_1x128 (e[rows][ceil(cols/128)]) or FP8Q_BLOCK_128x128
 *         (e[ceil(rows/128)][ceil(cols/128)]); FP8Q_TENSOR is unsupported.
 *  e, lde : output E8M0 bytes, row stride lde >= ceil(cols/128).
 * Other arguments, alignment and errors as fp8_quant_blockwise.
 */
int fp8_quant_blockwise_e8m0(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                             int kind, uint8_t* q, int64_t ldq, uint8_t* e, int64_t lde,
                             hipStream_t stream);

/*
 * fp8_quant_transpose_e8m0 -- fp8_quant_transpose with power-of-two scales:
 * row tiles e_row[rows][ceil(cols/128)] and transposed column tiles
 * e_colT[cols][ceil(rows/128)] as E8M0 bytes (strides lde_row, lde_colT).
 * Other arguments and errors as fp8_quant_transpose.
 */
int fp8_quant_transpose_e8m0(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* q_row, int64_t ldq_row, uint8_t* e_row, int64_t lde_row,
                             uint8_t* q_colT, int64_t ldq_colT, uint8_t* e_colT, int64_t lde_colT,
                             hipStream_t stream);

/*
 * fp8_gemm_e8m0 -- the block-scaled product (see Numerics) with SA, SB the
 * powers of two 2^(byte - 127) of E8M0 grids.  The chunk's scales are
 * applied inside the MFMA: each chunk's product, times 2^(ea + eb), is added
 * to the fp32 accumulator.
 *  a, lda, ea, ldea : A codes [M][K]; A scales 1x128, EA(m,kb) = ea[m*ldea + kb],
 *                     ldea >= ceil(K/128).
 *  b, ldb, b_layout : as fp8_gemm_blockscaled.
 *  eb, ldeb, eb_kind: FP8Q_BLOCK_128x128 (NK: eb[(n/128)*ldeb + kb]; KN:
 *                     eb[kb*ldeb + n/128]) or FP8Q_ROW_1x128 (NK only:
 *                     eb[n*ldeb + kb]).
 *  c, ldc, c_dtype  : output [M][N], FP8Q_F32 or FP8Q_BF16.
 * ea and eb must be 4-byte aligned with ldea % 4 == ldeb % 4 == 0
 * (FP8Q_ERR_ALIGN otherwise).  Scale bytes 0 and 255 are outside the
 * contract (the quantizers write 1..247).  Large operands are sliced as for
 * fp8_gemm_blockscaled, with the same FP8Q_ERR_UNSUPPORTED cases.
 */
int fp8_gemm_e8m0(int64_t M, int64_t N, int64_t K,
                  const uint8_t* a, int64_t lda, const uint8_t* ea, int64_t ldea,
                  const uint8_t* b, int64_t ldb, int b_layout,
                  const uint8_t* eb, int64_t ldeb, int eb_kind,
                  void* c, int64_t ldc, int c_dtype, hipStream_t stream);

/*
 * fp8_adam_step -- one AdamW step with both moments held in FP8.
 *
 * Adam keeps a first and a second moment per parameter, twice the
 * parameters' memory; held as E4M3 codes with fine-grained scales they take a
 * quarter of it and barely change convergence (Ling 2.0 FP8 blog, "FP8
 * Optimizer", after block-wise quantization of optimizer states).  Here each
 * moment is a flat vector of n E4M3 codes plus one fp32 scale per 128
 * consecutive elements (the 1x128 tile rule of fp8_quant_blockwise along the
 * flat vector: s = amax / 448, see Numerics).  The step (decoupled weight
 * decay, bias-corrected moments), with every fp32 operation rounded once in
 * this order:
 *   scalars, computed in double and rounded once to fp32:
 *     b1 = beta1, b2 = beta2, omb1 = 1 - beta1, omb2 = 1 - beta2,
 *     decay = 1 - lr * weight_decay, step_size = lr / (1 - beta1^step),
 *     bc2_sqrt = sqrt(1 - beta2^step), epsf = eps;
 *   per element:  m0 = dec(mq) * ms[i/128];  v0 = dec(vq) * vs[i/128];
 *     p = p * decay;  m = b1 * m0 + omb1 * g;  v = b2 * v0 + (omb2 * g) * g;
 *     p = p - step_size * (m / (sqrt(v) / bc2_sqrt + epsf));
 *   then m and v are re-quantized (codes into mq / vq, scales into ms / vs).
 *  n        : number of parameters (any n >= 0; the last block may be short).
 *  p        : fp32 parameters [n], updated in place.
 *  g        : gradient [n], g_dtype FP8Q_F32 or FP8Q_BF16.
 *  mq, ms   : first moment: codes [n], scales [ceil(n/128)], updated in place.
 *  vq, vs   : second moment, likewise.  A fresh state is all zero bytes.
 *  step     : the step number t >= 1 (bias correction).
 * p, g, mq and vq must be 16-byte aligned, ms and vs 4-byte aligned.
 * beta1 or beta2 outside [0, 1), step < 1 or a non-finite lr, eps or
 * weight_decay: FP8Q_ERR_UNSUPPORTED.  eps = 0 with a zero second moment
 * gives NaN, as the textbook step does.
 */
int fp8_adam_step(int64_t n, float* p, const void* g, int g_dtype, uint8_t* mq, float* ms,
                  uint8_t* vq, float* vs, double lr, double beta1, double beta2, double eps,
                  double weight_decay, int64_t step, hipStream_t stream);

/* Human-readable name of a status code (static string). */
const char* fp8q_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
