/*
 * dmu.h -- dense matrix-unit GEMM library for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every pointer argument is a DEVICE pointer (memory the caller
 * allocated on the GPU, e.g. a torch tensor's data_ptr()); the caller owns all
 * buffers and the library keeps no reference after a call returns.  `stream`
 * is a hipStream_t passed as void* (NULL = the default stream).  Every call
 * only validates its arguments on the host, enqueues its kernels on `stream`
 * and returns without synchronising; a nonzero status means nothing was
 * enqueued (or, for DMU_ERR_HIP, that the launch itself failed).  Faults
 * inside a kernel surface at the caller's next synchronisation.  Calls are
 * thread-safe.  Nothing is allocated except the per-tensor quantize_fp8
 * workspace (16 KiB per GPU, once); quantize_fp8_noalloc allocates nothing.
 *
 * Matrices are dense with a leading dimension counted in elements: element
 * (r, c) of a row-major matrix X lives at X[r * ldx + c].  Every pointer must
 * be 16-byte aligned and every leading dimension times the element size must
 * be a multiple of 16 bytes.
 *
 * What is computed follows the pages on tensor-core GEMMs:
 *  - "Tensor Cores: Matrix Instructions, Swizzling and FP8, Measured"
 *    (vidyal.ai), Step 1 (a matrix instruction computes D = A*B + C), Step 2
 *    (B stored N x K as PyTorch stores nn.Linear weights, BF16 inputs, FP32
 *    accumulation), Step 5 (FP8 E4M3 inputs, FP32 accumulator, promotion of
 *    partial sums to FP32 per block of K);
 *  - "Tensor Cores" chapter (ai-infra-handbooks), section "Precision: FP16,
 *    BF16, TF32, FP8" (FP16/BF16 in, FP32 accumulate; FP8 GEMMs carry
 *    per-tensor, per-row or per-block scale factors);
 *  - "Tensor cores and low precision" (learn-kernels.com), paragraphs on E4M3
 *    and E5M2 and on scaling before the cast (a tensor is scaled so that its
 *    largest values sit near 448 or 57,344, cast to FP8, and the scale is
 *    removed after the multiply).
 */
#ifndef DMU_H
#define DMU_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
#define DMU_OK 0
#define DMU_ERR_INVALID_ARG (-1) /* null pointer, bad size, alignment or enum */
#define DMU_ERR_UNSUPPORTED (-2) /* valid request this library does not implement */
#define DMU_ERR_HIP (-3)         /* the HIP runtime reported an error at launch */

/* Output element type of D. */
#define DMU_OUT_F32 0  /* IEEE binary32 */
#define DMU_OUT_BF16 1 /* bfloat16, rounded to nearest even from the FP32 result */
#define DMU_OUT_FP8_E4M3 2 /* fused entry points only: FP8 with a dequantisation scale */
#define DMU_OUT_FP8_E5M2 3
/* Activation of the fused epilogue. */
#define DMU_ACT_NONE 0
#define DMU_ACT_RELU 1 /* x > 0 ? x : 0 */
#define DMU_ACT_GELU 2 /* x * Phi(x) = x * (1 + erf(x / sqrt 2)) / 2 */
#define DMU_ACT_SILU 3 /* x / (1 + exp(-x)) */

/* Storage of the K x N operand B. */
#define DMU_B_ROW_MAJOR 0 /* B(k, n) at B[k * ldb + n] */
#define DMU_B_COL_MAJOR 1 /* B(k, n) at B[n * ldb + k]: B stored N x K ("TN") */

/* FP8 encodings (OCP 8-bit floating point). */
#define DMU_FP8_E4M3 0 /* 1/4/3 bits, bias 7, largest finite 448, no Inf, NaN = S.1111.111 */
#define DMU_FP8_E5M2 1 /* 1/5/2 bits, bias 15, largest finite 57344, IEEE Inf/NaN */

/* Scale granularity of gemm_fp8_scaled. */
#define DMU_SCALE_TENSOR 0 /* one FP32 scale per operand */
#define DMU_SCALE_BLOCK 1  /* A: one scale per 1 x 128 row segment; B: per 128 x 128 block */

/*
 * gemm_bf16: D = A * B (+ C), BF16 inputs, FP32 accumulation.
 *
 * Passages: "Tensor Cores: Matrix Instructions, Swizzling and FP8, Measured"
 * (vidyal.ai), Step 1 (a matrix instruction computes D = A*B + C with FP32
 * accumulation) and Step 2 (the whole product from such instructions, inputs
 * rounded to BF16, B stored N x K the way nn.Linear weights are); "Tensor
 * Cores" chapter (ai-infra-handbooks), section "Precision: FP16, BF16, TF32,
 * FP8" (BF16 inputs, FP32 accumulator).
 *
 *   A  : M x K BF16 (uint16 bit patterns), row-major, leading dimension lda.
 *   B  : K x N BF16, layout `b_layout` (DMU_B_ROW_MAJOR or DMU_B_COL_MAJOR),
 *        leading dimension ldb.
 *   C  : optional M x N FP32 addend, row-major, ldc (NULL = no addend).  C may
 *        be the same memory as D when d_dtype is DMU_OUT_F32 and ldc == ldd.
 *   D  : M x N output, row-major, ldd, type `d_dtype` (DMU_OUT_F32 or
 *        DMU_OUT_BF16).
 *   M, N >= 1; K >= 8 and K % 8 == 0.
 * Each D element is the FP32 sum over k of the exact products a_ik * b_kj
 * (summation order unspecified), plus C, rounded once to the output type.
 * Errors: DMU_ERR_INVALID_ARG for null A/B/D, non-positive sizes, K % 8 != 0,
 * lda < K, ldb < (row-major ? N : K), ldc/ldd < N, a misaligned pointer or
 * leading dimension, or an unknown enum value.
 */
int gemm_bf16(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int b_layout,
              const float* C, int64_t ldc, void* D, int64_t ldd, int d_dtype, int64_t M,
              int64_t N, int64_t K, void* stream);

/*
 * gemm_grouped_bf16: one launch for the experts of a mixture-of-experts layer,
 * each with its own number of rows ("How Blackwell's Tensor Memory Actually
 * Works", section "What this does to serving economics": each expert's M is
 * set by routing and changes from step to step).
 *
 *   A       : max_m x K BF16, row-major, lda; rows offsets[g] .. offsets[g+1]-1
 *             are the rows routed to expert g.
 *   B       : the experts' weights, each N x K BF16 stored N x K ("col-major"),
 *             leading dimension ldb; expert g's weight starts at B + g * stride_b
 *             (elements; stride_b >= N * ldb).
 *   offsets : DEVICE array of groups + 1 int64 row offsets, as routing writes
 *             them, read by the kernel (no host synchronisation).  Expected
 *             non-decreasing with offsets[0] >= 0 and offsets[groups] <= max_m;
 *             the kernel clamps every entry to [0, max_m] and to at least the
 *             entry before it, so no value makes it touch rows outside A or D.
 *   D       : max_m x N output, FP32 or BF16 (d_dtype), ldd.  D[r] = A[r] * B_g^T
 *             for r in expert g's range; rows outside every range are not
 *             written.
 *   groups in 1..65536; max_m >= 1 bounds the launch (max_m / 256 + groups
 *   row tiles); N >= 1; K >= 8, K % 8 == 0.
 * Accumulation and rounding are those of gemm_bf16.
 * Errors: DMU_ERR_INVALID_ARG for null pointers, sizes, strides or alignment
 * (A, B, D 16-byte aligned, offsets 8-byte aligned, stride_b * 2 a multiple
 * of 16).
 */
int gemm_grouped_bf16(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                      int64_t stride_b, const int64_t* offsets, int64_t groups, void* D,
                      int64_t ldd, int d_dtype, int64_t max_m, int64_t N, int64_t K,
                      void* stream);

/*
 * gemm_fp8_scaled: D = dequantised(A) * dequantised(B) (+ C) with FP8 inputs
 * and FP32 accumulation.
 *
 * Passages: "Tensor Cores: Matrix Instructions, Swizzling and FP8, Measured"
 * (vidyal.ai), Step 5 (E4M3 inputs, a scaled product that takes one scale per
 * operand, partial sums promoted into FP32 per block of K); "Tensor Cores"
 * chapter (ai-infra-handbooks), section "Precision: FP16, BF16, TF32, FP8"
 * (FP8 GEMMs carry per-tensor, per-row or per-block scaling factors); "Tensor
 * cores and low precision" (learn-kernels.com), opening paragraphs (the scale
 * is removed after the multiply).  gfx950's FP8 matrix instructions sum each
 * aligned group of 8 products after cutting every product toward zero to 13
 * fraction bits below the group's largest exponent-field sum, so a product
 * may lose |p| mod 2^(E - 13): the result is within the FP32-accumulation
 * bound plus those losses, not within the FP32 bound alone.
 *
 *   A       : M x K FP8 codes (format fmt_a), row-major, lda.
 *   B       : K x N operand stored N x K (column-major B), FP8 codes (fmt_b),
 *             leading dimension ldb (bytes per stored row).
 *   scale_a, scale_b : FP32 dequantisation factors (x ~ decode(code) * scale),
 *             device pointers:
 *     DMU_SCALE_TENSOR: one float each;
 *       D = (sum_k a_ik b_jk) * scale_a[0] * scale_b[0] (+ C).
 *     DMU_SCALE_BLOCK : scale_a is [M][K/128] row-major (one per 1 x 128 row
 *       segment of A), scale_b is [ceil(N/128)][K/128] row-major (one per
 *       128 x 128 block of the stored N x K matrix);
 *       D = sum_kb scale_a[i][kb] * scale_b[j/128][kb] * (sum_{k in kb} a_ik b_jk)
 *       (+ C): every 128-wide partial sum is formed from zero in the matrix
 *       unit and then promoted into the FP32 accumulator with its scales.
 *   C, D    : as for gemm_bf16.
 *   M, N >= 1; K % 16 == 0 (DMU_SCALE_TENSOR) or K % 128 == 0 (DMU_SCALE_BLOCK).
 * Errors: DMU_ERR_INVALID_ARG as for gemm_bf16, plus null scales or an
 * unknown format / scale mode.
 */
int gemm_fp8_scaled(const uint8_t* A, int64_t lda, int fmt_a, const uint8_t* B, int64_t ldb,
                    int fmt_b, const float* scale_a, const float* scale_b, int scale_mode,
                    const float* C, int64_t ldc, void* D, int64_t ldd, int d_dtype, int64_t M,
                    int64_t N, int64_t K, void* stream);

/*
 * quantize_fp8: FP32 -> FP8 with one scale per block.
 *
 * Passages: "Tensor cores and low precision" (learn-kernels.com), opening
 * paragraphs (E4M3 reaches 448 and has no infinity, E5M2 reaches 57,344; a
 * tensor is scaled so that its largest values sit near that maximum, cast,
 * and the scale is removed after the multiply); "Tensor Cores" chapter
 * (ai-infra-handbooks), section "Precision: FP16, BF16, TF32, FP8" (the 1/4/3
 * and 1/5/2 bit splits; per-tensor, per-row and per-block scaling factors).
 * Saturation and round-to-nearest-even are this library's reading of how the
 * cast treats values past the maximum and between codes.
 *
 *   X      : rows x cols FP32, row-major, ldx.
 *   fmt    : DMU_FP8_E4M3 (FMAX = 448) or DMU_FP8_E5M2 (FMAX = 57344).
 *   block_rows x block_cols : the scaling block.  Supported: (rows, cols) =
 *            one per-tensor scale; (1, 128) = per row segment; (128, 128).
 *            rows % block_rows == 0 and cols % block_cols == 0.
 *   Q      : rows x cols FP8 codes, row-major, ldq.
 *   scales : [rows/block_rows][cols/block_cols] FP32, row-major.
 * For each block: amax = max |x|; m = FMAX / amax and s = amax / FMAX, both
 * IEEE FP32 divisions; q = saturating round-to-nearest-even FP8 encoding of the
 * FP32 product x * m (magnitudes >= FMAX, Inf included, become +-FMAX; FP8
 * subnormals are kept; -0 stays -0); the stored scale is s, the factor that
 * dequantises (x ~ decode(q) * s), which is what gemm_fp8_scaled takes.
 * An all-zero block gets m = s = 1.  A block holding a NaN gets amax = NaN
 * (scale NaN, codes NaN); one holding an Inf and no NaN gets amax = +Inf
 * (scale +Inf, finite inputs encode to +-0, infinite ones to NaN).  The result
 * is bit-exact and independent of launch configuration.
 * The per-tensor mode reads a contiguous tensor (ldx == ldq == cols) of up to
 * 16384 values per compute unit once, with one kernel whose workgroups keep
 * their share in registers and exchange their amax partials through the
 * workspace; larger or strided tensors take two passes (per-workgroup amax
 * partials, then the encode).  The workspace (16 KiB: partial slots and the
 * one-pass kernel's counters) is allocated and zeroed by the library once per
 * GPU, at the first per-tensor call on it, and kept until the process ends;
 * each call makes its stream wait for the previous per-tensor call on that
 * GPU (an event), so calls on different streams never share it concurrently.
 * Block scales need no workspace.
 * Errors: DMU_ERR_INVALID_ARG for null pointers, bad sizes, leading dimensions
 * or alignment, an unknown format; DMU_ERR_UNSUPPORTED for other block shapes;
 * DMU_ERR_HIP if the workspace cannot be allocated or a launch fails.
 * Per-tensor calls on one GPU are ordered with each other across streams.
 */
int quantize_fp8(const float* X, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                 int64_t block_rows, int64_t block_cols, uint8_t* Q, int64_t ldq, float* scales,
                 void* stream);

/*
 * quantize_fp8_noalloc: quantize_fp8 for callers that cannot allocate device
 * memory -- code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, results and errors as quantize_fp8
 * (bit-identical output), but the per-tensor mode's amax partials and the
 * one-pass kernel's counters go to a static scratch array inside the library
 * (16 KiB per GPU: 1024 partial slots and 3072 counter words, zero when the
 * library loads, held until the process ends) instead of an allocated
 * workspace: the call allocates nothing.  Limit: a call needing more partial
 * slots than the scratch holds returns DMU_ERR_UNSUPPORTED; the per-tensor
 * passes use at most 512 slots whatever the tensor's size, so no valid tensor
 * is refused.  Every call on one GPU shares that GPU's scratch: calls that
 * overlap on one GPU (concurrent streams) race and must be serialised by the
 * caller.  A race can also leave the one-pass kernel's counters inconsistent,
 * after which per-tensor results of later calls on that GPU are undefined as
 * well.  Block scales use no scratch.
 */
int quantize_fp8_noalloc(const float* X, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                         int64_t block_rows, int64_t block_cols, uint8_t* Q, int64_t ldq,
                         float* scales, void* stream);

/*
 * Microscaling (MX) FP8: block-scaled operands with one power-of-two scale per
 * row and 32 consecutive values of K, the product D = C + (A x SFA)(B x SFB)
 * of "How Blackwell's Tensor Memory Actually Works", section "Quantization
 * became an allocation problem" (block-scaled MMA, one scale per 32 values,
 * E8M0 scales).  An E8M0 code c is the value 2^(c - 127); c = 255 is NaN.
 */
#define DMU_MX_BLOCK 32

/*
 * gemm_mxfp8: D = sum_k (a_ik * 2^(sa_i,k/32 - 127)) * (b_jk * 2^(sb_j,k/32 - 127))
 * (+ C), FP8 inputs, FP32 accumulation; the matrix unit applies the scales.
 *
 *   A       : M x K FP8 codes (fmt_a), row-major, lda.
 *   B       : K x N operand stored N x K (column-major B), FP8 codes (fmt_b), ldb.
 *   scale_a : M x (K/32) E8M0 codes, row-major with ld_sa bytes per row.
 *   scale_b : N x (K/32) E8M0 codes (one per stored row of B and 32 K), ld_sb.
 *   C, D    : as for gemm_bf16.
 *   M, N >= 1; K >= 128 and K % 128 == 0; ld_sa, ld_sb >= K/32 and multiples
 *   of 4; scale pointers 4-byte aligned.
 * Each 64-wide run of K is one matrix instruction whose inner sum is formed at
 * the instruction's own precision (about 14 bits below its largest term, as
 * for per-tensor FP8) and added into the FP32 accumulator.  A NaN code makes
 * every output that uses it NaN.  Scaled products below FP32 range flush to
 * zero; a 32-wide group whose scaled sum exceeds FP32 range makes the output
 * non-finite (Inf of unspecified sign, or NaN), whatever the exact sum.
 * Errors: DMU_ERR_INVALID_ARG as for gemm_fp8_scaled, plus K % 128 != 0, a
 * null scale array, a short or misaligned scale row stride.
 */
int gemm_mxfp8(const uint8_t* A, int64_t lda, int fmt_a, const uint8_t* B, int64_t ldb,
               int fmt_b, const uint8_t* scale_a, int64_t ld_sa, const uint8_t* scale_b,
               int64_t ld_sb, const float* C, int64_t ldc, void* D, int64_t ldd, int d_dtype,
               int64_t M, int64_t N, int64_t K, void* stream);

/*
 * quantize_mxfp8: FP32 -> FP8 with one E8M0 scale per 1 x 32 block.
 *
 *   X      : rows x cols FP32, row-major, ldx; cols % 32 == 0.
 *   fmt    : DMU_FP8_E4M3 (emax = 8) or DMU_FP8_E5M2 (emax = 15), the exponent
 *            of the format's largest power of two.
 *   Q      : rows x cols FP8 codes, row-major, ldq.
 *   S      : rows x (cols/32) E8M0 codes, row-major, lds bytes per row.
 * For each block: amax = max |x|; the scale is X = 2^(floor(log2 amax) - emax)
 * with the exponent clamped to [-127, 127] (the Open Compute microscaling
 * choice: the block's largest value lands in [2^emax, 2^(emax+1))), stored as
 * code floor(log2 amax) - emax + 127; every element is the saturating
 * round-to-nearest-even FP8 code of x / X (so x ~ decode(q) * X, what
 * gemm_mxfp8 takes).  An all-zero block gets code 0; a block holding NaN or
 * Inf gets code 255 and every element the NaN code of its own sign.  The
 * result is bit-exact and independent of launch configuration.
 * Errors: DMU_ERR_INVALID_ARG for null pointers, cols % 32 != 0, short or
 * misaligned leading dimensions, an unknown format.
 */
int quantize_mxfp8(const float* X, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* Q,
                   int64_t ldq, uint8_t* S, int64_t lds, void* stream);

/*
 * MXFP4: the same microscaled product with E2M1 elements (FP4: sign, 2
 * exponent bits with bias 1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3,
 * 4, 6; no Inf or NaN), the MXFP4 format [TM]'s section names beside MXFP8.
 * Elements are packed two per byte, element 2i in the low nibble of byte i of
 * the row.  Leading dimensions of packed arrays count elements (bytes x 2).
 */
#define DMU_FP4_E2M1 4

/*
 * gemm_mxfp4: D = sum_k (a_ik * 2^(sa_i,k/32 - 127)) * (b_jk * 2^(sb_j,k/32 - 127))
 * (+ C), E2M1 x E2M1 inputs, FP32 accumulation; the matrix unit applies the
 * scales.
 *
 *   A       : M x K E2M1 packed, row-major, lda elements (lda % 32 == 0).
 *   B       : K x N operand stored N x K, E2M1 packed, ldb elements (% 32 == 0).
 *   scale_a : M x (K/32) E8M0 codes, ld_sa bytes per row; scale_b : N x (K/32).
 *   C, D    : as for gemm_bf16.
 *   M, N >= 1; K >= 512 and K % 512 == 0; ld_sa, ld_sb >= K/32 and multiples
 *   of 16; A, B, scale_a, scale_b 16-byte aligned.
 * Accumulation and special values behave as for gemm_mxfp8.
 * Errors: DMU_ERR_INVALID_ARG for null pointers, sizes, strides or alignment
 * outside the above, an unknown output type.
 */
int gemm_mxfp4(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
               const uint8_t* scale_a, int64_t ld_sa, const uint8_t* scale_b, int64_t ld_sb,
               const float* C, int64_t ldc, void* D, int64_t ldd, int d_dtype, int64_t M,
               int64_t N, int64_t K, void* stream);

/*
 * quantize_mxfp4: FP32 -> E2M1 with one E8M0 scale per 1 x 32 block, as
 * quantize_mxfp8 with emax = 2 (the scale puts each block's largest value in
 * [4, 8)): q = saturating round-to-nearest-even E2M1 of x / X, ties to the even
 * code.  Q is rows x cols packed (ldq elements, a multiple of 32); S as for
 * quantize_mxfp8.  A block holding NaN or Inf gets code 255 and signed-zero
 * elements.  Bit-exact and independent of launch configuration.
 * Errors: DMU_ERR_INVALID_ARG for null pointers, cols % 32 != 0, short or
 * misaligned leading dimensions.
 */
int quantize_mxfp4(const float* X, int64_t rows, int64_t cols, int64_t ldx, uint8_t* Q,
                   int64_t ldq, uint8_t* S, int64_t lds, void* stream);

/*
 * Fused epilogue: the accumulator is turned into the layer's output while it
 * is still in registers -- scaled, biased, activated and cast down ("How
 * Blackwell's Tensor Memory Actually Works", section "The cost of getting the
 * answer back") -- instead of a second pass over D in HBM:
 *
 *   y[i][j] = act(alpha * acc[i][j] + bias[j])
 *
 * with acc the FP32 sum of the products, alpha = 1 (BF16) or
 * scale_a[0] * scale_b[0] (per-tensor FP8), bias an optional FP32 vector of N
 * (NULL: none) and act a DMU_ACT_* value evaluated in FP32 on the hardware
 * exp2 and reciprocal: SiLU directly, GELU with Phi from the erf
 * approximation of Abramowitz & Stegun formula 7.1.26 (absolute error at
 * most 1.5e-7, so GELU within 7.5e-8 |x| of x Phi(x)).  D receives y as FP32, as BF16 (RNE), or as
 * FP8 (DMU_OUT_FP8_*): q = saturating round-to-nearest-even of fl32(y * m),
 * m = fl32(1 / d_scale[0]) -- the quantize_fp8 convention (computed with the
 * hardware conversion after clamping to +-max, bit-exact with that encoder), so that
 * y ~ decode(q) * d_scale[0] and D can feed gemm_fp8_scaled directly.
 * d_scale is a device pointer to one float, required for FP8 output and
 * ignored otherwise.  FP8 output rows are ldd bytes apart (ldd % 16 == 0).
 * bias and d_scale are device pointers aligned to 4 bytes, read only; the
 * caller keeps ownership of every buffer.  An act or d_dtype outside the
 * values above, a missing d_scale for FP8 output, or a misaligned pointer
 * returns DMU_ERR_INVALID_ARG before anything is launched; the remaining
 * checks are those of the plain entry point.  With no bias, no activation
 * and no FP8 output the plain kernels run.
 */

/* gemm_bf16_fused: gemm_bf16 (no C addend) with the fused epilogue. */
int gemm_bf16_fused(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                    int b_layout, const float* bias, int act, void* D, int64_t ldd,
                    int d_dtype, const float* d_scale, int64_t M, int64_t N, int64_t K,
                    void* stream);

/* gemm_fp8_fused: per-tensor gemm_fp8_scaled (no C addend) with the fused
 * epilogue. */
int gemm_fp8_fused(const uint8_t* A, int64_t lda, int fmt_a, const uint8_t* B, int64_t ldb,
                   int fmt_b, const float* scale_a, const float* scale_b, const float* bias,
                   int act, void* D, int64_t ldd, int d_dtype, const float* d_scale, int64_t M,
                   int64_t N, int64_t K, void* stream);

/*
 * attention_bf16: two products chained through a row-wise softmax, the
 * scores never written to memory -- the chain the "Tensor Cores" chapter
 * (ai-infra-handbooks), section "mma.sync: the register layout is explicit",
 * names as FlashAttention's (one product's output worked on in registers and
 * fed to the next).  For each head bh < heads and query row i < Sq:
 *
 *   s_j    = scale * sum_k Q[i][k] K[j][k]            (FP32 accumulation)
 *   O[i]   = sum_j exp(s_j - max s) V[j] / sum_j exp(s_j - max s)
 *   lse[i] = log sum_j exp(s_j)
 *
 * over the keys j the row sees: all Sk of them, or with causal = 1 the keys
 * j <= i + (Sk - Sq) (the last query row sees every key; requires Sq <= Sk).
 * The softmax is taken online over blocks of keys: the weights are computed
 * in FP32 (hardware exp2), rounded to BF16 for the second product, which
 * accumulates in FP32; the row sum uses the FP32 weights.  O is rounded to
 * BF16 once at the end.
 *
 *   Q : heads x Sq x d BF16, row i of head bh at Q + bh*head_stride_q + i*ldq
 *   K, V : heads x Sk x d BF16, likewise (ldk, head_stride_k, ldv, head_stride_v)
 *   O : heads x Sq x d BF16 output, likewise (ldo, head_stride_o); must not
 *       overlap Q, K or V; with heads > 1 the heads' outputs must not
 *       overlap: head_stride_o >= (Sq - 1) * ldo + d (heads one after
 *       another) or head_stride_o >= d and ldo >= (heads - 1) * head_stride_o
 *       + d (heads side by side within each row, [Sq][heads][d] storage)
 *   lse : optional heads x Sq FP32 output (NULL: not written), natural log
 *   d = 64 or 128; scale > 0 and finite (typically 1 / sqrt(d)).
 * Scores must stay finite in FP32.  All pointers are device pointers owned by
 * the caller; Q, K, V, O 16-byte aligned, row and head strides multiples of
 * 8 elements, row strides >= d.
 * Errors: DMU_ERR_INVALID_ARG for a null or misaligned pointer, d not 64 or
 * 128, non-positive sizes, causal with Sq > Sk, a bad stride (including an
 * output head stride that makes heads overlap) or scale;
 * DMU_ERR_UNSUPPORTED when one head spans 2^31 bytes or more.
 */
int attention_bf16(const uint16_t* Q, int64_t ldq, int64_t head_stride_q, const uint16_t* K,
                   int64_t ldk, int64_t head_stride_k, const uint16_t* V, int64_t ldv,
                   int64_t head_stride_v, uint16_t* O, int64_t ldo, int64_t head_stride_o,
                   float* lse, int64_t heads, int64_t Sq, int64_t Sk, int64_t d, float scale,
                   int causal, void* stream);

/* Human-readable text for a status code (static storage, never NULL). */
const char* dmu_status_string(int status);

/* Library ABI version: (major << 16) | minor. */
int dmu_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DMU_H */
