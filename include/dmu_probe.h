/*
 * dmu_probe.h -- diagnostic entry points of libdmu (gfx950).
 *
 * One-instruction probes used by the test suite to pin the hardware facts the
 * GEMM kernels rely on, in the manner of the page "Tensor Cores: Matrix
 * Instructions, Swizzling and FP8, Measured" (vidyal.ai): Step 1 checks a
 * single matrix instruction against the CPU with small-integer inputs (exact
 * in the input format), and Step 5 probes how many bits the accumulator keeps
 * by adding a product of 1 to C = 2^e.  All pointers are device pointers owned
 * by the caller; calls enqueue on `stream` (a hipStream_t as void*) and return
 * without synchronising.
 */
#ifndef DMU_PROBE_H
#define DMU_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DMU_PROBE_BF16_16X16X32 0 /* v_mfma_f32_16x16x32_bf16 */
#define DMU_PROBE_BF16_32X32X16 1 /* v_mfma_f32_32x32x16_bf16 */
#define DMU_PROBE_FP8_16X16X128 2 /* v_mfma_f32_16x16x128_f8f6f4 */
#define DMU_PROBE_FP8_32X32X64 3  /* v_mfma_f32_32x32x64_f8f6f4 */
/* dmu_probe_mfma_rate only: v_mfma_scale_f32_32x32x64_f8f6f4 with E8M0 scale
 * codes 127 (x1) held in registers, the form the MX GEMM issues */
#define DMU_PROBE_MXFP8_32X32X64 4
/* dmu_probe_mfma_rate only: the same instruction on E2M1 (FP4) operands, 32
 * values in the low 16 bytes of each lane's fragment, unit E8M0 scales */
#define DMU_PROBE_MXFP4_32X32X64 5

/*
 * Run ONE matrix instruction of `kind` on a single wave: D = A * B + C with
 * A [m][k] row-major, B given as [n][k] row-major (B stored N x K), C and D
 * [m][n] row-major FP32, where (m, n, k) is the instruction's shape.  Elements
 * are BF16 bit patterns (kinds 0, 1) or FP8 codes in formats fmt_a / fmt_b
 * (0 = E4M3, 1 = E5M2; kinds 2, 3).  Fragments are loaded with the layout the
 * GEMM kernels assume (documented in probe.hip); a wrong assumption shows up
 * as a wrong D.  Returns DMU_OK or DMU_ERR_INVALID_ARG / DMU_ERR_HIP.
 */
int dmu_probe_mfma(int kind, int fmt_a, int fmt_b, const void* A, const void* B,
                   const float* C, float* D, void* stream);

/*
 * The same for `count` independent instructions in one launch (1 <= count <=
 * 2^20), one wave each: instance i reads its A and B at element offset
 * i * m * k and i * n * k (one instruction's operand: 2048 FP8 codes for
 * kinds 2 and 3, 512 BF16 values for kinds 0 and 1) and its C and D at
 * element offset i * m * n.  Used to
 * pin how one FP8 instruction forms its inner sum (which product bits it
 * keeps, where it rounds) on many random and constructed operand sets; the
 * vidyal.ai page, Step 5, probes the same property of Ada's FP8 instruction.
 * The caller sizes A, B, C and D for `count` instances (pointers 4-byte
 * aligned).  Returns DMU_OK, DMU_ERR_INVALID_ARG or DMU_ERR_HIP.
 */
int dmu_probe_mfma_batch(int kind, int fmt_a, int fmt_b, const void* A, const void* B,
                         const float* C, float* D, int count, void* stream);

/*
 * The BF16 GEMM of gemm_bf16 (B stored N x K, BF16 output, no C) with a chosen
 * LDS layout for its K slices, for the bank-conflict ablation of the vidyal.ai
 * page, Step 3 ("bank conflicts and the XOR swizzle"): layout 0 is the
 * XOR-swizzled layout every entry point uses (chunk c of 128-byte row r at
 * position c ^ ((r ^ r >> 3) & 7)), 1 plain 128-byte rows, 2 rows padded to
 * 144 bytes (the copies fill the padding position with zeros).  All three
 * compute the same product.  K % 64 == 0; other arguments as gemm_bf16.
 * Returns DMU_OK, DMU_ERR_INVALID_ARG, DMU_ERR_UNSUPPORTED or DMU_ERR_HIP.
 */
int dmu_probe_gemm_bf16_layout(int layout, const uint16_t* A, int64_t lda, const uint16_t* B,
                               int64_t ldb, void* D, int64_t ldd, int64_t M, int64_t N, int64_t K,
                               void* stream);

/*
 * Copy 64 x 16 bytes (mode 0) or 64 x 4 bytes (mode 1) from src into LDS with
 * one buffer load per lane that writes LDS directly (lane l's bytes are
 * expected at LDS offset l*size), lanes >= oob_from using an out-of-range
 * offset (expected to write zeros), after filling 2 KiB of LDS with 0xA5;
 * then write those 2 KiB of LDS to dst (2048 bytes).
 */
int dmu_probe_lds_load(const void* src, void* dst, int mode, int oob_from, void* stream);

/*
 * Sustained matrix-unit rate, the ceiling a GEMM's K loop can reach once the
 * memory pipeline is taken away (Step 2 of the same page reports each kernel
 * as a share of the peak at the clock it ran).  Launches `grid` workgroups of
 * 4 waves (one wave per SIMD); each wave runs `iters` rounds of a 4 x 4 block
 * of 32x32 MFMAs, kind DMU_PROBE_BF16_32X32X16 (32768 FLOP each),
 * DMU_PROBE_FP8_32X32X64 (E4M3 x E4M3, 131072 FLOP each) or
 * DMU_PROBE_MXFP8_32X32X64 (the same with unit E8M0 scales) or
 * DMU_PROBE_MXFP4_32X32X64 (E2M1 x E2M1, 131072 FLOP each), on operand
 * fragments read once from `src`: 8 fragments of 64 lanes x 16 bytes (BF16,
 * 8 KiB) or x 32 bytes (FP8, 16 KiB), fragments 0-3 for A and 4-7 for B.  The
 * values in `src` set the switching activity, hence the power drawn.
 * Lane l of wave w writes the sum of its 256 accumulator values to
 * out[w*64 + l] (grid * 256 floats; all-ones BF16 fragments give
 * 256 * 16 * iters, all-ones E4M3 256 * 64 * iters, with or without scales;
 * E2M1 bytes 0x22 (two ones) the same).
 * Requires 1 <= iters <= 2^20 and 1 <= grid <= 65536, else
 * DMU_ERR_INVALID_ARG.  Total work: grid * 4 * 16 * iters instructions.
 */
int dmu_probe_mfma_rate(int kind, const void* src, int iters, int grid, float* out, void* stream);

#define DMU_PROBE_MX_16X16X128 0 /* v_mfma_scale_f32_16x16x128_f8f6f4 */
#define DMU_PROBE_MX_32X32X64 1  /* v_mfma_scale_f32_32x32x64_f8f6f4 */

/*
 * Run ONE scaled matrix instruction on a single wave: the microscaling (MX)
 * product D = (A x SA)(B x SB) + C of the page "How Blackwell's Tensor Memory
 * Actually Works", section "Quantization became an allocation problem", with
 * one E8M0 scale (value 2^(code-127)) per row and 32-element run of K.
 * Shape DMU_PROBE_MX_16X16X128 (m = n = 16, k = 128) or DMU_PROBE_MX_32X32X64
 * (m = n = 32, k = 64).  A [m][k] and B [n][k] (B stored N x K) are FP8 codes
 * in fmt_a / fmt_b (0 = E4M3, 1 = E5M2), SA [m][k/32] and SB [n][k/32] are
 * E8M0 codes, C and D [m][n] row-major FP32.  Each lane puts the scale of the
 * row and K-run its fragment holds in byte `opsel` (0..3) of its scale
 * register and decoy codes (code ^ 4) in the other bytes, so a wrong layout or
 * byte selection shows up as a wrong D.  Returns DMU_OK or
 * DMU_ERR_INVALID_ARG / DMU_ERR_HIP.
 */
int dmu_probe_mfma_mx(int shape, int fmt_a, int fmt_b, int opsel, const void* A, const void* B,
                      const void* SA, const void* SB, const float* C, float* D, void* stream);

/*
 * Convert n FP32 values (n even, n <= 2^31) to FP8 codes with gfx950's
 * conversion instruction (v_cvt_pk_fp8_f32 for fmt 0 = E4M3,
 * v_cvt_pk_bf8_f32 for fmt 1 = E5M2), two values per instruction, on x as
 * given (clamp = 0) or on x clamped to +-the format's largest finite value
 * with NaN passed through (clamp = 1).  x and q
 * are device arrays of n floats / n bytes.  fmt 4 = E2M1 uses
 * v_cvt_scalef32_pk_fp4_f32 with scale 1 (clamp = 1: x clamped to +-6 first)
 * and writes the pair x[2i], x[2i+1] as byte i of q (n / 2 bytes).  Exists so
 * the tests can pin the conversion's rounding, saturation and special values
 * against the oracle.
 */
int dmu_probe_cvt_fp8(const float* x, int64_t n, int fmt, int clamp, uint8_t* q, void* stream);

/*
 * gfx950's transposing LDS read (ds_read_b64_tr_b16) on known data: src is a
 * device array of 1024 16-bit values, copied into LDS; lane l (of one wave)
 * reads with the transposing instruction at LDS byte offset offsets[l] and
 * writes the four 16-bit values it receives to out[4l .. 4l+3] (device, 256
 * values).  offsets is a HOST array of 64 byte offsets, each a multiple of 8
 * and at most 2040 (DMU_ERR_INVALID_ARG otherwise).  Exists so the tests can
 * pin the lane layout the attention kernel's V operand relies on.
 */
int dmu_probe_lds_tr16(const uint16_t* src, const uint32_t* offsets, uint16_t* out,
                       void* stream);

/*
 * Per-tensor quantize_fp8 of a contiguous rows x cols tensor (X and Q
 * row-major with no padding, scale one float) through the one-pass kernel,
 * with the bound on how many times a waiting workgroup polls for the tensor's
 * amax before it gives up and leaves its share to the last workgroup to
 * arrive.  quantize_fp8 uses a bound long enough that the fallback only runs
 * when the grid's workgroups are not all resident at once; spin_limit = 0
 * makes every waiting workgroup give up, so the tests can check that
 * fallback's codes (they must equal quantize_fp8's).  Uses the allocation-free
 * entry point's scratch, so it must not overlap such a call on the same GPU.
 * Returns DMU_ERR_UNSUPPORTED when the tensor is too large for the one-pass
 * kernel, DMU_ERR_INVALID_ARG as quantize_fp8 does or for spin_limit outside
 * [0, 65536] (quantize_fp8 itself uses 4096).
 */
int dmu_probe_quantize_tensor_resident(const float* X, int64_t rows, int64_t cols, int fmt,
                                       uint8_t* Q, float* scale, int spin_limit, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DMU_PROBE_H */
