// Host-side declarations shared between the C-ABI front end (dmu_api.cpp) and
// the kernel translation units.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dmu {

struct GemmArgs {
  const void* A;
  const void* B;
  const float* C;
  void* D;
  int64_t lda, ldb, ldc, ldd;  // elements
  int64_t M, N, K;
  const float* sa;  // FP8 scales (device)
  const float* sb;
  int out_bf16;  // 1: D is BF16, 0: FP32
  // microscaling (MX): E8M0 codes, one per row and 32 values of K (device)
  const uint8_t* xa = nullptr;
  const uint8_t* xb = nullptr;
  int64_t ldxa = 0, ldxb = 0;  // bytes per scale row
  // grouped (mixture of experts): rows goff[g] .. goff[g+1]-1 of A and D use
  // the weight at B + g * gstride (elements); every offset is clamped to
  // [0, Mmax], the rows A and D hold
  const int64_t* goff = nullptr;
  int64_t G = 0, gstride = 0, Mmax = 0;
  // fused epilogue: y = act(alpha * acc + C + bias[col]); D is FP32, BF16
  // (out_bf16) or FP8 (out_fp8 = 0 E4M3 / 1 E5M2) coded from y * out_mult[0]
  const float* bias = nullptr;
  int act = 0;       // 0 none, 1 ReLU, 2 GELU, 3 SiLU
  int out_fp8 = -1;  // -1: not FP8
  const float* out_scale = nullptr;  // FP8 out: D ~ decode(q) * out_scale[0]
};

// Attention chain, per head bh (0 <= bh < BH): O = softmax(scale * Q K^T) V,
// row i of a causal head seeing keys j <= i + Sk - Sq.  Strides in elements:
// row strides ld*, head strides h*.  lse (optional) is [BH][Sq] FP32.
struct AttnArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  uint16_t* O;
  float* lse;
  int64_t ldq, ldk, ldv, ldo;
  int64_t hq, hk, hv, ho;
  int64_t BH, Sq, Sk;
  float scale;
};

// kMX / kMX4: MXFP8, scales fetched one / four K slices at a time;
// kMXF4: MXFP4 (E2M1 x E2M1, row strides in bytes), scales two slices at a time
// kBF16G: BF16 grouped over experts (B stored N x K per expert);
// kBF16F / kFP8TensorF: BF16 / per-tensor FP8 with the fused epilogue (bias,
// activation, FP8 output), kept out of the plain kernels, whose register
// allocation its code would change
enum GemmKind { kBF16 = 0, kFP8Tensor = 1, kFP8Block = 2, kMX = 3, kMX4 = 4, kMXF4 = 5,
                kBF16G = 6, kBF16F = 7, kFP8TensorF = 8 };

// Launchers: argument checking is done by the caller; these only pick a
// kernel configuration and launch it.  They return a hipError_t.
hipError_t launch_gemm_bf16(const GemmArgs& a, int b_col_major, hipStream_t s);
// The BF16 kernel (B stored N x K, K a multiple of 64) with LDS layout 0
// (XOR-swizzled, the one every entry point uses), 1 (plain) or 2 (padded).
hipError_t launch_gemm_bf16_layout(const GemmArgs& a, int layout, hipStream_t s);
hipError_t launch_gemm_grouped_bf16(const GemmArgs& a, hipStream_t s);
hipError_t launch_attention_bf16(const AttnArgs& a, int d, int causal, hipStream_t s);
// fused epilogue (a.bias / a.act / a.out_fp8 set)
hipError_t launch_gemm_bf16_fused(const GemmArgs& a, int b_col_major, hipStream_t s);
hipError_t launch_gemm_fp8_fused(const GemmArgs& a, int fmt_a, int fmt_b, hipStream_t s);
// Skinny-M BF16 path (M <= 128, B stored N x K): HBM-bound streaming of B.
bool skinny_applies(const GemmArgs& a);
hipError_t launch_gemm_bf16_skinny(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_fp8(const GemmArgs& a, int fmt_a, int fmt_b, int block_scaled,
                           hipStream_t s);
// Per-block scaled FP8 (A 1 x 128, B 128 x 128 scales; K % 128 == 0).
hipError_t launch_gemm_fp8_block(const GemmArgs& a, int fmt_a, int fmt_b, hipStream_t s);
// MX-scaled FP8 (E8M0 scale per row and 32 K, applied by the matrix unit;
// K % 128 == 0, scale rows a multiple of 4 bytes).
hipError_t launch_gemm_mxfp8(const GemmArgs& a, int fmt_a, int fmt_b, hipStream_t s);
// MXFP4: A, B packed E2M1 (lda, ldb in bytes in GemmArgs), K % 512 == 0,
// scale rows 16-byte aligned with strides a multiple of 16 bytes.
hipError_t launch_gemm_mxfp4(const GemmArgs& a, hipStream_t s);
hipError_t launch_quantize_mxfp4(const float* X, int64_t rows, int64_t cols, int64_t ldx,
                                 uint8_t* Q, int64_t ldq_bytes, uint8_t* S, int64_t lds,
                                 hipStream_t s);
hipError_t launch_quantize_mxfp8(const float* X, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                                 uint8_t* Q, int64_t ldq, uint8_t* S, int64_t lds, hipStream_t s);
// quantize_fp8: the per-tensor mode uses a scratch of kQuantizeScratchSlots
// + kQuantizeSyncSlots words at `part`.  The two-pass walk writes one uint32
// amax partial per pass-1 workgroup to the first kQuantizeScratchSlots words
// and reads them all in the second pass; quantize_scratch_slots gives how many
// (at most 512 whatever the tensor's size; 0 for block scales, which need no
// scratch).  The one-pass kernel for tensors its grid holds in registers
// synchronises through the last kQuantizeSyncSlots words, which must be zero
// before the first call on a scratch and which every call leaves zero.
int64_t quantize_scratch_slots(int64_t rows, int64_t cols, int64_t ldx, int64_t ldq, int64_t br,
                               int64_t bc);
hipError_t launch_quantize_fp8(const float* X, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                               int64_t br, int64_t bc, uint8_t* Q, int64_t ldq, float* scales,
                               uint32_t* part, hipStream_t s);
constexpr int64_t kQuantizeScratchSlots = 1024;  // pass-1 partial slots of either scratch
constexpr int64_t kQuantizeSyncSlots = 3072;     // the one-pass kernel's words after them
constexpr int64_t kQuantizeScratchWords = kQuantizeScratchSlots + kQuantizeSyncSlots;  // 16 KiB
constexpr int kMaxDevices = 64;
// Per-tensor quantize_fp8 on the library's workspace of the stream's GPU
// (allocated on first use, calls on different streams ordered by an event).
hipError_t launch_quantize_fp8_tensor_ws(const float* X, int64_t rows, int64_t cols, int64_t ldx,
                                         int fmt, uint8_t* Q, int64_t ldq, float* scales,
                                         hipStream_t s);
// The allocation-free variant's scratch: a static device array of
// kQuantizeScratchWords words per GPU; its address on the stream's GPU
// (looked up once per device, with that device current).
hipError_t quantize_scratch_address(hipStream_t s, uint32_t** out);
// The one-pass per-tensor kernel with a chosen wait bound (diagnostic);
// hipErrorInvalidValue when the tensor does not take the one-pass kernel.
hipError_t launch_probe_quantize_resident(const float* X, int64_t rows, int64_t cols, int fmt,
                                          uint8_t* Q, float* scale, int spin_limit,
                                          hipStream_t s);

hipError_t launch_probe_mfma(int kind, int fa, int fb, const void* A, const void* B,
                             const float* C, float* D, int count, hipStream_t s);
hipError_t launch_probe_lds(const void* src, void* dst, int mode, int oob_from, hipStream_t s);
hipError_t launch_probe_rate(int kind, const void* src, int iters, int grid, float* out,
                             hipStream_t s);
hipError_t launch_probe_tr16(const uint16_t* src, const uint32_t* offsets, uint16_t* out,
                             hipStream_t s);
hipError_t launch_probe_cvt(const float* x, int64_t n, int fmt, int clamp, uint8_t* q,
                            hipStream_t s);
hipError_t launch_probe_mx(int shape, int fa, int fb, int opsel, const void* A, const void* B,
                           const void* SA, const void* SB, const float* C, float* D,
                           hipStream_t s);

}  // namespace dmu
