// C-ABI front end of libdmu: argument validation and kernel dispatch.
// Semantics and error behaviour of each entry point are documented in
// include/dmu.h and include/dmu_probe.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/dmu.h"
#include "../../include/dmu_probe.h"
#include "dmu_internal.h"

namespace {

constexpr int64_t kMaxTileBytes = (int64_t)1 << 31;  // 32-bit buffer offsets inside a tile
constexpr int kTileRows = 256;                        // largest workgroup tile edge

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int finish(hipError_t e) { return e == hipSuccess ? DMU_OK : DMU_ERR_HIP; }

// Common checks of D = A*B (+C): sizes, output type, C and D.
int check_out(const float* C, int64_t ldc, const void* D, int64_t ldd, int d_dtype, int64_t M,
              int64_t N) {
  if (!D || M < 1 || N < 1 || M > INT32_MAX || N > INT32_MAX) return DMU_ERR_INVALID_ARG;
  if (d_dtype != DMU_OUT_F32 && d_dtype != DMU_OUT_BF16) return DMU_ERR_INVALID_ARG;
  const int64_t osz = d_dtype == DMU_OUT_F32 ? 4 : 2;
  if (ldd < N || !aligned(D, 16) || (ldd * osz) % 16) return DMU_ERR_INVALID_ARG;
  if (C) {
    if (ldc < N || !aligned(C, 16) || (ldc * 4) % 16) return DMU_ERR_INVALID_ARG;
    if ((const void*)C == D && (d_dtype != DMU_OUT_F32 || ldc != ldd)) return DMU_ERR_INVALID_ARG;
  }
  return DMU_OK;
}

}  // namespace

extern "C" {

int gemm_bf16(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int b_layout,
              const float* C, int64_t ldc, void* D, int64_t ldd, int d_dtype, int64_t M,
              int64_t N, int64_t K, void* stream) {
  int rc = check_out(C, ldc, D, ldd, d_dtype, M, N);
  if (rc) return rc;
  if (!A || !B || K < 8 || K % 8 || K > INT32_MAX) return DMU_ERR_INVALID_ARG;
  if (b_layout != DMU_B_ROW_MAJOR && b_layout != DMU_B_COL_MAJOR) return DMU_ERR_INVALID_ARG;
  if (lda < K || (lda * 2) % 16 || !aligned(A, 16) || !aligned(B, 16)) return DMU_ERR_INVALID_ARG;
  if (b_layout == DMU_B_ROW_MAJOR ? ldb < N : ldb < K) return DMU_ERR_INVALID_ARG;
  if ((ldb * 2) % 16) return DMU_ERR_INVALID_ARG;
  if (kTileRows * lda * 2 >= kMaxTileBytes) return DMU_ERR_UNSUPPORTED;
  if (b_layout == DMU_B_COL_MAJOR ? kTileRows * ldb * 2 >= kMaxTileBytes
                                  : K * ldb * 2 >= kMaxTileBytes)
    return DMU_ERR_UNSUPPORTED;
  dmu::GemmArgs a{A, B, C, D, lda, ldb, ldc, ldd, M, N, K, nullptr, nullptr,
                  d_dtype == DMU_OUT_BF16};
  (void)hipGetLastError();
  return finish(dmu::launch_gemm_bf16(a, b_layout == DMU_B_COL_MAJOR, (hipStream_t)stream));
}

int gemm_grouped_bf16(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                      int64_t stride_b, const int64_t* offsets, int64_t groups, void* D,
                      int64_t ldd, int d_dtype, int64_t max_m, int64_t N, int64_t K,
                      void* stream) {
  int rc = check_out(nullptr, 0, D, ldd, d_dtype, max_m, N);
  if (rc) return rc;
  if (!A || !B || !offsets || groups < 1 || groups > 65536) return DMU_ERR_INVALID_ARG;
  if (K < 8 || K % 8 || K > INT32_MAX) return DMU_ERR_INVALID_ARG;
  if (lda < K || ldb < K || (lda * 2) % 16 || (ldb * 2) % 16) return DMU_ERR_INVALID_ARG;
  if (stride_b < N * ldb || (stride_b * 2) % 16) return DMU_ERR_INVALID_ARG;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(offsets, 8)) return DMU_ERR_INVALID_ARG;
  if (kTileRows * lda * 2 >= kMaxTileBytes || kTileRows * ldb * 2 >= kMaxTileBytes)
    return DMU_ERR_UNSUPPORTED;
  dmu::GemmArgs a{A, B, nullptr, D, lda, ldb, 0, ldd, max_m, N, K, nullptr, nullptr,
                  d_dtype == DMU_OUT_BF16};
  a.goff = offsets;
  a.G = groups;
  a.gstride = stride_b;
  a.Mmax = max_m;
  (void)hipGetLastError();
  return finish(dmu::launch_gemm_grouped_bf16(a, (hipStream_t)stream));
}

int attention_bf16(const uint16_t* Q, int64_t ldq, int64_t head_stride_q, const uint16_t* K,
                   int64_t ldk, int64_t head_stride_k, const uint16_t* V, int64_t ldv,
                   int64_t head_stride_v, uint16_t* O, int64_t ldo, int64_t head_stride_o,
                   float* lse, int64_t heads, int64_t Sq, int64_t Sk, int64_t d, float scale,
                   int causal, void* stream) {
  if (!Q || !K || !V || !O) return DMU_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return DMU_ERR_INVALID_ARG;
  if (heads < 1 || Sq < 1 || Sk < 1 || (causal != 0 && causal != 1)) return DMU_ERR_INVALID_ARG;
  if (causal && Sq > Sk) return DMU_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || !(scale < INFINITY)) return DMU_ERR_INVALID_ARG;
  const int64_t ld[4] = {ldq, ldk, ldv, ldo};
  const int64_t hs[4] = {head_stride_q, head_stride_k, head_stride_v, head_stride_o};
  for (int t = 0; t < 4; ++t)
    if (ld[t] < d || (ld[t] * 2) % 16 || hs[t] < 0 || (hs[t] * 2) % 16) return DMU_ERR_INVALID_ARG;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) ||
      (lse && !aligned(lse, 4)))
    return DMU_ERR_INVALID_ARG;
  // the heads' outputs must be disjoint, or workgroups of different heads
  // would store to the same O elements: heads one after another
  // ([heads][Sq][d]-like) or side by side within each row stride
  // ([Sq][heads][d]-like)
  if (heads > 1) {
    const bool stacked = head_stride_o >= (Sq - 1) * ldo + d;
    const bool side_by_side = head_stride_o >= d && ldo >= (heads - 1) * head_stride_o + d;
    if (!stacked && !side_by_side) return DMU_ERR_INVALID_ARG;
  }
  // one head's rows are addressed with 32-bit byte offsets
  if (Sq * ldq * 2 >= kMaxTileBytes || Sk * ldk * 2 >= kMaxTileBytes ||
      Sk * ldv * 2 >= kMaxTileBytes || ((Sq + 127) / 128) * heads > INT32_MAX)
    return DMU_ERR_UNSUPPORTED;
  dmu::AttnArgs a{Q,     K,     V,     O,  lse, ldq, ldk, ldv, ldo, head_stride_q, head_stride_k,
                  head_stride_v, head_stride_o, heads, Sq, Sk, scale};
  (void)hipGetLastError();
  return finish(dmu::launch_attention_bf16(a, (int)d, causal, (hipStream_t)stream));
}

int gemm_fp8_scaled(const uint8_t* A, int64_t lda, int fmt_a, const uint8_t* B, int64_t ldb,
                    int fmt_b, const float* scale_a, const float* scale_b, int scale_mode,
                    const float* C, int64_t ldc, void* D, int64_t ldd, int d_dtype, int64_t M,
                    int64_t N, int64_t K, void* stream) {
  int rc = check_out(C, ldc, D, ldd, d_dtype, M, N);
  if (rc) return rc;
  if (!A || !B || !scale_a || !scale_b) return DMU_ERR_INVALID_ARG;
  if (fmt_a != DMU_FP8_E4M3 && fmt_a != DMU_FP8_E5M2) return DMU_ERR_INVALID_ARG;
  if (fmt_b != DMU_FP8_E4M3 && fmt_b != DMU_FP8_E5M2) return DMU_ERR_INVALID_ARG;
  if (scale_mode != DMU_SCALE_TENSOR && scale_mode != DMU_SCALE_BLOCK) return DMU_ERR_INVALID_ARG;
  if (K < 16 || K > INT32_MAX || K % (scale_mode == DMU_SCALE_BLOCK ? 128 : 16))
    return DMU_ERR_INVALID_ARG;
  if (lda < K || ldb < K || lda % 16 || ldb % 16) return DMU_ERR_INVALID_ARG;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(scale_a, 4) || !aligned(scale_b, 4))
    return DMU_ERR_INVALID_ARG;
  if (kTileRows * lda >= kMaxTileBytes || kTileRows * ldb >= kMaxTileBytes)
    return DMU_ERR_UNSUPPORTED;
  if (scale_mode == DMU_SCALE_BLOCK && kTileRows * (K / 128) * 4 >= kMaxTileBytes)
    return DMU_ERR_UNSUPPORTED;
  dmu::GemmArgs a{A, B, C, D, lda, ldb, ldc, ldd, M, N, K, scale_a, scale_b,
                  d_dtype == DMU_OUT_BF16};
  (void)hipGetLastError();
  return finish(dmu::launch_gemm_fp8(a, fmt_a, fmt_b, scale_mode == DMU_SCALE_BLOCK,
                                     (hipStream_t)stream));
}

namespace {

// Checks shared by quantize_fp8 and quantize_fp8_noalloc.
int quantize_args(const float* X, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                  int64_t block_rows, int64_t block_cols, const uint8_t* Q, int64_t ldq,
                  const float* scales) {
  if (!X || !Q || !scales || rows < 1 || cols < 1) return DMU_ERR_INVALID_ARG;
  if (fmt != DMU_FP8_E4M3 && fmt != DMU_FP8_E5M2) return DMU_ERR_INVALID_ARG;
  if (ldx < cols || ldq < cols || ldx % 4 || ldq % 16) return DMU_ERR_INVALID_ARG;
  if (!aligned(X, 16) || !aligned(Q, 16) || !aligned(scales, 4)) return DMU_ERR_INVALID_ARG;
  if (block_rows < 1 || block_cols < 1 || rows % block_rows || cols % block_cols)
    return DMU_ERR_INVALID_ARG;
  const bool tensor = block_rows == rows && block_cols == cols;
  const bool row128 = block_rows == 1 && block_cols == 128;
  const bool blk128 = block_rows == 128 && block_cols == 128;
  if (!tensor && !row128 && !blk128) return DMU_ERR_UNSUPPORTED;
  if (tensor && cols % 4) return DMU_ERR_UNSUPPORTED;
  if ((rows / block_rows) * (cols / block_cols) > INT32_MAX) return DMU_ERR_UNSUPPORTED;
  return DMU_OK;
}

}  // namespace

int quantize_fp8(const float* X, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                 int64_t block_rows, int64_t block_cols, uint8_t* Q, int64_t ldq, float* scales,
                 void* stream) {
  int rc = quantize_args(X, rows, cols, ldx, fmt, block_rows, block_cols, Q, ldq, scales);
  if (rc) return rc;
  const int64_t slots = dmu::quantize_scratch_slots(rows, cols, ldx, ldq, block_rows, block_cols);
  if (slots > dmu::kQuantizeScratchSlots) return DMU_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  hipStream_t s = (hipStream_t)stream;
  if (slots > 0)  // per tensor: the library's workspace on the stream's GPU
    return finish(dmu::launch_quantize_fp8_tensor_ws(X, rows, cols, ldx, fmt, Q, ldq, scales, s));
  return finish(dmu::launch_quantize_fp8(X, rows, cols, ldx, fmt, block_rows, block_cols, Q, ldq,
                                         scales, nullptr, s));
}

int quantize_fp8_noalloc(const float* X, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                         int64_t block_rows, int64_t block_cols, uint8_t* Q, int64_t ldq,
                         float* scales, void* stream) {
  int rc = quantize_args(X, rows, cols, ldx, fmt, block_rows, block_cols, Q, ldq, scales);
  if (rc) return rc;
  const int64_t slots = dmu::quantize_scratch_slots(rows, cols, ldx, ldq, block_rows, block_cols);
  if (slots > dmu::kQuantizeScratchSlots) return DMU_ERR_UNSUPPORTED;  // beyond the static scratch
  (void)hipGetLastError();
  hipStream_t s = (hipStream_t)stream;
  uint32_t* part = nullptr;
  if (slots > 0 && dmu::quantize_scratch_address(s, &part) != hipSuccess) return DMU_ERR_HIP;
  return finish(dmu::launch_quantize_fp8(X, rows, cols, ldx, fmt, block_rows, block_cols, Q, ldq,
                                         scales, part, s));
}

int gemm_mxfp8(const uint8_t* A, int64_t lda, int fmt_a, const uint8_t* B, int64_t ldb,
               int fmt_b, const uint8_t* scale_a, int64_t ld_sa, const uint8_t* scale_b,
               int64_t ld_sb, const float* C, int64_t ldc, void* D, int64_t ldd, int d_dtype,
               int64_t M, int64_t N, int64_t K, void* stream) {
  int rc = check_out(C, ldc, D, ldd, d_dtype, M, N);
  if (rc) return rc;
  if (!A || !B || !scale_a || !scale_b) return DMU_ERR_INVALID_ARG;
  if (fmt_a != DMU_FP8_E4M3 && fmt_a != DMU_FP8_E5M2) return DMU_ERR_INVALID_ARG;
  if (fmt_b != DMU_FP8_E4M3 && fmt_b != DMU_FP8_E5M2) return DMU_ERR_INVALID_ARG;
  if (K < 128 || K > INT32_MAX || K % 128) return DMU_ERR_INVALID_ARG;
  if (lda < K || ldb < K || lda % 16 || ldb % 16) return DMU_ERR_INVALID_ARG;
  if (ld_sa < K / DMU_MX_BLOCK || ld_sb < K / DMU_MX_BLOCK || ld_sa % 4 || ld_sb % 4)
    return DMU_ERR_INVALID_ARG;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(scale_a, 4) || !aligned(scale_b, 4))
    return DMU_ERR_INVALID_ARG;
  if (kTileRows * lda >= kMaxTileBytes || kTileRows * ldb >= kMaxTileBytes ||
      kTileRows * ld_sa >= kMaxTileBytes || kTileRows * ld_sb >= kMaxTileBytes)
    return DMU_ERR_UNSUPPORTED;
  dmu::GemmArgs a{A, B, C, D, lda, ldb, ldc, ldd, M, N, K, nullptr, nullptr,
                  d_dtype == DMU_OUT_BF16};
  a.xa = scale_a;
  a.xb = scale_b;
  a.ldxa = ld_sa;
  a.ldxb = ld_sb;
  (void)hipGetLastError();
  return finish(dmu::launch_gemm_mxfp8(a, fmt_a, fmt_b, (hipStream_t)stream));
}

int quantize_mxfp8(const float* X, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* Q,
                   int64_t ldq, uint8_t* S, int64_t lds, void* stream) {
  if (!X || !Q || !S || rows < 1 || cols < DMU_MX_BLOCK || cols % DMU_MX_BLOCK)
    return DMU_ERR_INVALID_ARG;
  if (fmt != DMU_FP8_E4M3 && fmt != DMU_FP8_E5M2) return DMU_ERR_INVALID_ARG;
  if (ldx < cols || ldq < cols || lds < cols / DMU_MX_BLOCK || ldx % 4 || ldq % 16)
    return DMU_ERR_INVALID_ARG;
  if (!aligned(X, 16) || !aligned(Q, 16)) return DMU_ERR_INVALID_ARG;
  if (rows * (cols / DMU_MX_BLOCK) > INT32_MAX) return DMU_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  return finish(
      dmu::launch_quantize_mxfp8(X, rows, cols, ldx, fmt, Q, ldq, S, lds, (hipStream_t)stream));
}

int gemm_mxfp4(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
               const uint8_t* scale_a, int64_t ld_sa, const uint8_t* scale_b, int64_t ld_sb,
               const float* C, int64_t ldc, void* D, int64_t ldd, int d_dtype, int64_t M,
               int64_t N, int64_t K, void* stream) {
  int rc = check_out(C, ldc, D, ldd, d_dtype, M, N);
  if (rc) return rc;
  if (!A || !B || !scale_a || !scale_b) return DMU_ERR_INVALID_ARG;
  if (K < 512 || K > INT32_MAX || K % 512) return DMU_ERR_INVALID_ARG;
  if (lda < K || ldb < K || lda % 32 || ldb % 32) return DMU_ERR_INVALID_ARG;
  if (ld_sa < K / DMU_MX_BLOCK || ld_sb < K / DMU_MX_BLOCK || ld_sa % 16 || ld_sb % 16)
    return DMU_ERR_INVALID_ARG;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(scale_a, 16) || !aligned(scale_b, 16))
    return DMU_ERR_INVALID_ARG;
  if (kTileRows * (lda / 2) >= kMaxTileBytes || kTileRows * (ldb / 2) >= kMaxTileBytes ||
      kTileRows * ld_sa >= kMaxTileBytes || kTileRows * ld_sb >= kMaxTileBytes)
    return DMU_ERR_UNSUPPORTED;
  // the kernel addresses packed rows in bytes
  dmu::GemmArgs a{A, B, C, D, lda / 2, ldb / 2, ldc, ldd, M, N, K, nullptr, nullptr,
                  d_dtype == DMU_OUT_BF16};
  a.xa = scale_a;
  a.xb = scale_b;
  a.ldxa = ld_sa;
  a.ldxb = ld_sb;
  (void)hipGetLastError();
  return finish(dmu::launch_gemm_mxfp4(a, (hipStream_t)stream));
}

int quantize_mxfp4(const float* X, int64_t rows, int64_t cols, int64_t ldx, uint8_t* Q,
                   int64_t ldq, uint8_t* S, int64_t lds, void* stream) {
  if (!X || !Q || !S || rows < 1 || cols < DMU_MX_BLOCK || cols % DMU_MX_BLOCK)
    return DMU_ERR_INVALID_ARG;
  if (ldx < cols || ldq < cols || lds < cols / DMU_MX_BLOCK || ldx % 4 || ldq % 32)
    return DMU_ERR_INVALID_ARG;
  if (!aligned(X, 16) || !aligned(Q, 16)) return DMU_ERR_INVALID_ARG;
  if (rows * (cols / DMU_MX_BLOCK) > INT32_MAX) return DMU_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  return finish(
      dmu::launch_quantize_mxfp4(X, rows, cols, ldx, Q, ldq / 2, S, lds, (hipStream_t)stream));
}

namespace {

// Output checks of the fused entry points (FP8 output allowed) and the
// epilogue fields of the launch arguments.
int fused_out(const void* D, int64_t ldd, int d_dtype, const float* d_scale, const float* bias,
              int act, int64_t M, int64_t N, dmu::GemmArgs& a) {
  if (!D || M < 1 || N < 1 || M > INT32_MAX || N > INT32_MAX) return DMU_ERR_INVALID_ARG;
  if (act < DMU_ACT_NONE || act > DMU_ACT_SILU) return DMU_ERR_INVALID_ARG;
  const bool fp8 = d_dtype == DMU_OUT_FP8_E4M3 || d_dtype == DMU_OUT_FP8_E5M2;
  if (d_dtype != DMU_OUT_F32 && d_dtype != DMU_OUT_BF16 && !fp8) return DMU_ERR_INVALID_ARG;
  const int64_t osz = d_dtype == DMU_OUT_F32 ? 4 : d_dtype == DMU_OUT_BF16 ? 2 : 1;
  if (ldd < N || !aligned(D, 16) || (ldd * osz) % 16) return DMU_ERR_INVALID_ARG;
  if (fp8 && (!d_scale || !aligned(d_scale, 4))) return DMU_ERR_INVALID_ARG;
  if (bias && !aligned(bias, 4)) return DMU_ERR_INVALID_ARG;
  a.out_bf16 = d_dtype == DMU_OUT_BF16;
  a.out_fp8 = d_dtype == DMU_OUT_FP8_E4M3 ? 0 : d_dtype == DMU_OUT_FP8_E5M2 ? 1 : -1;
  a.out_scale = fp8 ? d_scale : nullptr;
  a.bias = bias;
  a.act = act;
  return DMU_OK;
}

}  // namespace

int gemm_bf16_fused(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                    int b_layout, const float* bias, int act, void* D, int64_t ldd,
                    int d_dtype, const float* d_scale, int64_t M, int64_t N, int64_t K,
                    void* stream) {
  dmu::GemmArgs a{A, B, nullptr, D, lda, ldb, 0, ldd, M, N, K, nullptr, nullptr, 0};
  int rc = fused_out(D, ldd, d_dtype, d_scale, bias, act, M, N, a);
  if (rc) return rc;
  if (!A || !B || K < 8 || K % 8 || K > INT32_MAX) return DMU_ERR_INVALID_ARG;
  if (b_layout != DMU_B_ROW_MAJOR && b_layout != DMU_B_COL_MAJOR) return DMU_ERR_INVALID_ARG;
  if (lda < K || (lda * 2) % 16 || !aligned(A, 16) || !aligned(B, 16)) return DMU_ERR_INVALID_ARG;
  if (b_layout == DMU_B_ROW_MAJOR ? ldb < N : ldb < K) return DMU_ERR_INVALID_ARG;
  if ((ldb * 2) % 16) return DMU_ERR_INVALID_ARG;
  if (kTileRows * lda * 2 >= kMaxTileBytes) return DMU_ERR_UNSUPPORTED;
  if (b_layout == DMU_B_COL_MAJOR ? kTileRows * ldb * 2 >= kMaxTileBytes
                                  : K * ldb * 2 >= kMaxTileBytes)
    return DMU_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  const bool plain = !a.bias && !a.act && a.out_fp8 < 0;  // nothing to fuse: the plain kernels
  return finish(plain ? dmu::launch_gemm_bf16(a, b_layout == DMU_B_COL_MAJOR, (hipStream_t)stream)
                      : dmu::launch_gemm_bf16_fused(a, b_layout == DMU_B_COL_MAJOR,
                                                    (hipStream_t)stream));
}

int gemm_fp8_fused(const uint8_t* A, int64_t lda, int fmt_a, const uint8_t* B, int64_t ldb,
                   int fmt_b, const float* scale_a, const float* scale_b, const float* bias,
                   int act, void* D, int64_t ldd, int d_dtype, const float* d_scale, int64_t M,
                   int64_t N, int64_t K, void* stream) {
  dmu::GemmArgs a{A, B, nullptr, D, lda, ldb, 0, ldd, M, N, K, scale_a, scale_b, 0};
  int rc = fused_out(D, ldd, d_dtype, d_scale, bias, act, M, N, a);
  if (rc) return rc;
  if (!A || !B || !scale_a || !scale_b) return DMU_ERR_INVALID_ARG;
  if (fmt_a != DMU_FP8_E4M3 && fmt_a != DMU_FP8_E5M2) return DMU_ERR_INVALID_ARG;
  if (fmt_b != DMU_FP8_E4M3 && fmt_b != DMU_FP8_E5M2) return DMU_ERR_INVALID_ARG;
  if (K < 16 || K > INT32_MAX || K % 16) return DMU_ERR_INVALID_ARG;
  if (lda < K || ldb < K || lda % 16 || ldb % 16) return DMU_ERR_INVALID_ARG;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(scale_a, 4) || !aligned(scale_b, 4))
    return DMU_ERR_INVALID_ARG;
  if (kTileRows * lda >= kMaxTileBytes || kTileRows * ldb >= kMaxTileBytes)
    return DMU_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  const bool plain = !a.bias && !a.act && a.out_fp8 < 0;
  return finish(plain ? dmu::launch_gemm_fp8(a, fmt_a, fmt_b, 0, (hipStream_t)stream)
                      : dmu::launch_gemm_fp8_fused(a, fmt_a, fmt_b, (hipStream_t)stream));
}

const char* dmu_status_string(int status) {
  switch (status) {
    case DMU_OK:
      return "DMU_OK";
    case DMU_ERR_INVALID_ARG:
      return "DMU_ERR_INVALID_ARG: null pointer, bad size, alignment, leading dimension or enum";
    case DMU_ERR_UNSUPPORTED:
      return "DMU_ERR_UNSUPPORTED: valid request outside what this library implements";
    case DMU_ERR_HIP:
      return "DMU_ERR_HIP: the HIP runtime reported an error at launch";
    default:
      return "unknown dmu status";
  }
}

int dmu_version(void) { return (1 << 16) | 0; }

int dmu_probe_mfma_batch(int kind, int fmt_a, int fmt_b, const void* A, const void* B,
                         const float* C, float* D, int count, void* stream) {
  if (!A || !B || !C || !D || kind < 0 || kind > 3) return DMU_ERR_INVALID_ARG;
  if (fmt_a < 0 || fmt_a > 1 || fmt_b < 0 || fmt_b > 1) return DMU_ERR_INVALID_ARG;
  if (count < 1 || count > (1 << 20)) return DMU_ERR_INVALID_ARG;
  if (!aligned(A, 4) || !aligned(B, 4) || !aligned(C, 4) || !aligned(D, 4))
    return DMU_ERR_INVALID_ARG;
  (void)hipGetLastError();
  return finish(
      dmu::launch_probe_mfma(kind, fmt_a, fmt_b, A, B, C, D, count, (hipStream_t)stream));
}

int dmu_probe_mfma(int kind, int fmt_a, int fmt_b, const void* A, const void* B,
                   const float* C, float* D, void* stream) {
  return dmu_probe_mfma_batch(kind, fmt_a, fmt_b, A, B, C, D, 1, stream);
}

int dmu_probe_gemm_bf16_layout(int layout, const uint16_t* A, int64_t lda, const uint16_t* B,
                               int64_t ldb, void* D, int64_t ldd, int64_t M, int64_t N, int64_t K,
                               void* stream) {
  if (layout < 0 || layout > 2) return DMU_ERR_INVALID_ARG;
  int rc = check_out(nullptr, 0, D, ldd, DMU_OUT_BF16, M, N);
  if (rc) return rc;
  if (!A || !B || K < 64 || K % 64 || K > INT32_MAX) return DMU_ERR_INVALID_ARG;
  if (lda < K || ldb < K || (lda * 2) % 16 || (ldb * 2) % 16) return DMU_ERR_INVALID_ARG;
  if (!aligned(A, 16) || !aligned(B, 16)) return DMU_ERR_INVALID_ARG;
  if (kTileRows * lda * 2 >= kMaxTileBytes || kTileRows * ldb * 2 >= kMaxTileBytes)
    return DMU_ERR_UNSUPPORTED;
  dmu::GemmArgs a{A, B, nullptr, D, lda, ldb, 0, ldd, M, N, K, nullptr, nullptr, 1};
  (void)hipGetLastError();
  return finish(dmu::launch_gemm_bf16_layout(a, layout, (hipStream_t)stream));
}

int dmu_probe_lds_load(const void* src, void* dst, int mode, int oob_from, void* stream) {
  if (!src || !dst || (mode != 0 && mode != 1) || oob_from < 0 || oob_from > 64)
    return DMU_ERR_INVALID_ARG;
  if (!aligned(src, 16) || !aligned(dst, 16)) return DMU_ERR_INVALID_ARG;
  (void)hipGetLastError();
  return finish(dmu::launch_probe_lds(src, dst, mode, oob_from, (hipStream_t)stream));
}

int dmu_probe_mfma_rate(int kind, const void* src, int iters, int grid, float* out, void* stream) {
  if (!src || !out ||
      (kind != DMU_PROBE_BF16_32X32X16 && kind != DMU_PROBE_FP8_32X32X64 &&
       kind != DMU_PROBE_MXFP8_32X32X64 && kind != DMU_PROBE_MXFP4_32X32X64))
    return DMU_ERR_INVALID_ARG;
  if (iters < 1 || iters > (1 << 20) || grid < 1 || grid > 65536) return DMU_ERR_INVALID_ARG;
  if (!aligned(src, 16) || !aligned(out, 4)) return DMU_ERR_INVALID_ARG;
  (void)hipGetLastError();
  return finish(dmu::launch_probe_rate(kind, src, iters, grid, out, (hipStream_t)stream));
}

int dmu_probe_mfma_mx(int shape, int fmt_a, int fmt_b, int opsel, const void* A, const void* B,
                      const void* SA, const void* SB, const float* C, float* D, void* stream) {
  if (!A || !B || !SA || !SB || !C || !D || shape < 0 || shape > 1) return DMU_ERR_INVALID_ARG;
  auto fmt_ok = [](int f) { return f == 0 || f == 1 || f == 4; };
  if (!fmt_ok(fmt_a) || !fmt_ok(fmt_b) || opsel < 0 || opsel > 3) return DMU_ERR_INVALID_ARG;
  if ((fmt_a == 1 && fmt_b == 4) || (fmt_a == 4 && fmt_b == 1)) return DMU_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  return finish(
      dmu::launch_probe_mx(shape, fmt_a, fmt_b, opsel, A, B, SA, SB, C, D, (hipStream_t)stream));
}

int dmu_probe_lds_tr16(const uint16_t* src, const uint32_t* offsets, uint16_t* out,
                       void* stream) {
  if (!src || !offsets || !out || !aligned(src, 2) || !aligned(out, 2)) return DMU_ERR_INVALID_ARG;
  for (int l = 0; l < 64; ++l)
    if (offsets[l] % 8 || offsets[l] > 2040) return DMU_ERR_INVALID_ARG;
  (void)hipGetLastError();
  return finish(dmu::launch_probe_tr16(src, offsets, out, (hipStream_t)stream));
}

int dmu_probe_quantize_tensor_resident(const float* X, int64_t rows, int64_t cols, int fmt,
                                       uint8_t* Q, float* scale, int spin_limit, void* stream) {
  const int rc = quantize_args(X, rows, cols, cols, fmt, rows, cols, Q, cols, scale);
  if (rc) return rc;
  if (spin_limit < 0 || spin_limit > (1 << 16)) return DMU_ERR_INVALID_ARG;  // every wait stays short
  (void)hipGetLastError();
  const hipError_t e = dmu::launch_probe_quantize_resident(X, rows, cols, fmt, Q, scale,
                                                           spin_limit, (hipStream_t)stream);
  if (e == hipErrorInvalidValue) return DMU_ERR_UNSUPPORTED;
  return finish(e);
}

int dmu_probe_cvt_fp8(const float* x, int64_t n, int fmt, int clamp, uint8_t* q, void* stream) {
  if (!x || !q || n < 2 || n % 2 || n > ((int64_t)1 << 31)) return DMU_ERR_INVALID_ARG;
  if ((fmt != 0 && fmt != 1 && fmt != 4) || (clamp != 0 && clamp != 1) || !aligned(x, 8))
    return DMU_ERR_INVALID_ARG;
  (void)hipGetLastError();
  return finish(dmu::launch_probe_cvt(x, n, fmt, clamp, q, (hipStream_t)stream));
}

}  // extern "C"
