// One-instruction probes of the gfx950 matrix unit and of the direct
// global -> LDS copy.  They exist so the test suite can pin the lane/register
// layouts the GEMM kernels rely on, the way the page "Tensor Cores: Matrix
// Instructions, Swizzling and FP8, Measured" (vidyal.ai), Step 1, checks one
// mma.sync against the CPU with small-integer inputs, and Step 5 probes how
// many bits the accumulator keeps (C = 2^e plus a product of 1).
//
// Layouts assumed (and therefore tested) for one wave of 64 lanes, with
// g = lane / rows-per-group:
//  * 16x16xK MFMA (K = 32 bf16 or 128 fp8): lane l supplies row l%16 of A and
//    column l%16 of B, holding the K-run [g*K/4, (g+1)*K/4) with g = l/16;
//    result register v of lane l is D[4*(l/16) + v][l%16].
//  * 32x32xK MFMA (K = 16 bf16 or 64 fp8): lane l supplies row l%32 of A and
//    column l%32 of B, holding the K-run [g*K/2, (g+1)*K/2) with g = l/32;
//    result register v of lane l is D[8*(v/4) + 4*(l/32) + v%4][l%32].
// Without scales a product is the same under any permutation of K shared by
// A and B, so these probes pin rows, columns and result registers but not
// which K positions a lane's bytes stand for.  The scaled (MX) probe does:
// there a lane's 32 FP8 bytes are two 16-byte halves, half h holding K
// positions [h*K/2 + 16*g, h*K/2 + 16*g + 16), and lane group b supplies the
// scale of the 32-wide K block b.
#include "dmu_device.h"
#include "dmu_internal.h"

namespace dmu {
namespace {

// A: [M][K] row-major, B: [N][K] row-major (B stored N x K), C/D: [M][N] FP32.
// Workgroup i (one wave) runs instance i of a batch: its A, B, C and D follow
// instance i-1's, one instruction's operands each (A and B: 512 BF16 values
// = 1024 bytes, or 2048 FP8 codes; C and D: 16x16 or 32x32 floats).
template <int KIND, int FA, int FB>
__global__ void probe_mfma_kernel(const void* Av, const void* Bv, const float* C, float* D) {
  const int l = threadIdx.x;
  {
    constexpr int64_t kOperandBytes = KIND < 2 ? 1024 : 2048;      // one A (or B) instance
    constexpr int64_t kOut = KIND == 0 || KIND == 2 ? 256 : 1024;  // floats of C (or D)
    const int64_t i = blockIdx.x;
    Av = (const uint8_t*)Av + i * kOperandBytes;
    Bv = (const uint8_t*)Bv + i * kOperandBytes;
    C += i * kOut;
    D += i * kOut;
  }
  if constexpr (KIND == 0) {  // bf16 16x16x32
    const uint16_t* A = (const uint16_t*)Av;
    const uint16_t* B = (const uint16_t*)Bv;
    bf16x8_t a, b;
    for (int p = 0; p < 8; ++p) {
      a[p] = __builtin_bit_cast(__bf16, A[(l % 16) * 32 + 8 * (l / 16) + p]);
      b[p] = __builtin_bit_cast(__bf16, B[(l % 16) * 32 + 8 * (l / 16) + p]);
    }
    f32x4_t c;
    for (int v = 0; v < 4; ++v) c[v] = C[(4 * (l / 16) + v) * 16 + l % 16];
    const f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    for (int v = 0; v < 4; ++v) D[(4 * (l / 16) + v) * 16 + l % 16] = d[v];
  } else if constexpr (KIND == 1) {  // bf16 32x32x16
    const uint16_t* A = (const uint16_t*)Av;
    const uint16_t* B = (const uint16_t*)Bv;
    bf16x8_t a, b;
    for (int p = 0; p < 8; ++p) {
      a[p] = __builtin_bit_cast(__bf16, A[(l % 32) * 16 + 8 * (l / 32) + p]);
      b[p] = __builtin_bit_cast(__bf16, B[(l % 32) * 16 + 8 * (l / 32) + p]);
    }
    f32x16_t c;
    for (int v = 0; v < 16; ++v) c[v] = C[(8 * (v / 4) + 4 * (l / 32) + v % 4) * 32 + l % 32];
    const f32x16_t d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    for (int v = 0; v < 16; ++v) D[(8 * (v / 4) + 4 * (l / 32) + v % 4) * 32 + l % 32] = d[v];
  } else if constexpr (KIND == 2) {  // fp8 16x16x128
    const uint8_t* A = (const uint8_t*)Av;
    const uint8_t* B = (const uint8_t*)Bv;
    i32x8_t a, b;
    for (int w = 0; w < 8; ++w) {
      uint32_t x = 0, y = 0;
      for (int q = 0; q < 4; ++q) {
        x |= (uint32_t)A[(l % 16) * 128 + 32 * (l / 16) + 4 * w + q] << (8 * q);
        y |= (uint32_t)B[(l % 16) * 128 + 32 * (l / 16) + 4 * w + q] << (8 * q);
      }
      a[w] = (int)x;
      b[w] = (int)y;
    }
    f32x4_t c;
    for (int v = 0; v < 4; ++v) c[v] = C[(4 * (l / 16) + v) * 16 + l % 16];
    const f32x4_t d =
        __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
    for (int v = 0; v < 4; ++v) D[(4 * (l / 16) + v) * 16 + l % 16] = d[v];
  } else {  // fp8 32x32x64
    const uint8_t* A = (const uint8_t*)Av;
    const uint8_t* B = (const uint8_t*)Bv;
    i32x8_t a, b;
    for (int w = 0; w < 8; ++w) {
      uint32_t x = 0, y = 0;
      for (int q = 0; q < 4; ++q) {
        x |= (uint32_t)A[(l % 32) * 64 + 32 * (l / 32) + 4 * w + q] << (8 * q);
        y |= (uint32_t)B[(l % 32) * 64 + 32 * (l / 32) + 4 * w + q] << (8 * q);
      }
      a[w] = (int)x;
      b[w] = (int)y;
    }
    f32x16_t c;
    for (int v = 0; v < 16; ++v) c[v] = C[(8 * (v / 4) + 4 * (l / 32) + v % 4) * 32 + l % 32];
    const f32x16_t d =
        __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
    for (int v = 0; v < 16; ++v) D[(8 * (v / 4) + 4 * (l / 32) + v % 4) * 32 + l % 32] = d[v];
  }
}

// One scaled matrix instruction (microscaling, MX): D = (A x SA)(B x SB) + C
// with one E8M0 scale (2^(code-127)) per row and 32-element K block, the
// block-scaled product of the page "How Blackwell's Tensor Memory Actually
// Works", section "Quantization became an allocation problem".  Layout (with
// g = l / rows, rows = 16 or 32): lane l holds row l % rows; byte o of its
// data half h (0, 1) is K position h*K/2 + 16*g + o; it supplies the scale of
// K block g -- SA[l%16][l/16] for 16x16x128, SA[l%32][l/32] for 32x32x64 --
// in byte OPSEL of its 32-bit scale register, the other three bytes holding
// decoys (code ^ 4, a factor 16 away) so a wrong byte choice shows in D.
// Byte o (0..31) of the operand registers of lane group g, for one row of
// an operand of instruction width K: FP8 (one value per byte) as described
// above; FP4 (format 4, E2M1 two per byte, 16 bytes per lane) as byte o of
// the row's packed bytes [16 g, 16 g + 16).
template <int FMT, int K>
__device__ __forceinline__ int mx_src_byte(int g, int o) {
  if constexpr (FMT == 4) return 16 * g + o;
  else return (o / 16) * (K / 2) + 16 * g + o % 16;
}

template <int FMT, int K>
__device__ __forceinline__ i32x8_t mx_fragment(const uint8_t* rowp, int g) {
  constexpr int NB = FMT == 4 ? 16 : 32;  // bytes per lane
  i32x8_t v = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int w = 0; w < NB / 4; ++w) {
    uint32_t x = 0;
    for (int q = 0; q < 4; ++q) x |= (uint32_t)rowp[mx_src_byte<FMT, K>(g, 4 * w + q)] << (8 * q);
    v[w] = (int)x;
  }
  return v;
}

template <int SHAPE, int FA, int FB, int OPSEL>
__global__ void probe_mx_kernel(const uint8_t* A, const uint8_t* B, const uint8_t* SA,
                                const uint8_t* SB, const float* C, float* D) {
  const int l = threadIdx.x;
  constexpr int R = SHAPE == 0 ? 16 : 32;   // rows per K group
  constexpr int K = SHAPE == 0 ? 128 : 64;  // instruction K
  const int row = l % R, g = l / R;
  constexpr int RBA = FA == 4 ? K / 2 : K, RBB = FB == 4 ? K / 2 : K;  // bytes per row
  const i32x8_t a = mx_fragment<FA, K>(A + row * RBA, g);
  const i32x8_t b = mx_fragment<FB, K>(B + row * RBB, g);
  auto word = [&](uint8_t code) {
    uint32_t v = 0;
    for (int q = 0; q < 4; ++q) v |= (uint32_t)(q == OPSEL ? code : (uint8_t)(code ^ 4)) << (8 * q);
    return (int)v;
  };
  const int sa = word(SA[row * (K / 32) + g]), sb = word(SB[row * (K / 32) + g]);
  if constexpr (SHAPE == 0) {
    f32x4_t c;
    for (int v = 0; v < 4; ++v) c[v] = C[(4 * g + v) * 16 + row];
    const f32x4_t d =
        __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, OPSEL, sa, OPSEL, sb);
    for (int v = 0; v < 4; ++v) D[(4 * g + v) * 16 + row] = d[v];
  } else {
    f32x16_t c;
    for (int v = 0; v < 16; ++v) c[v] = C[(8 * (v / 4) + 4 * g + v % 4) * 32 + row];
    const f32x16_t d =
        __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, OPSEL, sa, OPSEL, sb);
    for (int v = 0; v < 16; ++v) D[(8 * (v / 4) + 4 * g + v % 4) * 32 + row] = d[v];
  }
}

// FP32 -> FP8 with the hardware conversion, two values per instruction:
// v_cvt_pk_fp8_f32 (E4M3) / v_cvt_pk_bf8_f32 (E5M2), applied to x as it is
// (CLAMP == 0), or through cvt4_fp8 (CLAMP == 1: x clamped to the format's
// largest finite magnitude, NaN passed through, then converted; the function
// the fused epilogue and the quantizers use).  Thread t converts x[2t],
// x[2t+1] into q[2t], q[2t+1].  FMT 4: E2M1 by v_cvt_scalef32_pk_fp4_f32 with
// scale 1 (CLAMP == 1: through cvt4_fp4, clamped to +-6), both codes of the
// pair into byte q[t].
template <int FMT, int CLAMP>
__global__ void probe_cvt_kernel(const float* x, int64_t npairs, uint8_t* q) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= npairs) return;
  const float a = x[2 * t], b = x[2 * t + 1];
  uint32_t r;
  if constexpr (FMT == 4) {
    // E2M1: both codes in one byte
    r = CLAMP ? cvt4_fp4(f32x4_t{a, b, 0.0f, 0.0f})
              : (uint32_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0);
    q[t] = (uint8_t)(r & 0xFF);
    return;
  } else if constexpr (CLAMP) {
    r = cvt4_fp8<FMT>(f32x4_t{a, b, 0.0f, 0.0f});
  } else if constexpr (FMT == 0) {
    r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  } else {
    r = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
  }
  q[2 * t] = (uint8_t)(r & 0xFF);
  q[2 * t + 1] = (uint8_t)((r >> 8) & 0xFF);
}

// gfx950's transposing LDS read, ds_read_b64_tr_b16: one wave loads 2 KiB
// of 16-bit values into LDS, then lane l issues the transposing read at byte
// offset off.v[l] (checked on the host: 8-byte aligned, inside the 2 KiB) and
// writes the four 16-bit values it receives to out[4l .. 4l+3].
struct TrOffsets {
  uint32_t v[64];
};
typedef short tr_v4i16 __attribute__((ext_vector_type(4)));
__global__ void probe_tr16_kernel(const uint16_t* src, TrOffsets off, uint16_t* out) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[1024];
  const int l = threadIdx.x;
  for (int i = l; i < 1024; i += 64) lds[i] = src[i];
  __syncthreads();
  const uint32_t o = off.v[l] & 2040u;  // in range by construction (host check)
  const tr_v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) tr_v4i16*)((uint8_t*)lds + o));
  for (int e = 0; e < 4; ++e) out[4 * l + e] = (uint16_t)r[e];
}

// One wave copies 64 x 16 bytes (mode 0) or 64 x 4 bytes (mode 1) from src to
// LDS with buffer loads that write LDS directly, then dumps 2 KiB of LDS to
// dst.  Lanes >= oob_from get an out-of-range offset (they must write zeros).
__global__ void probe_lds_kernel(const uint8_t* src, uint8_t* dst, int mode, int oob_from) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2048];
  const int l = threadIdx.x;
  for (int i = l; i < 2048 / 4; i += 64) ((uint32_t*)lds)[i] = 0xA5A5A5A5u;
  __syncthreads();
  const int sz = mode == 0 ? 16 : 4;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(src, 64 * sz);
  const uint32_t voff = l < oob_from ? (uint32_t)(l * sz) : kOOB;
  if (mode == 0)
    buffer_load_lds16(r, lds, voff, 0);
  else
    buffer_load_lds4(r, lds, voff, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int i = l; i < 2048 / 4; i += 64) ((uint32_t*)dst)[i] = ((uint32_t*)lds)[i];
}

// Sustained matrix-unit rate with operands that change from one instruction
// to the next, and no memory traffic in the loop.  Each wave loads four A and
// four B fragments from `src` (fragment f of lane l at src + (f*64 + l)*FB,
// FB = 16 bytes for BF16, 32 for FP8), then runs `iters` rounds of the 4 x 4
// block of 32x32 MFMAs the GEMM kernel's wave tile issues per K step, into 16
// independent accumulators (256 registers, one wave per SIMD).  Lane l of
// wave w then writes the sum of its 256 accumulator values to
// out[w * 64 + l], which keeps every instruction live.
template <int KIND>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void probe_rate_kernel(
    const uint8_t* src, int iters, float* out, int scale_word) {
  const int l = threadIdx.x & 63;
  constexpr int FB = KIND == 1 ? 16 : 32;  // fragment bytes per lane
  i32x8_t a[4], b[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const i32x4_t* pa = (const i32x4_t*)(src + (f * 64 + l) * FB);
    const i32x4_t* pb = (const i32x4_t*)(src + ((4 + f) * 64 + l) * FB);
    const i32x4_t a0 = pa[0], b0 = pb[0];
    const i32x4_t a1 = FB == 32 ? pa[1] : i32x4_t{0, 0, 0, 0};
    const i32x4_t b1 = FB == 32 ? pb[1] : i32x4_t{0, 0, 0, 0};
    a[f] = i32x8_t{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    b[f] = i32x8_t{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
  }
  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (KIND == 1) {
          const i32x4_t x = {a[i][0], a[i][1], a[i][2], a[i][3]};
          const i32x4_t y = {b[j][0], b[j][1], b[j][2], b[j][3]};
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, y), __builtin_bit_cast(bf16x8_t, x), acc[i][j], 0, 0, 0);
        } else if constexpr (KIND == 4) {  // scaled form, E8M0 codes in registers
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              b[j], a[i], acc[i][j], 0, 0, 0, scale_word, 0, scale_word);
        } else if constexpr (KIND == 5) {  // FP4 (E2M1) operands: low 16 bytes of each fragment
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              b[j], a[i], acc[i][j], 4, 4, 0, scale_word, 0, scale_word);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a[i], acc[i][j], 0, 0,
                                                                      0, 0, 0, 0);
        }
      }
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) sum += acc[i][j][v];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = sum;
}

template <int KIND>
hipError_t probe_fmt(int fa, int fb, const void* A, const void* B, const float* C, float* D,
                     int count, hipStream_t s) {
#define DMU_PROBE_LAUNCH(FA, FB)                                                           \
  hipLaunchKernelGGL((probe_mfma_kernel<KIND, FA, FB>), dim3(count), dim3(64), 0, s, A, B, C, \
                     D)
  if (fa == 0 && fb == 0) DMU_PROBE_LAUNCH(0, 0);
  else if (fa == 0 && fb == 1) DMU_PROBE_LAUNCH(0, 1);
  else if (fa == 1 && fb == 0) DMU_PROBE_LAUNCH(1, 0);
  else DMU_PROBE_LAUNCH(1, 1);
#undef DMU_PROBE_LAUNCH
  return hipGetLastError();
}

template <int SHAPE, int FA, int FB>
hipError_t probe_mx_opsel(int opsel, const uint8_t* A, const uint8_t* B, const uint8_t* SA,
                          const uint8_t* SB, const float* C, float* D, hipStream_t s) {
#define DMU_PROBE_MX(O)                                                                      \
  hipLaunchKernelGGL((probe_mx_kernel<SHAPE, FA, FB, O>), dim3(1), dim3(64), 0, s, A, B, SA, \
                     SB, C, D)
  switch (opsel) {
    case 0: DMU_PROBE_MX(0); break;
    case 1: DMU_PROBE_MX(1); break;
    case 2: DMU_PROBE_MX(2); break;
    default: DMU_PROBE_MX(3); break;
  }
#undef DMU_PROBE_MX
  return hipGetLastError();
}

template <int SHAPE>
hipError_t probe_mx_fmt(int fa, int fb, int opsel, const uint8_t* A, const uint8_t* B,
                        const uint8_t* SA, const uint8_t* SB, const float* C, float* D,
                        hipStream_t s) {
  if (fa == 0 && fb == 0) return probe_mx_opsel<SHAPE, 0, 0>(opsel, A, B, SA, SB, C, D, s);
  if (fa == 0 && fb == 1) return probe_mx_opsel<SHAPE, 0, 1>(opsel, A, B, SA, SB, C, D, s);
  if (fa == 1 && fb == 0) return probe_mx_opsel<SHAPE, 1, 0>(opsel, A, B, SA, SB, C, D, s);
  if (fa == 1 && fb == 1) return probe_mx_opsel<SHAPE, 1, 1>(opsel, A, B, SA, SB, C, D, s);
  if (fa == 4 && fb == 4) return probe_mx_opsel<SHAPE, 4, 4>(opsel, A, B, SA, SB, C, D, s);
  if (fa == 4 && fb == 0) return probe_mx_opsel<SHAPE, 4, 0>(opsel, A, B, SA, SB, C, D, s);
  return probe_mx_opsel<SHAPE, 0, 4>(opsel, A, B, SA, SB, C, D, s);
}

}  // namespace

hipError_t launch_probe_mfma(int kind, int fa, int fb, const void* A, const void* B,
                             const float* C, float* D, int count, hipStream_t s) {
  switch (kind) {
    case 0:
      hipLaunchKernelGGL((probe_mfma_kernel<0, 0, 0>), dim3(count), dim3(64), 0, s, A, B, C, D);
      return hipGetLastError();
    case 1:
      hipLaunchKernelGGL((probe_mfma_kernel<1, 0, 0>), dim3(count), dim3(64), 0, s, A, B, C, D);
      return hipGetLastError();
    case 2:
      return probe_fmt<2>(fa, fb, A, B, C, D, count, s);
    default:
      return probe_fmt<3>(fa, fb, A, B, C, D, count, s);
  }
}

hipError_t launch_probe_lds(const void* src, void* dst, int mode, int oob_from, hipStream_t s) {
  hipLaunchKernelGGL(probe_lds_kernel, dim3(1), dim3(64), 0, s, (const uint8_t*)src,
                     (uint8_t*)dst, mode, oob_from);
  return hipGetLastError();
}

hipError_t launch_probe_rate(int kind, const void* src, int iters, int grid, float* out,
                             hipStream_t s) {
  if (kind == 1)
    hipLaunchKernelGGL(probe_rate_kernel<1>, dim3(grid), dim3(256), 0, s, (const uint8_t*)src,
                       iters, out, 0);
  else if (kind == 4)
    hipLaunchKernelGGL(probe_rate_kernel<4>, dim3(grid), dim3(256), 0, s, (const uint8_t*)src,
                       iters, out, 0x7F7F7F7F);
  else if (kind == 5)
    hipLaunchKernelGGL(probe_rate_kernel<5>, dim3(grid), dim3(256), 0, s, (const uint8_t*)src,
                       iters, out, 0x7F7F7F7F);
  else
    hipLaunchKernelGGL(probe_rate_kernel<3>, dim3(grid), dim3(256), 0, s, (const uint8_t*)src,
                       iters, out, 0);
  return hipGetLastError();
}

hipError_t launch_probe_mx(int shape, int fa, int fb, int opsel, const void* A, const void* B,
                           const void* SA, const void* SB, const float* C, float* D,
                           hipStream_t s) {
  const uint8_t *a = (const uint8_t*)A, *b = (const uint8_t*)B;
  const uint8_t *sa = (const uint8_t*)SA, *sb = (const uint8_t*)SB;
  if (shape == 0) return probe_mx_fmt<0>(fa, fb, opsel, a, b, sa, sb, C, D, s);
  return probe_mx_fmt<1>(fa, fb, opsel, a, b, sa, sb, C, D, s);
}

hipError_t launch_probe_tr16(const uint16_t* src, const uint32_t* offsets, uint16_t* out,
                             hipStream_t s) {
  TrOffsets o;
  for (int l = 0; l < 64; ++l) o.v[l] = offsets[l];
  hipLaunchKernelGGL(probe_tr16_kernel, dim3(1), dim3(64), 0, s, src, o, out);
  return hipGetLastError();
}

hipError_t launch_probe_cvt(const float* x, int64_t n, int fmt, int clamp, uint8_t* q,
                            hipStream_t s) {
  const int64_t np = n / 2;
  const dim3 grid((unsigned)((np + 255) / 256));
#define DMU_CVT(F, C) hipLaunchKernelGGL((probe_cvt_kernel<F, C>), grid, dim3(256), 0, s, x, np, q)
  if (fmt == 0 && !clamp) DMU_CVT(0, 0);
  else if (fmt == 0) DMU_CVT(0, 1);
  else if (fmt == 4 && !clamp) DMU_CVT(4, 0);
  else if (fmt == 4) DMU_CVT(4, 1);
  else if (!clamp) DMU_CVT(1, 0);
  else DMU_CVT(1, 1);
#undef DMU_CVT
  return hipGetLastError();
}

}  // namespace dmu
