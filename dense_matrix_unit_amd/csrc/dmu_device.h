// Device-side helpers shared by the gfx950 kernels of the dmu library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dmu {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// Word 3 of a raw buffer resource on gfx950: 32-bit data format, no
// swizzling, no index stride (CDNA3/CDNA4 ISA, "Buffer Resource").
constexpr int kRsrcWord3 = 0x00020000;
// Any voffset at or beyond this value is outside every resource built by
// make_rsrc (num_records is clamped below it): loads return zero.
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  if (bytes > 0x7FFFFFFF) bytes = 0x7FFFFFFF;
  if (bytes < 0) bytes = 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

// Direct global -> LDS copy of 16 bytes per lane: lane l's bytes land at
// lds + 16*l (lds must be wave-uniform).  Out-of-range offsets write zeros.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void* lds,
                                                  uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, soff, 0, 0);
}

// Same with 4 bytes per lane: lane l's dword lands at lds + 4*l.
__device__ __forceinline__ void buffer_load_lds4(__amdgpu_buffer_rsrc_t r, void* lds,
                                                 uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 4, voff, soff, 0, 0);
}

__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                 uint32_t soff) {
  i32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return __builtin_bit_cast(u32x4_t, v);
}

// FP32 -> BF16 bits, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = (__bf16)x;
  return __builtin_bit_cast(uint16_t, h);
}

// Two FP32 values -> two BF16 (round to nearest even), lo in the low half:
// one v_cvt_pk_bf16_f32, where two f32_to_bf16_bits and an OR take three.
typedef __bf16 dmu_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float dmu_f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(dmu_f32x2_t{lo, hi}, dmu_bf16x2_t));
}

// FP8 formats (OCP): E4M3 (FN: no Inf, S.1111.111 NaN, max 448) and E5M2.
template <int FMT>
struct Fp8Fmt;
template <>
struct Fp8Fmt<0> {  // E4M3 (OCP FN)
  static constexpr int kMant = 3, kBias = 7;
  static constexpr uint32_t kMaxBits = 0x43E00000u;  // 448.0f
  static constexpr uint32_t kMaxCode = 0x7E;
  static constexpr float kMax = 448.0f;
};
template <>
struct Fp8Fmt<1> {  // E5M2
  static constexpr int kMant = 2, kBias = 15;
  static constexpr uint32_t kMaxBits = 0x47600000u;  // 57344.0f
  static constexpr uint32_t kMaxCode = 0x7B;
  static constexpr float kMax = 57344.0f;
};

// Saturating round-to-nearest-even FP32 -> FP8 on the bit pattern.
template <int FMT>
__device__ __forceinline__ uint32_t encode_fp8(float y) {
  using F = Fp8Fmt<FMT>;
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;         // NaN
  if (a >= F::kMaxBits) return sign | F::kMaxCode;  // saturate (Inf included)
  constexpr uint32_t kMinNormal = (uint32_t)(127 + 1 - F::kBias) << 23;
  constexpr int kDrop = 23 - F::kMant;
  if (a >= kMinNormal) {
    // keep kMant fraction bits, round half to even, re-bias the exponent
    const uint32_t r = (a + ((1u << (kDrop - 1)) - 1u) + ((a >> kDrop) & 1u)) >> kDrop;
    return sign | (r - ((uint32_t)(127 - F::kBias) << F::kMant));
  }
  if (a < 0x00800000u) return sign;  // zero or FP32 subnormal: far below half an FP8 step
  // FP8 subnormal: count multiples of 2^(1 - bias - mant), round half to even
  const int e = (int)(a >> 23);
  const uint32_t sig = (a & 0x007FFFFFu) | 0x00800000u;
  const int shift = 150 + 1 - F::kBias - F::kMant - e;
  if (shift > 24) return sign;
  const uint32_t n = (sig + (1u << (shift - 1)) - 1u + ((sig >> shift) & 1u)) >> shift;
  return sign | n;
}

// Four FP32 values -> four FP8 codes (byte r = value r), saturating RNE: the
// hardware conversion (v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32) rounds to nearest
// even but turns values past the largest finite one into NaN / Inf, so they
// are clamped first (NaN passed through).
template <int FMT>
__device__ __forceinline__ uint32_t cvt4_fp8(f32x4_t y) {
  constexpr float kMax = FMT == 0 ? 448.0f : 57344.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) y[r] = y[r] != y[r] ? y[r] : fminf(fmaxf(y[r], -kMax), kMax);
  int w;
  if constexpr (FMT == 0) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(y[0], y[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(y[2], y[3], w, true);
  }
  return (uint32_t)w;
}

// Four FP32 values -> four E2M1 codes in 16 bits (value r in nibble r), round
// to nearest even, saturating at +-6: gfx950's v_cvt_scalef32_pk_fp4_f32 with
// a scale operand of 1 (no scaling), two values per instruction into byte
// `sel` of its result, after a clamp to +-6.  Only for finite values (the
// quantizer sends blocks with NaN or Inf elsewhere).
__device__ __forceinline__ uint32_t cvt4_fp4(f32x4_t y) {
#pragma unroll
  for (int r = 0; r < 4; ++r) y[r] = fminf(fmaxf(y[r], -6.0f), 6.0f);
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[0], y[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
  return w & 0xFFFFu;
}

}  // namespace dmu
