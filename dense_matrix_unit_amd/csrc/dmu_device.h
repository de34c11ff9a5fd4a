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

}  // namespace dmu
