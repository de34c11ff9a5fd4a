// Device helpers shared by the tiled GEMM kernels (gemm.hip, gemm_block.hip).
#pragma once

#include "dmu_device.h"
#include "dmu_internal.h"

namespace dmu {

constexpr int kThreads = 256;  // 4 waves, one per SIMD

// A compile-time int passed as a value (loop bodies instantiated per stage,
// per output type).
template <int V>
struct IntConst {
  static constexpr int value = V;
};

// LDS position of logical 16-byte chunk c in row r for RB-byte rows.
template <int RB>
__device__ __forceinline__ int swz(int r) {
  if constexpr (RB == 128) return (r ^ (r >> 3)) & 7;
  else return ((r >> 1) ^ (r >> 2)) & 3;
}

// s_waitcnt immediate for gfx9-family: vmcnt(N) and lgkmcnt(0), expcnt free.
template <int N>
constexpr int waitcnt_vm_lgkm0() {
  return (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4);
}

// Workgroup barrier for the K loop.  The caller has already waited for its
// own copies and LDS reads with an explicit s_waitcnt; __syncthreads() would
// add a release fence, i.e. a wait for every outstanding vector memory
// operation, including the L2 prefetch that is meant to stay in flight.  The
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup -> output tile.  Workgroups are dispatched to the 8 XCDs round
// robin (id % 8); give each XCD a contiguous run of logical tile ids, and walk
// logical ids in column-major groups of kGroupM tile rows so that the tiles
// resident on one XCD share few A and B panels.
template <int kGroupM>
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int b = blockIdx.x, T = gridDim.x;
  const int x = b & 7, j = b >> 3, per = T >> 3, rem = T & 7;
  const int logical = x * per + (x < rem ? x : rem) + j;
  const int group = kGroupM * tiles_n;
  const int g = logical / group;
  const int first = g * kGroupM;
  const int gs = min(tiles_m - first, kGroupM);
  const int r = logical - g * group;
  tm = first + r % gs;
  tn = r / gs;
}

__device__ __forceinline__ i32x8_t cat(const i32x4_t& lo, const i32x4_t& hi) {
  return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Activations of the fused epilogue, in few instructions: every output
// element goes through one, and a wave holds 16384 of them per tile.
// e^y is 2^(y log2 e) on the hardware exp2 (v_exp_f32), 1 / y the hardware
// reciprocal (v_rcp_f32).
constexpr float kLog2e = 1.44269504088896341f;

// GELU, x * Phi(x).  For z = |x| / sqrt 2, (1 - erf z) / 2 is taken from the
// erf approximation of Abramowitz & Stegun, Handbook of Mathematical
// Functions, formula 7.1.26 (absolute error <= 1.5e-7):
// 1 - erf z ~ t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) e^(-z^2), t = 1 / (1 + p z).
// Phi(x) is that half-complement for x < 0 and 1 minus it otherwise, so the
// negative tail is not a difference of nearly equal numbers.
__device__ __forceinline__ float gelu(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
  const float poly =
      t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f),
                       -0.284496736f),
               0.254829592f);
  const float q = 0.5f * poly * __builtin_amdgcn_exp2f(-z * z * kLog2e);
  return x * (x < 0.0f ? q : 1.0f - q);
}

// SiLU, x / (1 + e^-x).
__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
}

// 1 ReLU (x > 0 ? x : 0), 2 GELU, 3 SiLU, else x.
__device__ __forceinline__ float activate(float x, int act) {
  if (act == 1) return x > 0.0f ? x : 0.0f;
  if (act == 2) return gelu(x);
  if (act == 3) return silu(x);
  return x;
}

// D[row][col .. col+3] = x (+ C), masked to the matrix.
__device__ __forceinline__ void store4(const GemmArgs& p, int64_t row, int64_t col, f32x4_t x) {
  if (row >= p.M || col >= p.N) return;
  const bool full = col + 3 < p.N;
  if (p.C) {
    const float* c = p.C + row * p.ldc + col;
    if (full) {
      x += *(const f32x4_t*)c;
    } else {
      for (int r = 0; r < 4; ++r)
        if (col + r < p.N) x[r] += c[r];
    }
  }
  if (p.out_bf16) {
    uint16_t* d = (uint16_t*)p.D + row * p.ldd + col;
    const uint32_t lo = pack2_bf16(x[0], x[1]);
    const uint32_t hi = pack2_bf16(x[2], x[3]);
    if (full) {
      *(uint2*)d = make_uint2(lo, hi);
    } else {
      for (int r = 0; r < 4; ++r)
        if (col + r < p.N) d[r] = f32_to_bf16_bits(x[r]);
    }
  } else {
    float* d = (float*)p.D + row * p.ldd + col;
    if (full) {
      *(f32x4_t*)d = x;
    } else {
      for (int r = 0; r < 4; ++r)
        if (col + r < p.N) d[r] = x[r];
    }
  }
}

}  // namespace dmu
