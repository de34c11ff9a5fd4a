// FP32 -> FP8 (E4M3 / E5M2) quantisation with one scale per block, for gfx950.
//
// What is computed (page "Tensor cores and low precision", learn-kernels.com,
// paragraph on rescaling before the cast; "Tensor Cores" chapter,
// ai-infra-handbooks, "Precision" section on per-tensor / per-block scaling
// factors): for each block, amax = max |x|, m = FMAX / amax, every element is
// encoded as the saturating round-to-nearest-even FP8 value of the FP32
// product x*m, and the dequantisation factor s = amax / FMAX is stored.
//
// Kernels (all HBM-bound streaming; every value is read once per pass):
//  * per tensor, contiguous and small enough for the grid's registers: one
//    pass (quant_tensor_resident, described at the kernel).  Amaxes are
//    compared as the bit patterns of |x|: for non-negative floats the
//    integer order is the numeric order, and any NaN pattern sorts above
//    +Inf, so a NaN anywhere yields a NaN amax.
//  * per tensor, otherwise: two passes.  Pass 1: each workgroup writes the
//    max of the |x| bit patterns over its grid-stride share to its own
//    scratch slot.  Pass 2: each workgroup takes the max of all slots (the
//    tensor's amax), then encodes its share; workgroup 0 stores the scale.
//    No slot needs clearing and no atomics are used; the slot count is the
//    pass-1 grid (at most 512, whatever the tensor's size).
//  * 1 x 128 blocks: 32 lanes per block (16 bytes per lane), half-wave max,
//    rows walked by the grid's y dimension.
//  * 128 x 128 blocks: one 256-thread workgroup per block keeps its 64 values
//    per thread in registers between the amax and the encode (one HBM read).
//  * MX (1 x 32 blocks, E8M0 scales; "How Blackwell's Tensor Memory Actually
//    Works", section "Quantization became an allocation problem", with the
//    Open Compute microscaling choice of scale): 8 lanes per block, rows
//    walked by the grid's y dimension.  The
//    scale is X = 2^(floor(log2 amax) - emax), emax = 8 (E4M3) or 15 (E5M2),
//    the largest power of two that keeps amax / X below 2^(emax+1); its code
//    is the biased exponent of amax minus emax, clamped at 0.  Elements are
//    the saturating RNE codes of x * 2^(127 - code), an exact FP32 product
//    (the multiplier is a normal power of two, and a product that leaves the
//    normal range is far below half the smallest FP8 step).  A block holding
//    NaN or Inf gets code 255 (NaN) and NaN element codes of the elements'
//    signs.  MXFP4 (E2M1, emax = 2) packs the four codes of a lane into 16
//    bits, element 2i in the low nibble; a NaN/Inf block's elements are
//    signed zeros (E2M1 has no NaN).
#include <hip/hip_ext.h>

#include <atomic>
#include <mutex>

#include "dmu_device.h"
#include "dmu_internal.h"

namespace dmu {

int device_of(hipStream_t s, hipError_t* e);
int compute_units(hipStream_t s);

namespace {

__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

__device__ __forceinline__ uint32_t half_wave_max(uint32_t v) {
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

// m = FMAX / amax (or 1 for an all-zero block), IEEE division.
template <int FMT>
__device__ __forceinline__ float mult_from_amax(float amax) {
  return amax == 0.0f ? 1.0f : Fp8Fmt<FMT>::kMax / amax;
}
template <int FMT>
__device__ __forceinline__ float scale_from_amax(float amax) {
  return amax == 0.0f ? 1.0f : amax / Fp8Fmt<FMT>::kMax;
}

template <int FMT>
__device__ __forceinline__ uint32_t encode4(f32x4_t x, float m) {
  return encode_fp8<FMT>(x[0] * m) | (encode_fp8<FMT>(x[1] * m) << 8) |
         (encode_fp8<FMT>(x[2] * m) << 16) | (encode_fp8<FMT>(x[3] * m) << 24);
}

// When amax and m are both finite, every product x*m of the block is finite
// and at most about FMAX, and the hardware conversion after a clamp to +-FMAX
// (cvt4_fp8) is exactly the saturating RNE encoder (pinned against the
// oracle's encoder by a GPU test) at a few instructions per value.  A block
// with NaN or Inf, or a subnormal amax (m = FMAX / amax overflows, 0 * m is
// NaN), keeps the integer encoder.
__device__ __forceinline__ bool hw_encode_ok(float amax, float m) {
  return amax < __builtin_huge_valf() && m < __builtin_huge_valf();
}

// ---- per tensor -----------------------------------------------------------

__device__ __forceinline__ uint32_t amax4(const f32x4_t& v) {
  return max(max(abs_bits(v[0]), abs_bits(v[1])), max(abs_bits(v[2]), abs_bits(v[3])));
}

// Workgroup-wide max of one value per thread (every thread gets the result).
template <int NT>
__device__ __forceinline__ uint32_t block_max(uint32_t m) {
  __shared__ uint32_t red[NT / 64];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t b = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) b = max(b, red[w]);
  return b;
}

// Contiguous tensor (ldx == ldq == cols): a flat grid-stride walk, 8 float4
// loads in flight per thread.  Pass 1 reads with ordinary loads, so a tensor
// that fits the 256 MB Infinity Cache is still there for pass 2; pass 2 reads
// nontemporally (its reads are the last).
constexpr int kFlatThreads = 1024;
constexpr int kFlatGrid = 256;     // one workgroup per CU
constexpr int kRowsGrid = 512;     // strided rows: at most this many workgroups
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kFlatThreads) void amax_flat(const f32x4_t* X, int64_t n4,
                                                          uint32_t* part) {
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * kFlatThreads;
  int64_t i = (int64_t)blockIdx.x * kFlatThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n4; i += kUnroll * stride) {
    f32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = X[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) m = max(m, amax4(v[u]));
  }
  for (; i < n4; i += stride) m = max(m, amax4(X[i]));
  m = block_max<kFlatThreads>(m);
  if (threadIdx.x == 0) part[blockIdx.x] = m;
}

// The tensor's amax: the max of the nparts slots pass 1 wrote.
template <int NT>
__device__ __forceinline__ float gather_amax(const uint32_t* part, int nparts) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < nparts; i += NT) m = max(m, part[i]);
  return __uint_as_float(block_max<NT>(m));
}

template <int FMT>
__global__ __launch_bounds__(kFlatThreads) void encode_flat(const f32x4_t* X, int64_t n4,
                                                            uint32_t* Q4, const uint32_t* part,
                                                            int nparts, float* scales) {
  const float amax = gather_amax<kFlatThreads>(part, nparts);
  const float m = mult_from_amax<FMT>(amax);
  if (blockIdx.x == 0 && threadIdx.x == 0) scales[0] = scale_from_amax<FMT>(amax);
  const int64_t stride = (int64_t)gridDim.x * kFlatThreads;
  int64_t i = (int64_t)blockIdx.x * kFlatThreads + threadIdx.x;
  if (hw_encode_ok(amax, m)) {
    for (; i + (kUnroll - 1) * stride < n4; i += kUnroll * stride) {
      f32x4_t v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(X + i + u * stride);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) Q4[i + u * stride] = cvt4_fp8<FMT>(v[u] * m);
    }
    for (; i < n4; i += stride) Q4[i] = cvt4_fp8<FMT>(__builtin_nontemporal_load(X + i) * m);
    return;
  }
  for (; i + (kUnroll - 1) * stride < n4; i += kUnroll * stride) {
    f32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(X + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) Q4[i + u * stride] = encode4<FMT>(v[u], m);
  }
  for (; i < n4; i += stride) Q4[i] = encode4<FMT>(__builtin_nontemporal_load(X + i), m);
}

// One pass for a contiguous tensor that the grid can hold in registers
// (kResident float4 per thread, the grid at most one workgroup per compute
// unit).  Each workgroup loads its share once and keeps it, stores the max of
// its |x| bit patterns in its own 64-bit slot tagged with the call's epoch,
// and counts itself in: first in the counter of its group of kGroupSize
// workgroups, and the group's last arrival then in the top counter (two
// short chains of increments on one address each instead of one as long as
// the grid).  The workgroup that completes the top count reads every slot,
// waiting for each to carry this call's tag, takes the tensor's amax, stores
// the scale, advances the epoch, and releases each other workgroup by
// swapping its state word from kWaiting (0) to kReleased with the amax in the
// upper half; each then encodes the share it still holds.  X is read once.
// Nothing that passes between workgroups relies on the order of two
// different words becoming visible: the amax travels in tagged slots and in
// the state words, so no fence is needed (an agent-scope fence writes back
// and invalidates the XCD's L2; one per arrival cost about 3 us here), and
// the counters take plain increments (compare-and-swap loops on one word,
// contended by 32 workgroups, cost more than the fences).
//
// The grid is sized so that every workgroup can be resident at once, but
// nothing guarantees it (another kernel may hold compute units).  So every
// wait is bounded: a workgroup that sees no release after spin_limit polls
// swaps kWaiting for kGaveUp and exits, and the last arrival, whose swap then
// fails, encodes that workgroup's share from X itself.  Each state word has
// one swap that succeeds, so every share is encoded exactly once, and every
// workgroup exits.  A slot whose tag never arrives (which the counters rule
// out) would count as NaN, so such a failure could not pass unseen.
//
// The sync area is zero before the first call.  Every call leaves the
// counters and state words zero (each counter is cleared by the arrival that
// completes it, a released workgroup clears its own state word, the last
// arrival those of the workgroups that gave up) and the epoch advanced; a
// slot's tag is the epoch plus one, so the zeroed slots never match.  32-bit
// word offsets: top counter 0, epoch 1, group g's counter kSyncGroup + 16 g
// (64 bytes apart), workgroup w's slot kSyncSlot + 2 w and state
// kSyncState + 2 w.
constexpr int kResident = 16;           // float4 per thread held in registers
constexpr int kGroupSize = 32;          // workgroups per first-level counter
constexpr int kMaxResidentGrid = 512;
constexpr int kSyncGroup = 16;
constexpr int kSyncSlot = kSyncGroup + 16 * (kMaxResidentGrid / kGroupSize);
constexpr int kSyncState = kSyncSlot + 2 * kMaxResidentGrid;
static_assert(kSyncSlot % 2 == 0 && kSyncState % 2 == 0 &&
                  kSyncState + 2 * kMaxResidentGrid <= kQuantizeSyncSlots,
              "sync area");
constexpr uint64_t kWaiting = 0, kReleased = 2, kGaveUp = 3;
constexpr int kSpinLimit = 4096;        // polls before a waiting workgroup gives up
constexpr int kSlotPolls = 1 << 16;     // polls of one slot by the last arrival

template <int FMT>
__global__ __launch_bounds__(kFlatThreads) void quant_tensor_resident(const f32x4_t* X,
                                                                      int64_t n4, uint32_t* Q4,
                                                                      uint32_t* sync,
                                                                      float* scales,
                                                                      int spin_limit) {
  constexpr int kScope = __HIP_MEMORY_SCOPE_AGENT;
  uint32_t epoch = 0;
  if (threadIdx.x == 0) epoch = __hip_atomic_load(&sync[1], __ATOMIC_RELAXED, kScope);
  const int64_t stride = (int64_t)gridDim.x * kFlatThreads;
  const int64_t i0 = (int64_t)blockIdx.x * kFlatThreads + threadIdx.x;
  f32x4_t v[kResident];
#pragma unroll
  for (int u = 0; u < kResident; ++u) {
    const int64_t i = i0 + u * stride;
    v[u] = i < n4 ? __builtin_nontemporal_load(X + i) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  uint32_t mx = 0;
#pragma unroll
  for (int u = 0; u < kResident; ++u) mx = max(mx, amax4(v[u]));
  mx = block_max<kFlatThreads>(mx);

  uint64_t* slot = (uint64_t*)(sync + kSyncSlot);
  uint64_t* state = (uint64_t*)(sync + kSyncState);
  __shared__ uint32_t s_last, s_run, s_amax, s_ngone, s_tag;
  __shared__ uint32_t s_gone[kMaxResidentGrid];
  if (threadIdx.x == 0) {
    const uint32_t w = blockIdx.x, grid = gridDim.x, tag = epoch + 1;
    __hip_atomic_store(&slot[w], ((uint64_t)tag << 32) | mx, __ATOMIC_RELAXED, kScope);
    const uint32_t g = w / kGroupSize, in_g = min(grid - g * kGroupSize, (uint32_t)kGroupSize);
    uint32_t* gc = &sync[kSyncGroup + 16 * g];
    bool last = false;
    if (__hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, kScope) == in_g - 1) {
      __hip_atomic_store(gc, 0u, __ATOMIC_RELAXED, kScope);
      const uint32_t groups = (grid + kGroupSize - 1) / kGroupSize;
      last = __hip_atomic_fetch_add(&sync[0], 1u, __ATOMIC_RELAXED, kScope) == groups - 1;
      if (last) {
        __hip_atomic_store(&sync[0], 0u, __ATOMIC_RELAXED, kScope);
        __hip_atomic_store(&sync[1], tag, __ATOMIC_RELAXED, kScope);  // the next call's epoch
      }
    }
    s_last = last;
    s_tag = tag;
    s_ngone = 0;
  }
  __syncthreads();
  if (s_last) {
    // every workgroup has counted itself in after storing its slot; a slot
    // still showing an older tag is a store not yet visible here
    uint32_t a = 0;
    for (uint32_t w = threadIdx.x; w < gridDim.x; w += kFlatThreads) {
      uint64_t sv = __hip_atomic_load(&slot[w], __ATOMIC_RELAXED, kScope);
      for (int it = 0; it < kSlotPolls && (uint32_t)(sv >> 32) != s_tag; ++it) {
        __builtin_amdgcn_s_sleep(1);
        sv = __hip_atomic_load(&slot[w], __ATOMIC_RELAXED, kScope);
      }
      a = max(a, (uint32_t)(sv >> 32) == s_tag ? (uint32_t)sv : 0x7FC00000u);
    }
    a = block_max<kFlatThreads>(a);
    if (threadIdx.x == 0) {
      scales[0] = scale_from_amax<FMT>(__uint_as_float(a));
      s_amax = a;  // read after the barrier below
    }
    const uint64_t rel = kReleased | ((uint64_t)a << 32);
    for (uint32_t w = threadIdx.x; w < gridDim.x; w += kFlatThreads) {
      if (w == blockIdx.x) continue;
      uint64_t expect = kWaiting;
      if (!__hip_atomic_compare_exchange_strong(&state[w], &expect, rel, __ATOMIC_RELAXED,
                                                __ATOMIC_RELAXED, kScope)) {
        // it gave up and exited: its share is encoded here
        s_gone[atomicAdd(&s_ngone, 1u)] = w;
        __hip_atomic_store(&state[w], kWaiting, __ATOMIC_RELAXED, kScope);
      }
    }
    __syncthreads();
    const float amax = __uint_as_float(a);
    const float m = mult_from_amax<FMT>(amax);
    const bool hw = hw_encode_ok(amax, m);
    for (uint32_t g = 0; g < s_ngone; ++g) {
      const int64_t j0 = (int64_t)s_gone[g] * kFlatThreads + threadIdx.x;
      for (int u = 0; u < kResident; ++u) {
        const int64_t i = j0 + u * stride;
        if (i < n4)
          __builtin_nontemporal_store(hw ? cvt4_fp8<FMT>(X[i] * m) : encode4<FMT>(X[i], m), Q4 + i);
      }
    }
  } else {
    if (threadIdx.x == 0) {
      uint64_t st = kWaiting;
      for (int it = 0; it < spin_limit && st == kWaiting; ++it) {
        __builtin_amdgcn_s_sleep(2);
        st = __hip_atomic_load(&state[blockIdx.x], __ATOMIC_RELAXED, kScope);
      }
      if (st == kWaiting) {
        uint64_t expect = kWaiting;
        st = __hip_atomic_compare_exchange_strong(&state[blockIdx.x], &expect, kGaveUp,
                                                  __ATOMIC_RELAXED, __ATOMIC_RELAXED, kScope)
                 ? kGaveUp
                 : expect;  // released after the last poll
      }
      // a released workgroup clears its own state word; a given-up one is
      // cleared by the last arrival
      if (st != kGaveUp) __hip_atomic_store(&state[blockIdx.x], kWaiting, __ATOMIC_RELAXED, kScope);
      s_run = st != kGaveUp;
      s_amax = (uint32_t)(st >> 32);
    }
    __syncthreads();
    if (!s_run) return;
  }
  // Q is written with streaming stores: its 16.8 MB (at 4096^2) would
  // otherwise sit dirty in the L2s and be written back at the kernel's end,
  // after the last encode (2.1 us more per call here)
  const float amax = __uint_as_float(s_amax);
  const float m = mult_from_amax<FMT>(amax);
  if (hw_encode_ok(amax, m)) {
#pragma unroll
    for (int u = 0; u < kResident; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < n4) __builtin_nontemporal_store(cvt4_fp8<FMT>(v[u] * m), Q4 + i);
    }
  } else {
#pragma unroll
    for (int u = 0; u < kResident; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < n4) __builtin_nontemporal_store(encode4<FMT>(v[u], m), Q4 + i);
    }
  }
}

// Strided rows: workgroup b walks rows b, b + grid, ..., threads striding
// over each row's float4 columns.
__global__ __launch_bounds__(256) void amax_rows(const float* X, int64_t rows, int64_t cols4,
                                                 int64_t ldx, uint32_t* part) {
  uint32_t m = 0;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const float* row = X + r * ldx;
    int64_t c = threadIdx.x;
    for (; c + 768 < cols4; c += 1024) {
      f32x4_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = *(const f32x4_t*)(row + 4 * (c + 256 * u));
#pragma unroll
      for (int u = 0; u < 4; ++u) m = max(m, amax4(v[u]));
    }
    for (; c < cols4; c += 256) m = max(m, amax4(*(const f32x4_t*)(row + 4 * c)));
  }
  m = block_max<256>(m);
  if (threadIdx.x == 0) part[blockIdx.x] = m;
}

template <int FMT>
__global__ __launch_bounds__(256) void encode_rows(const float* X, int64_t rows, int64_t cols4,
                                                   int64_t ldx, uint8_t* Q, int64_t ldq,
                                                   const uint32_t* part, int nparts,
                                                   float* scales) {
  const float amax = gather_amax<256>(part, nparts);
  const float m = mult_from_amax<FMT>(amax);
  if (blockIdx.x == 0 && threadIdx.x == 0) scales[0] = scale_from_amax<FMT>(amax);
  if (hw_encode_ok(amax, m)) {
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
      const float* row = X + r * ldx;
      uint8_t* qrow = Q + r * ldq;
      int64_t c = threadIdx.x;
      for (; c + 768 < cols4; c += 1024) {
        f32x4_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *(const f32x4_t*)(row + 4 * (c + 256 * u));
#pragma unroll
        for (int u = 0; u < 4; ++u) *(uint32_t*)(qrow + 4 * (c + 256 * u)) = cvt4_fp8<FMT>(v[u] * m);
      }
      for (; c < cols4; c += 256)
        *(uint32_t*)(qrow + 4 * c) = cvt4_fp8<FMT>(*(const f32x4_t*)(row + 4 * c) * m);
    }
    return;
  }
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const float* row = X + r * ldx;
    uint8_t* qrow = Q + r * ldq;
    int64_t c = threadIdx.x;
    for (; c + 768 < cols4; c += 1024) {
      f32x4_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = *(const f32x4_t*)(row + 4 * (c + 256 * u));
#pragma unroll
      for (int u = 0; u < 4; ++u) *(uint32_t*)(qrow + 4 * (c + 256 * u)) = encode4<FMT>(v[u], m);
    }
    for (; c < cols4; c += 256)
      *(uint32_t*)(qrow + 4 * c) = encode4<FMT>(*(const f32x4_t*)(row + 4 * c), m);
  }
}

// ---- 1 x 128 blocks -------------------------------------------------------
// Workgroup (x, y) walks rows y, y + gridDim.y, ...; in each it covers
// kRounds chunks of 1024 columns starting at x * 1024 * kRounds, thread t
// taking columns 4t .. 4t+3 of every chunk, so the 32 lanes of a half-wave
// own one block and no division is needed.  Loads of all rounds are issued
// first; X is read once, with nontemporal loads.
constexpr int kRounds = 4;
template <int FMT>
__global__ __launch_bounds__(256) void quant_1x128(const float* X, int64_t rows, int64_t cols,
                                                   int64_t ldx, uint8_t* Q, int64_t ldq,
                                                   float* scales) {
  const int lane = threadIdx.x & 31;
  const int64_t nbc = cols / 128;
  const int64_t c0 = (int64_t)blockIdx.x * (1024 * kRounds) + 4 * threadIdx.x;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const float* xr = X + r * ldx;
    f32x4_t v[kRounds];
#pragma unroll
    for (int u = 0; u < kRounds; ++u) {
      const int64_t c = c0 + u * 1024;
      v[u] = c < cols ? __builtin_nontemporal_load((const f32x4_t*)(xr + c))
                      : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kRounds; ++u) {
      const int64_t c = c0 + u * 1024;
      const uint32_t m = half_wave_max(amax4(v[u]));
      if (c < cols) {  // cols % 128 == 0: a block is entirely in or out
        const float amax = __uint_as_float(m);
        const float mult = mult_from_amax<FMT>(amax);
        *(uint32_t*)(Q + r * ldq + c) =
            hw_encode_ok(amax, mult) ? cvt4_fp8<FMT>(v[u] * mult) : encode4<FMT>(v[u], mult);
        if (lane == 0) scales[r * nbc + c / 128] = scale_from_amax<FMT>(amax);
      }
    }
  }
}

// ---- 128 x 128 blocks -----------------------------------------------------
template <int FMT>
__global__ __launch_bounds__(256) void quant_128x128(const float* X, int64_t nbc, int64_t ldx,
                                                     uint8_t* Q, int64_t ldq, float* scales) {
  const int64_t bi = blockIdx.x / nbc, bj = blockIdx.x - (blockIdx.x / nbc) * nbc;
  const int t = threadIdx.x, c4 = t & 31, r0 = t >> 5;  // rows r0, r0+8, ... ; float4 column c4
  const float* base = X + (bi * 128) * ldx + bj * 128 + 4 * c4;
  f32x4_t v[16];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = *(const f32x4_t*)(base + (int64_t)(r0 + 8 * i) * ldx);
    m = max(m, max(max(abs_bits(v[i][0]), abs_bits(v[i][1])),
                   max(abs_bits(v[i][2]), abs_bits(v[i][3]))));
  }
  m = wave_max(m);
  __shared__ uint32_t red[4];
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  m = max(max(red[0], red[1]), max(red[2], red[3]));
  const float amax = __uint_as_float(m);
  const float mult = mult_from_amax<FMT>(amax);
  uint8_t* qb = Q + (bi * 128) * ldq + bj * 128 + 4 * c4;
  if (hw_encode_ok(amax, mult)) {  // uniform over the workgroup
#pragma unroll
    for (int i = 0; i < 16; ++i)
      *(uint32_t*)(qb + (int64_t)(r0 + 8 * i) * ldq) = cvt4_fp8<FMT>(v[i] * mult);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      *(uint32_t*)(qb + (int64_t)(r0 + 8 * i) * ldq) = encode4<FMT>(v[i], mult);
  }
  if (t == 0) scales[blockIdx.x] = scale_from_amax<FMT>(amax);
}

// ---- MX: 1 x 32 blocks, E8M0 scale codes ---------------------------------
// Workgroup (x, y) walks rows y, y + gridDim.y, ...; in each it covers
// kRounds chunks of 1024 columns starting at x * 1024 * kRounds, thread t
// taking columns 4t .. 4t+3 of every chunk, so 8 consecutive lanes own one
// block and no division is needed.  Loads of all rounds are issued first; X
// is read once, with nontemporal loads.
template <int FMT>
__global__ __launch_bounds__(256) void quant_mx(const float* X, int64_t rows, int64_t cols,
                                                int64_t ldx, uint8_t* Q, int64_t ldq, uint8_t* S,
                                                int64_t lds) {
  constexpr uint32_t kEmax = FMT == 0 ? 8u : FMT == 1 ? 15u : 2u;
  const int sub = threadIdx.x & 7;
  const int64_t c0 = (int64_t)blockIdx.x * (1024 * kRounds) + 4 * threadIdx.x;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const float* xr = X + r * ldx;
    f32x4_t v[kRounds];
#pragma unroll
    for (int u = 0; u < kRounds; ++u) {
      const int64_t c = c0 + u * 1024;
      v[u] = c < cols ? __builtin_nontemporal_load((const f32x4_t*)(xr + c))
                      : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kRounds; ++u) {
      const int64_t c = c0 + u * 1024;
      uint32_t m = amax4(v[u]);
#pragma unroll
      for (int o = 4; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
      if (c < cols) {  // cols % 32 == 0: a block is entirely in or out
        uint32_t code, q;
        if (m >= 0x7F800000u) {  // Inf or NaN in the block
          code = 255u;
          q = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t sgn = __float_as_uint(v[u][e]) >> 24 & 0x80u;
            q |= FMT == 4 ? (sgn >> 4) << (4 * e) : (sgn | 0x7Fu) << (8 * e);
          }
        } else {
          const uint32_t eb = m >> 23;  // biased exponent of amax (0: zero or subnormal)
          code = eb > kEmax ? eb - kEmax : 0u;
          const float mult = __uint_as_float((254u - code) << 23);
          // finite block, normal power-of-two multiplier: every product is
          // finite, where the clamped hardware conversion is the encoder
          if constexpr (FMT == 4)
            q = cvt4_fp4(v[u] * mult);
          else
            q = cvt4_fp8<FMT>(v[u] * mult);
        }
        if constexpr (FMT == 4)
          *(uint16_t*)(Q + r * ldq + c / 2) = (uint16_t)q;
        else
          *(uint32_t*)(Q + r * ldq + c) = q;
        if (sub == 0) S[r * lds + c / 32] = (uint8_t)code;
      }
    }
  }
}

// Per-tensor geometry: contiguous tensors take the flat walk, others rows.
struct TensorPasses {
  bool flat;
  int nparts;  // pass-1 workgroups = scratch slots
};

TensorPasses tensor_passes(int64_t rows, int64_t cols, int64_t ldx, int64_t ldq) {
  TensorPasses t;
  t.flat = ldx == cols && ldq == cols;
  t.nparts = t.flat ? kFlatGrid : (int)(rows < kRowsGrid ? rows : kRowsGrid);
  return t;
}

// The two per-tensor passes.  `done`, when given, is recorded by the second
// kernel's own completion (hipExtLaunchKernelGGL's stop event): a separate
// event record between two calls would put a gap of its own between them.
// The one-pass kernel's grid for n4 float4, or 0 when the tensor is not
// contiguous or more than the resident grid can hold.
int64_t resident_grid(const TensorPasses& t, int64_t n4, hipStream_t s) {
  if (!t.flat || n4 < 1) return 0;
  const int64_t cus = compute_units(s), need = (n4 + kFlatThreads - 1) / kFlatThreads;
  const int64_t grid = need < cus ? need : cus;
  if (grid < 1 || grid > kMaxResidentGrid || n4 > grid * kFlatThreads * kResident) return 0;
  return grid;
}

template <int FMT>
void launch_tensor(const float* X, int64_t rows, int64_t cols, int64_t ldx, uint8_t* Q,
                   int64_t ldq, float* scales, uint32_t* part, const TensorPasses& t,
                   hipStream_t s, hipEvent_t done, int spin_limit) {
  const int64_t cols4 = cols / 4;
  if (t.flat) {
    const int64_t n4 = rows * cols4;
    if (const int64_t grid = resident_grid(t, n4, s)) {
      hipExtLaunchKernelGGL(quant_tensor_resident<FMT>, dim3((unsigned)grid), dim3(kFlatThreads),
                            0, s, nullptr, done, 0, (const f32x4_t*)X, n4, (uint32_t*)Q,
                            part + kQuantizeScratchSlots, scales, spin_limit);
      return;
    }
    hipLaunchKernelGGL(amax_flat, dim3((unsigned)t.nparts), dim3(kFlatThreads), 0, s,
                       (const f32x4_t*)X, n4, part);
    hipExtLaunchKernelGGL(encode_flat<FMT>, dim3((unsigned)t.nparts), dim3(kFlatThreads), 0, s,
                          nullptr, done, 0, (const f32x4_t*)X, n4, (uint32_t*)Q,
                          (const uint32_t*)part, t.nparts, scales);
  } else {
    hipLaunchKernelGGL(amax_rows, dim3((unsigned)t.nparts), dim3(256), 0, s, X, rows, cols4,
                       ldx, part);
    hipExtLaunchKernelGGL(encode_rows<FMT>, dim3((unsigned)t.nparts), dim3(256), 0, s, nullptr,
                          done, 0, X, rows, cols4, ldx, Q, ldq, (const uint32_t*)part, t.nparts,
                          scales);
  }
}

template <int FMT>
hipError_t launch_fmt(const float* X, int64_t rows, int64_t cols, int64_t ldx, int64_t br,
                      int64_t bc, uint8_t* Q, int64_t ldq, float* scales, uint32_t* part,
                      hipStream_t s, hipEvent_t done = nullptr, int spin_limit = kSpinLimit) {
  if (br == rows && bc == cols) {
    launch_tensor<FMT>(X, rows, cols, ldx, Q, ldq, scales, part,
                       tensor_passes(rows, cols, ldx, ldq), s, done, spin_limit);
  } else if (br == 1 && bc == 128) {
    const dim3 grid((unsigned)((cols + 1024 * kRounds - 1) / (1024 * kRounds)),
                    (unsigned)(rows < 65535 ? rows : 65535));
    hipLaunchKernelGGL(quant_1x128<FMT>, grid, dim3(256), 0, s, X, rows, cols, ldx, Q, ldq, scales);
  } else {
    const int64_t nbc = cols / 128, nblk = (rows / 128) * nbc;
    hipLaunchKernelGGL(quant_128x128<FMT>, dim3((unsigned)nblk), dim3(256), 0, s, X, nbc, ldx, Q,
                       ldq, scales);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_mxfp8(const float* X, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                                 uint8_t* Q, int64_t ldq, uint8_t* S, int64_t lds, hipStream_t s) {
  const dim3 grid((unsigned)((cols + 1024 * kRounds - 1) / (1024 * kRounds)),
                  (unsigned)(rows < 65535 ? rows : 65535));
  if (fmt == 0)
    hipLaunchKernelGGL(quant_mx<0>, grid, dim3(256), 0, s, X, rows, cols, ldx, Q, ldq, S, lds);
  else
    hipLaunchKernelGGL(quant_mx<1>, grid, dim3(256), 0, s, X, rows, cols, ldx, Q, ldq, S, lds);
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp4(const float* X, int64_t rows, int64_t cols, int64_t ldx,
                                 uint8_t* Q, int64_t ldq_bytes, uint8_t* S, int64_t lds,
                                 hipStream_t s) {
  const dim3 grid((unsigned)((cols + 1024 * kRounds - 1) / (1024 * kRounds)),
                  (unsigned)(rows < 65535 ? rows : 65535));
  hipLaunchKernelGGL(quant_mx<4>, grid, dim3(256), 0, s, X, rows, cols, ldx, Q, ldq_bytes, S,
                     lds);
  return hipGetLastError();
}

int64_t quantize_scratch_slots(int64_t rows, int64_t cols, int64_t ldx, int64_t ldq,
                               int64_t br, int64_t bc) {
  if (br != rows || bc != cols) return 0;  // block scales need no scratch
  return tensor_passes(rows, cols, ldx, ldq).nparts;
}

hipError_t launch_quantize_fp8(const float* X, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                               int64_t br, int64_t bc, uint8_t* Q, int64_t ldq, float* scales,
                               uint32_t* part, hipStream_t s) {
  if (fmt == 0) return launch_fmt<0>(X, rows, cols, ldx, br, bc, Q, ldq, scales, part, s);
  return launch_fmt<1>(X, rows, cols, ldx, br, bc, Q, ldq, scales, part, s);
}

// ---- scratch of the per-tensor passes --------------------------------------

int device_of(hipStream_t s, hipError_t* e) {
  hipDevice_t dev = 0;
  *e = hipStreamGetDevice(s, &dev);
  return dev;
}

// Compute units of the stream's GPU, looked up once per device; 0 if the
// query fails (the per-tensor quantizer then takes its two-pass walk).
int compute_units(hipStream_t s) {
  static std::atomic<int> cached[kMaxDevices];
  hipError_t e;
  const int dev = device_of(s, &e);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// quantize_fp8 (the allocating entry point): one workspace of
// kQuantizeScratchWords words per GPU, allocated and zeroed on the first
// per-tensor call on that GPU and kept until the process ends.  Calls on
// different streams would otherwise share it concurrently, so every call
// first makes its stream wait for the previous call's completion event; its
// last kernel records that event when it completes.
hipError_t launch_quantize_fp8_tensor_ws(const float* X, int64_t rows, int64_t cols, int64_t ldx,
                                         int fmt, uint8_t* Q, int64_t ldq, float* scales,
                                         hipStream_t s) {
  struct Workspace {
    uint32_t* slots = nullptr;
    hipEvent_t done = nullptr;  // recorded after each call's last kernel
    hipStream_t last = nullptr;
    bool used = false;
  };
  static std::mutex mu;
  static Workspace ws[kMaxDevices];
  hipError_t e;
  const int dev = device_of(s, &e);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  Workspace& w = ws[dev];
  if (!w.slots) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    e = hipMalloc((void**)&w.slots, kQuantizeScratchWords * sizeof(uint32_t));
    // the one-pass kernel's sync words start at zero (every call leaves them so)
    if (e == hipSuccess) e = hipMemset(w.slots, 0, kQuantizeScratchWords * sizeof(uint32_t));
    if (e == hipSuccess) e = hipEventCreate(&w.done);
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) {
      if (w.slots) (void)hipFree(w.slots);
      w.slots = nullptr;
      return e;
    }
  }
  // a call on the stream that used the workspace last is ordered after it
  // already; another stream waits for that call's completion first
  if (w.used && s != w.last && (e = hipStreamWaitEvent(s, w.done, 0)) != hipSuccess) return e;
  e = fmt == 0 ? launch_fmt<0>(X, rows, cols, ldx, rows, cols, Q, ldq, scales, w.slots, s, w.done)
               : launch_fmt<1>(X, rows, cols, ldx, rows, cols, Q, ldq, scales, w.slots, s, w.done);
  if (e != hipSuccess) return e;
  w.used = true;
  w.last = s;
  return hipSuccess;
}

// ---- the allocation-free entry point's scratch ----------------------------
// For callers that cannot allocate device memory (code under graph capture,
// serving loops, harnesses that forbid hipMalloc): the per-tensor pass-1
// slots and the one-pass kernel's sync words live in this file-scope array,
// one copy per GPU, zero when the library loads and held until the process
// ends.  Host code never passes the array's name to a kernel (on the
// host it is a stand-in, not a device address): it asks once per device, with
// that device current, for the array's address on that device and passes
// that.  Calls that overlap on one GPU share the array and race.
static __device__ __align__(256) uint32_t scratch[kQuantizeScratchWords];  // zero at load
static_assert(kFlatGrid <= kQuantizeScratchSlots && kRowsGrid <= kQuantizeScratchSlots,
              "every per-tensor pass-1 grid fits the scratch");

hipError_t quantize_scratch_address(hipStream_t s, uint32_t** out) {
  static std::mutex mu;
  static uint32_t* addr[kMaxDevices] = {};
  hipError_t e;
  const int device = device_of(s, &e);
  if (e != hipSuccess) return e;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != device) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    addr[device] = (uint32_t*)p;
  }
  *out = addr[device];
  return hipSuccess;
}

// The one-pass per-tensor kernel with a chosen wait bound, on the
// allocation-free scratch.  Diagnostic: a bound of 0 makes waiting
// workgroups give up at once, so the last arrival encodes their shares.
hipError_t launch_probe_quantize_resident(const float* X, int64_t rows, int64_t cols, int fmt,
                                          uint8_t* Q, float* scale, int spin_limit,
                                          hipStream_t s) {
  if (!resident_grid(tensor_passes(rows, cols, cols, cols), rows * (cols / 4), s))
    return hipErrorInvalidValue;
  uint32_t* part = nullptr;
  const hipError_t e = quantize_scratch_address(s, &part);
  if (e != hipSuccess) return e;
  return fmt == 0 ? launch_fmt<0>(X, rows, cols, cols, rows, cols, Q, cols, scale, part, s,
                                  nullptr, spin_limit)
                  : launch_fmt<1>(X, rows, cols, cols, rows, cols, Q, cols, scale, part, s,
                                  nullptr, spin_limit);
}

}  // namespace dmu
