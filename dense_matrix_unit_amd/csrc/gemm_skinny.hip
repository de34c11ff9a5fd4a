// Skinny-M BF16 GEMM for gfx950: D = A*B (+ C) with M <= 128 and B stored
// N x K, the shape of a decode-time linear layer (few activation rows against
// a large weight matrix).
//
// Such a product does little arithmetic per byte of B, so its bound is HBM
// bandwidth, not the matrix unit: the page "How Blackwell's Tensor Memory
// Actually Works" (thesoftwarefrontier.com), section "What this does to
// serving economics", makes the point that a decode step is a GEMM whose M
// (the batch) is skinny, so most of the matrix instruction's M dimension is
// empty and the cost sits in reading the weights.  The design therefore
// aims to keep B streaming at full bandwidth and treats the MFMAs as cheap:
//  * a workgroup of 7 waves owns 112 columns of D (16 per wave), so N = 28672
//    gives exactly 256 workgroups, one per CU;
//  * every wave streams its own 16 rows of B straight into registers (no LDS
//    round trip), 16 bytes per lane per 32-wide K step, in a ring of K
//    chunks.  For M <= 64 a chunk is 256 K wide and the ring holds two (one
//    in flight while one is multiplied); M = 128, whose A stages would not
//    fit in LDS at 256, takes three 128-wide chunks.  The longer run of each
//    B row per chunk took M = 16 from 97.4 to 94.4 us and M = 64 from 101.1
//    to 97.4 us (N = 28672, K = 8192, bit-identical output), and the shorter
//    ring another 1-2%; 512-wide chunks were slower at M = 16;
//  * A (at most 128 x K) is shared by the workgroup through LDS, one K chunk
//    per stage, copied with buffer loads that write LDS directly; its
//    16-byte chunks are XOR-swizzled with the row index so the MFMA fragment
//    reads are bank-conflict free.  There is one A stage more than the ring
//    holds chunks, so the copy of chunk c + ring goes into the stage of chunk
//    c - 1, which every wave has finished reading by the barrier that opens
//    chunk c: one barrier per chunk instead of two, and the copy leaves before
//    chunk c is multiplied (128.3 -> 117.6 us at M = 128, N = 28672,
//    K = 8192, bit-identical output);
//  * the MFMA is 16x16x32 BF16 with the B fragment as the first operand, so
//    each lane ends up holding 4 consecutive output columns of one row.
#include "dmu_device.h"
#include "dmu_internal.h"

namespace dmu {
namespace {

constexpr int kWaves = 7;
constexpr int kThreads = kWaves * 64;
constexpr int kBN = kWaves * 16;  // columns of D per workgroup

// kNB: chunks in the ring (kNB-1 in flight while one is multiplied); enough
// bytes must be in flight per CU to cover HBM latency at full bandwidth.
// kKC: K elements per chunk.
template <int MB, int kNB, int kKC>
__global__ __launch_bounds__(kThreads) void gemm_skinny_kernel(GemmArgs p) {
  constexpr int kRowB = kKC * 2;    // bytes per A row per chunk
  constexpr int kSteps = kKC / 32;  // 16x16x32 MFMA steps per chunk
  // LDS position of 16-byte chunk c of A row r: flip the low four bits of c
  // with the row, so 16 consecutive rows at the same c hit 16 distinct
  // 16-byte bank groups.
  auto aswz = [](int r, int c) { return c ^ (r & (kRowB / 16 - 1) & 15); };
  static_assert(MB % 16 == 0 && MB <= 128, "rows");
  constexpr int MT = MB / 16;                  // 16-row MFMA blocks
  constexpr int A_STAGE = MB * kRowB;          // bytes of one A chunk
  constexpr int NLA = MB * (kRowB / 16) / 256; // A copies per thread (first 4 waves)
  constexpr int NA = kNB + 1;                 // A stages: one more than the ring
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NA * A_STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g16 = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * kBN + wave * 16;
  const int64_t kbytes = p.K * 2;
  const int nch = (int)((p.K + kKC - 1) / kKC);

  // ---- B: this wave's 16 rows, lane reads row n0 + r16, 16 bytes at k-group g16
  const int64_t rowsB = p.N - n0;  // may be <= 0 for the last workgroup's idle waves
  const uint32_t ldbB = (uint32_t)(p.ldb * 2);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(
      (const uint8_t*)p.B + (rowsB > 0 ? n0 : 0) * p.ldb * 2,
      rowsB > 0 ? (min(rowsB, (int64_t)16) - 1) * ldbB + kbytes : 0);
  const uint32_t voffB = r16 < rowsB ? (uint32_t)r16 * ldbB + (uint32_t)g16 * 16 : kOOB;

  // ---- A: rows 0..M-1, copied into LDS by the first 4 waves
  const __amdgpu_buffer_rsrc_t rA =
      make_rsrc(p.A, (int64_t)(p.M - 1) * p.lda * 2 + kbytes);
  uint32_t voffA[NLA > 0 ? NLA : 1], cA[NLA > 0 ? NLA : 1];
#pragma unroll
  for (int it = 0; it < NLA; ++it) {
    const int q = it * 256 + (tid & 255), row = q / (kRowB / 16), c = q % (kRowB / 16);
    const int src = aswz(row, c);  // chunk stored at position c comes from logical chunk src
    cA[it] = (uint32_t)src * 16;
    voffA[it] = row < p.M ? (uint32_t)row * (uint32_t)(p.lda * 2) + (uint32_t)src * 16 : kOOB;
  }

  auto load_a = [&](int ch, int st) __attribute__((always_inline)) {
    if (wave >= 4) return;
    const bool active = ch < nch;
    const uint32_t koff = active ? (uint32_t)ch * kRowB : 0u;
    const uint32_t klim = active ? (uint32_t)kbytes : 0u;
#pragma unroll
    for (int it = 0; it < NLA; ++it) {
      const uint32_t v = koff + cA[it] < klim ? voffA[it] : kOOB;
      buffer_load_lds16(rA, smem + st * A_STAGE + (it * 256 + wave * 64) * 16, v, koff);
    }
  };
  auto load_b = [&](int ch, u32x4_t* breg) __attribute__((always_inline)) {
    const bool active = ch < nch;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const uint32_t kb = (uint32_t)ch * kRowB + (uint32_t)s * 64;
      breg[s] = buffer_load16(rB, active && kb + g16 * 16 < (uint32_t)kbytes ? voffB : kOOB,
                              active ? kb : 0u);
    }
  };

  f32x4_t acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t breg[kNB][kSteps];

  auto compute = [&](int st, const u32x4_t* b) __attribute__((always_inline)) {
    const uint8_t* sA = smem + st * A_STAGE;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int row = i * 16 + r16;
        const i32x4_t a = *(const i32x4_t*)(sA + row * kRowB + aswz(row, 4 * s + g16) * 16);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b[s]),
                                                          __builtin_bit_cast(bf16x8_t, a), acc[i],
                                                          0, 0, 0);
      }
    }
  };

  // Ring of kNB chunks: A stage / B register buffer P holds chunks P, P+kNB, ...
  // Chunk c is consumed once only the kNB-1 younger chunks' copies are
  // pending; then its buffers are refilled with chunk c+kNB.
  constexpr int kPer = kSteps + NLA;  // copies per chunk issued by waves 0-3
#pragma unroll
  for (int P = 0; P < kNB; ++P) {
    load_a(P, P);
    load_b(P, breg[P]);
  }
  for (int ch = 0; ch < nch; ch += kNB) {
#pragma unroll
    for (int P = 0; P < kNB; ++P) {
      if (P > 0 && ch + P >= nch) break;
      if (wave < 4)
        __builtin_amdgcn_s_waitcnt((((kNB - 1) * kPer) & 0xF) | ((((kNB - 1) * kPer) >> 4) << 14) |
                                   (0x7 << 4));
      else
        __builtin_amdgcn_s_waitcnt((((kNB - 1) * kSteps) & 0xF) |
                                   ((((kNB - 1) * kSteps) >> 4) << 14) | (0x7 << 4));
      __syncthreads();  // chunk c landed; every wave is done with chunk c - 1
      const int c = ch + P;
      load_a(c + kNB, (c + kNB) % NA);  // into chunk c - 1's stage
      compute(c % NA, breg[P]);
      load_b(c + kNB, breg[P]);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);

  // lane l, register r of a transposed 16x16 accumulator: D[row = 16i + l%16][col = 4(l/16) + r]
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int64_t row = i * 16 + r16;
    const int64_t col = n0 + 4 * g16;
    if (row >= p.M || col >= p.N) continue;
    f32x4_t x = acc[i];
    const bool full = col + 3 < p.N;
    if (p.C) {
      const float* c = p.C + row * p.ldc + col;
      for (int r = 0; r < 4; ++r)
        if (full || col + r < p.N) x[r] += c[r];
    }
    if (p.out_bf16) {
      uint16_t* d = (uint16_t*)p.D + row * p.ldd + col;
      if (full) {
        *(uint2*)d = make_uint2(pack2_bf16(x[0], x[1]),
                                pack2_bf16(x[2], x[3]));
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
}

template <int MB, int NB, int KC>
hipError_t launch_mb(const GemmArgs& a, hipStream_t s) {
  const int64_t wgs = (a.N + kBN - 1) / kBN;
  hipLaunchKernelGGL((gemm_skinny_kernel<MB, NB, KC>), dim3((unsigned)wgs), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// the skinny kernel has no fused epilogue (bias, activation, FP8 output)
bool skinny_applies(const GemmArgs& a) {
  return a.M <= 128 && !a.bias && !a.act && a.out_fp8 < 0;
}

hipError_t launch_gemm_bf16_skinny(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 16) return launch_mb<16, 2, 256>(a, s);
  if (a.M <= 32) return launch_mb<32, 2, 256>(a, s);
  if (a.M <= 64) return launch_mb<64, 2, 256>(a, s);
  return launch_mb<128, 3, 128>(a, s);
}

}  // namespace dmu
