// FP8 GEMM with per-block scales for gfx950: A (M x K, E4M3 or E5M2) carries
// one FP32 dequantisation scale per row per 128-wide K block, B (stored N x K)
// one per 128 x 128 block; D = sum over K blocks kb of
// sa[i][kb] * sb[j/128][kb] * (A_kb B_kb^T)[i][j]  (+ C), FP32 accumulate.
//
// The page "Tensor Cores: Matrix Instructions, Swizzling and FP8, Measured"
// (vidyal.ai), Step 5, describes promotion: FP8 partial sums are formed from
// zero over a stretch of K by the matrix unit and then added into FP32
// registers, here with the block's two scales folded in.  The per-block
// scaling layout is the one the "Tensor Cores" chapter of ai-infra-handbooks
// ("Precision" section) lists among FP8 scaling granularities.
//
// On gfx950 one v_mfma_f32_16x16x128_f8f6f4 covers a whole 128-wide K block
// of a 16x16 sub-tile, so every MFMA produces one block's partial product P,
// from zero, and the promotion acc += P * (sa * sb) is four FMAs per lane.
// VALU instructions cannot read accumulator registers (AGPRs), so the
// accumulator lives in ordinary VGPRs; that caps a wave's tile at 128 x 64
// (128 VGPRs of accumulator), and the workgroup tile at 256 x 128:
//  * 4 waves (2 x 2), each a 128 x 64 quadrant of 8 x 4 sub-tiles;
//  * 128-byte K slices (one scale block) in a 3-stage LDS ring, copied with
//    buffer loads that write LDS directly, XOR-swizzled as in gemm.hip; the
//    slice's A scales (256 floats) and B scale ride along in the same ring;
//  * the MFMAs run in a software pipeline: MFMA g writes P buffer g % 4 and
//    the promotion of MFMA g-2 follows it, so the FMAs never wait on a
//    result that is still being computed; the copies of slice k+2 and an L2
//    prefetch of slice k+3 are spread between the MFMAs;
//  * the second half of a slice's MFMAs runs after the slice barrier, with
//    the next slice's fragment reads spread between them.
#include "gemm_common.h"

namespace dmu {
namespace {

constexpr int kBM = 256, kBN = 128, kRB = 128, kS = 3, kGroupM = 4, kPD = 3;
constexpr int kWM = kBM / 2, kWN = kBN / 2;     // wave tile 128 x 64
constexpr int kTM = kWM / 16, kTN = kWN / 16;   // 8 x 4 sub-tiles of 16 x 16
constexpr int kNM = kTM * kTN;                  // MFMAs per slice per wave
constexpr int kABytes = kBM * kRB, kBBytes = kBN * kRB;
constexpr int kSAOff = kABytes + kBBytes;       // 256 A-row scales (1 KB)
constexpr int kSBOff = kSAOff + kBM * 4;        // 4 x 256 B: one B-scale area per wave
constexpr int kStage = kSBOff + 4 * 256;
constexpr int kPFOff = kS * kStage;             // L2-prefetch landing area, 256 B per wave
constexpr int kLDS = kPFOff + 4 * 256;
constexpr int kNLA = kBM * 8 / kThreads, kNLB = kBN * 8 / kThreads;
constexpr int kNLD = kNLA + kNLB;               // 16-byte copies per thread per slice
constexpr int kNL = kNLD + 2;                   // + A-scale and B-scale dwords
constexpr int kNR = (kTM + kTN) * 2;            // 16-byte fragment reads per slice
static_assert(kLDS <= 160 * 1024, "LDS");
static_assert(kBM / 8 == 32 && kBN / kGroupM == 32, "prefetch partition: 32 rows per part");

template <int FA, int FB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void
gemm_fp8_block_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLDS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int swave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = swave >> 1, wn = swave & 1;
  const int r16 = lane & 15, g16 = lane >> 4;
  const int tiles_m = (int)((p.M + kBM - 1) / kBM), tiles_n = (int)((p.N + kBN - 1) / kBN);
  int tm, tn;
  tile_coords<kGroupM>(tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
  const int64_t kbytes = p.K;  // one byte per FP8 element; K % 128 == 0
  const int nkt = (int)(p.K / 128);

  // ---- copy descriptors (rows beyond M / N read as zeros)
  const int rowsA = (int)min((int64_t)kBM, p.M - m0);
  const int rowsB = (int)min((int64_t)kBN, p.N - n0);
  const uint32_t ldaB = (uint32_t)p.lda, ldbB = (uint32_t)p.ldb;
  const __amdgpu_buffer_rsrc_t rA =
      make_rsrc((const uint8_t*)p.A + m0 * p.lda, (int64_t)(rowsA - 1) * ldaB + kbytes);
  const __amdgpu_buffer_rsrc_t rB =
      make_rsrc((const uint8_t*)p.B + n0 * p.ldb, (int64_t)(rowsB - 1) * ldbB + kbytes);
  uint32_t voffA[kNLA], voffB[kNLB];
#pragma unroll
  for (int it = 0; it < kNLA; ++it) {
    const int q = it * kThreads + tid, row = q / 8;
    const uint32_t c = (uint32_t)(((q % 8) ^ swz<kRB>(row)) << 4);
    voffA[it] = row < rowsA ? (uint32_t)row * ldaB + c : kOOB;
  }
#pragma unroll
  for (int it = 0; it < kNLB; ++it) {
    const int q = it * kThreads + tid, row = q / 8;
    const uint32_t c = (uint32_t)(((q % 8) ^ swz<kRB>(row)) << 4);
    voffB[it] = row < rowsB ? (uint32_t)row * ldbB + c : kOOB;
  }
  // scales: sa row-major [M][nkt], sb row-major [ceil(N/128)][nkt]; the
  // workgroup's 128 columns are one B-scale block
  const __amdgpu_buffer_rsrc_t rSA = make_rsrc(p.sa + m0 * nkt, (int64_t)rowsA * nkt * 4);
  const uint32_t voffSA = tid < rowsA ? (uint32_t)tid * (uint32_t)nkt * 4 : kOOB;
  const __amdgpu_buffer_rsrc_t rSB = make_rsrc(p.sb + (int64_t)tn * nkt, (int64_t)nkt * 4);
  const uint32_t voffSB = lane == 0 ? 0u : kOOB;

  // Copy number idx (0 <= idx < kNL) of slice kt into stage st; inactive
  // (kt beyond the last slice) copies use an out-of-range offset.
  auto issue_one = [&](int kt, int st, int idx) __attribute__((always_inline)) {
    uint8_t* sA = smem + st * kStage;
    const bool active = kt < nkt;
    const uint32_t koff = active ? (uint32_t)kt * kRB : 0u;
    if (idx < kNLA) {
      buffer_load_lds16(rA, sA + (idx * kThreads + swave * 64) * 16, active ? voffA[idx] : kOOB,
                        koff);
    } else if (idx < kNLD) {
      const int it = idx - kNLA;
      buffer_load_lds16(rB, sA + kABytes + (it * kThreads + swave * 64) * 16,
                        active ? voffB[it] : kOOB, koff);
    } else if (idx == kNLD) {
      buffer_load_lds4(rSA, sA + kSAOff + swave * 256, active ? voffSA : kOOB,
                       active ? (uint32_t)kt * 4 : 0u);
    } else {
      buffer_load_lds4(rSB, sA + kSBOff + swave * 256, active ? voffSB : kOOB,
                       active ? (uint32_t)kt * 4 : 0u);
    }
  };

  // L2 prefetch of slice kt (see gemm.hip): the workgroups one XCD runs
  // together form a kGroupM x 8 block of tiles; wave 0 fetches 1/8 of the A
  // rows, wave 1 1/kGroupM of the B rows, one 4-byte copy per 64-byte half
  // line into a scratch LDS area.
  __amdgpu_buffer_rsrc_t rP = rA;
  uint32_t voffP = kOOB;
  const uint32_t cP = (uint32_t)(lane & 1) * 64;
  if (swave == 0) {
    const int row = (tn & 7) * (kBM / 8) + (lane >> 1);
    voffP = row < rowsA ? (uint32_t)row * ldaB + cP : kOOB;
  } else if (swave == 1) {
    rP = rB;
    const int row = (tm & (kGroupM - 1)) * (kBN / kGroupM) + (lane >> 1);
    voffP = row < rowsB ? (uint32_t)row * ldbB + cP : kOOB;
  }
  auto issue_pf = [&](int kt) __attribute__((always_inline)) {
    const bool active = kt < nkt;
    buffer_load_lds4(rP, smem + kPFOff + swave * 256, active ? voffP : kOOB,
                     active ? (uint32_t)kt * kRB : 0u);
  };

  auto lds16 = [&](const uint8_t* base, int row, int c) __attribute__((always_inline)) -> i32x4_t {
    return *(const i32x4_t*)(base + row * kRB + ((c ^ swz<kRB>(row)) << 4));
  };

  // Fragments: lane l holds row l%16 of a 16-row block and the 32-byte K
  // group l/16 (two 16-byte chunks), for A and B alike.
  i32x4_t fa[2][kTM][2], fb[2][kTN][2];
  // Read k (0 <= k < kNR) of a slice, in first-use order: A block 0, B blocks
  // 0 .. kTN-1, A blocks 1 .. kTM-1.
  auto read_one = [&](int st, int buf, int k) __attribute__((always_inline)) {
    const uint8_t* sA = smem + st * kStage;
    const int slot = k / 2, h = k % 2;
    if (slot == 0)
      fa[buf][0][h] = lds16(sA, wm * kWM + r16, 2 * g16 + h);
    else if (slot <= kTN)
      fb[buf][slot - 1][h] = lds16(sA + kABytes, wn * kWN + (slot - 1) * 16 + r16, 2 * g16 + h);
    else
      fa[buf][slot - kTN][h] = lds16(sA, wm * kWM + (slot - kTN) * 16 + r16, 2 * g16 + h);
  };

  // ---- prologue: slices 0 and 1 in flight, slices 2 .. kPD-1 prefetched
#pragma unroll
  for (int t = 0; t < kS - 1; ++t)
#pragma unroll
    for (int idx = 0; idx < kNL; ++idx) issue_one(t, t, idx);
#pragma unroll
  for (int t = kS - 1; t < kPD; ++t) issue_pf(t);
  // slice 0 landed: one slice of copies and the prefetches may be pending
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<kNL + (kPD - kS + 1)>());
  stage_barrier();
#pragma unroll
  for (int k = 0; k < kNR; ++k) {
    read_one(0, 0, k);
    __builtin_amdgcn_sched_barrier(0);
  }

  f32x4_t acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t part[4];
  float sc[kTM];        // this slice's sa(row) * sb for each 16-row block of the lane
  float sc_prev = 0.f;  // previous slice's scale of block kTM-1 (pending promotions)

  auto mfma_one = [&](int buf, int g) __attribute__((always_inline)) {
    const int i = g / kTN, j = g % kTN;
    part[g % 4] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
        cat(fb[buf][j][0], fb[buf][j][1]), cat(fa[buf][i][0], fa[buf][i][1]),
        f32x4_t{0.f, 0.f, 0.f, 0.f}, FB, FA, 0, 0, 0, 0);
  };
  auto promote = [&](int g, float s) __attribute__((always_inline)) {
    const int i = g / kTN, j = g % kTN;
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(part[g % 4][v], s, acc[i][j][v]);
  };

  // One slice.  buf holds its fragments; the next slice's go to buf ^ 1.
  auto slice = [&](int kt, int st, int buf, bool first) __attribute__((always_inline)) {
    const int ld_st = st == 0 ? kS - 1 : st - 1;  // stage of slice kt + 2
    const int nx_st = st == kS - 1 ? 0 : st + 1;  // stage of slice kt + 1
    {
      const float* sSA = (const float*)(smem + st * kStage + kSAOff);
      const float sbv = *(const float*)(smem + st * kStage + kSBOff + swave * 256);
#pragma unroll
      for (int i = 0; i < kTM; ++i) sc[i] = sSA[wm * kWM + i * 16 + r16] * sbv;
    }
#pragma unroll
    for (int g = 0; g < kNM; ++g) {
      if (g == kNM / 2) {
        // first half done: wait for slice kt+1 (only the copies of slice kt+2
        // and the newest prefetch may still be in flight), then hand over
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<kNL + 1>());
        stage_barrier();
      }
      __builtin_amdgcn_sched_barrier(0);
      mfma_one(buf, g);
      // promotion of MFMA g-2 (the two pending from the previous slice first)
      if (g >= 2)
        promote(g - 2, sc[(g - 2) / kTN]);
      else if (!first)
        promote(kNM - 2 + g, sc_prev);
      // copies of slice kt+2, then the prefetch of slice kt+3
      static_assert(kNL <= kNM / 2, "copies fit in the first half");
      if (g < kNL) issue_one(kt + kS - 1, ld_st, g);
      if (g == kNL - 1) issue_pf(kt + kPD);
      // next slice's fragments, after the barrier
      if (g >= kNM / 2) {
        const int gl = g - kNM / 2;
#pragma unroll
        for (int k = gl * kNR / (kNM / 2); k < (gl + 1) * kNR / (kNM / 2); ++k)
          read_one(nx_st, buf ^ 1, k);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    sc_prev = sc[kTM - 1];
  };

  int st = 0;
  int kt = 0;
  for (; kt + 1 < nkt; kt += 2) {
    slice(kt, st, 0, kt == 0);
    st = st == kS - 1 ? 0 : st + 1;
    slice(kt + 1, st, 1, false);
    st = st == kS - 1 ? 0 : st + 1;
  }
  if (kt < nkt) slice(kt, st, 0, kt == 0);
  __builtin_amdgcn_sched_barrier(0);
  promote(kNM - 2, sc_prev);
  promote(kNM - 1, sc_prev);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // every wave is done with the K-slice stages

  // ---- epilogue.  Lane l, register v of a transposed 16x16 accumulator is
  // D[row = l%16][col = 4*(l/16) + v].
  if (p.out_bf16 && !p.C) {
    // Round to BF16 and stage the wave's 128 x 64 quadrant (16 KB) in LDS,
    // 16-byte unit u of row r at u ^ (r % 8); read back 8 rows x 128 B per
    // instruction and store 16 bytes (8 columns) per lane.
    constexpr int RBY = kWN * 2;  // staged row bytes
    uint8_t* wbase = smem + swave * (kWM * RBY);
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        const f32x4_t x = acc[i][j];
        const uint32_t lo = f32_to_bf16_bits(x[0]) | ((uint32_t)f32_to_bf16_bits(x[1]) << 16);
        const uint32_t hi = f32_to_bf16_bits(x[2]) | ((uint32_t)f32_to_bf16_bits(x[3]) << 16);
        const int r = i * 16 + r16, u = 2 * j + (g16 >> 1);
        *(uint2*)(wbase + r * RBY + ((u ^ (r & 7)) << 4) + (g16 & 1) * 8) = make_uint2(lo, hi);
      }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<0>());  // own region only
    constexpr int UPR = RBY / 16, RPI = 64 / UPR;
#pragma unroll
    for (int it = 0; it < kWM / RPI; ++it) {
      const int r = it * RPI + lane / UPR, u = lane % UPR;
      const u32x4_t v = *(const u32x4_t*)(wbase + r * RBY + ((u ^ (r & 7)) << 4));
      const int64_t row = m0 + wm * kWM + r, col = n0 + wn * kWN + u * 8;
      if (row < p.M && col < p.N) {
        uint16_t* d = (uint16_t*)p.D + row * p.ldd + col;
        if (col + 7 < p.N) {
          *(u32x4_t*)d = v;
        } else {
          for (int e = 0; e < 8; ++e)
            if (col + e < p.N) d[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int64_t row = m0 + wm * kWM + i * 16 + r16;
#pragma unroll
      for (int j = 0; j < kTN; ++j) store4(p, row, n0 + wn * kWN + j * 16 + 4 * g16, acc[i][j]);
    }
  }
}

template <int FA, int FB>
hipError_t launch_fmt(const GemmArgs& a, hipStream_t s) {
  const int64_t tiles = ((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN);
  hipLaunchKernelGGL((gemm_fp8_block_kernel<FA, FB>), dim3((unsigned)tiles), dim3(kThreads), 0, s,
                     a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp8_block(const GemmArgs& a, int fmt_a, int fmt_b, hipStream_t s) {
  if (fmt_a == 0 && fmt_b == 0) return launch_fmt<0, 0>(a, s);
  if (fmt_a == 0 && fmt_b == 1) return launch_fmt<0, 1>(a, s);
  if (fmt_a == 1 && fmt_b == 0) return launch_fmt<1, 0>(a, s);
  return launch_fmt<1, 1>(a, s);
}

}  // namespace dmu
