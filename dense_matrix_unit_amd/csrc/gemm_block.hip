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
// accumulator lives in ordinary VGPRs, 128 of them per wave: a 64 x 128 wave
// tile of 4 x 8 sub-tiles.
//
// The promotion FMAs, the fragment reads and the copies together are more
// instructions per MFMA than one wave can issue in the MFMA's 32 cycles, so
// each SIMD runs two waves: a workgroup of 8 waves (4 x 2) computes a 256 x 256
// tile (BN = 256; 256 x 128 with 64 x 64 wave tiles when the problem has too
// few 256 x 256 tiles to fill the chip).  Register budget per wave: 128
// accumulator, 16 partial-product, 32 A-fragment and 32 B-fragment VGPRs.
//  * K slices of 128 bytes (one scale block) in two LDS stages, copied with
//    buffer loads that write LDS directly, XOR-swizzled; the slice's 256
//    A-row scales and BN/128 B scales ride along.
//  * MFMA g = j * 4 + i (column block j outer).  The four A fragments stay in
//    registers for the slice; B fragments stream two columns ahead through
//    four register slots.  The one barrier per slice sits where every wave has
//    read the last of this slice and before the first read of the next; the
//    next slice's A fragments replace this slice's right after their last MFMA.
//  * The copies of slice k+2 start right after the barrier of slice k (which
//    frees its stage) and are spread over 16 MFMA slots, into slice k+1, so
//    that the CU's one texture unit is not flooded; an L2 prefetch touches
//    slice k+4.
//  * MFMA g writes partial buffer g % 4 and the promotion of MFMA g-3 follows
//    it, so the FMAs never wait on a result still being computed.
//  * The second wave on each SIMD (waves 4..7) runs at raised issue priority:
//    by default the older wave wins every tie and the younger one falls a
//    third of a slice behind, to run alone while the older waits at the
//    barrier.
#include "gemm_common.h"

namespace dmu {
namespace {

constexpr int kNT = 512, kBM = 256, kRB = 128, kGroupM = 4;
constexpr int kFD = 2;    // B-fragment read distance, in column blocks
constexpr int kPD = 4;    // L2 prefetch distance, in K slices
constexpr int kNS2 = 16;  // MFMA slots the copies of one slice are spread over
constexpr int kLag = 3;   // MFMAs between a partial product and its promotion

// 16-byte chunk position of logical chunk c in 128-byte LDS row r: c ^ swz8(r).
// Any 16 consecutive rows starting at a multiple of 16 use every (row parity,
// position) pair once, so the 16-lane fragment reads are conflict-free under
// either bank organisation (32 banks x 8 lanes or 64 banks x 16 lanes per
// pass), and the pattern does not depend on the row block.
__device__ __forceinline__ int swz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int BN>
struct Cfg {
  static constexpr int WM = 64, WN = BN / 2;  // 4 x 2 waves
  static constexpr int TM = WM / 16, TN = WN / 16;
  static constexpr int NM = TM * TN;          // MFMAs per slice per wave
  static constexpr int ABytes = kBM * kRB, BBytes = BN * kRB;
  static constexpr int AOff = 0;              // A stages 0, 1
  static constexpr int BOff = 2 * ABytes;     // B stages 0, 1
  static constexpr int SAOff = BOff + 2 * BBytes;  // A-row scales, 1 KB per stage (waves 0..3)
  static constexpr int SBOff = SAOff + 2 * 1024;   // B scales, 1 KB per stage (waves 4..7)
  static constexpr int PFOff = SBOff + 2 * 1024;   // L2-prefetch landing, 256 B per wave
  static constexpr int LDS = PFOff + 8 * 256;
  static constexpr int NLA = kBM * 8 / kNT, NLB = BN * 8 / kNT;
  static constexpr int NLD = NLA + NLB, NL = NLD + 1;  // + one scale copy per wave
  static constexpr int NS1 = kFD * TM;                 // copy slots after the barrier
  static constexpr int NP1 = NS1 * NL / kNS2;          // copies issued in them
  static_assert(TN % 4 == 0 && TN > kFD, "B fragment slots");
  static_assert(kNS2 >= NS1 && kNS2 - NS1 <= (TN - kFD) * TM, "copy slots end before the barrier");
  static_assert(NM > kLag && kLag < 4, "partial buffers");
  static_assert(LDS <= 160 * 1024 && 8 * WM * WN * 2 <= SAOff, "LDS");
  static_assert(kBM / 8 == 32 && BN / kGroupM <= 64, "prefetch partition");
};

template <int FA, int FB, int BN>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(2, 2))) void
gemm_fp8_block_kernel(GemmArgs p) {
  using C = Cfg<BN>;
  constexpr int TM = C::TM, TN = C::TN, NM = C::NM;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int swave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = swave >> 1, wn = swave & 1;
  const int r16 = lane & 15, g16 = lane >> 4;
  const int tiles_m = (int)((p.M + kBM - 1) / kBM), tiles_n = (int)((p.N + BN - 1) / BN);
  int tm, tn;
  tile_coords<kGroupM>(tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * BN;
  const int nkt = (int)(p.K / 128);  // K % 128 == 0

  // ---- copy descriptors (rows beyond M / N read as zeros)
  const int rowsA = (int)min((int64_t)kBM, p.M - m0);
  const int rowsB = (int)min((int64_t)BN, p.N - n0);
  const uint32_t ldaB = (uint32_t)p.lda, ldbB = (uint32_t)p.ldb;
  const __amdgpu_buffer_rsrc_t rA =
      make_rsrc((const uint8_t*)p.A + m0 * p.lda, (int64_t)(rowsA - 1) * ldaB + p.K);
  const __amdgpu_buffer_rsrc_t rB =
      make_rsrc((const uint8_t*)p.B + n0 * p.ldb, (int64_t)(rowsB - 1) * ldbB + p.K);
  uint32_t voffA[C::NLA], voffB[C::NLB];
#pragma unroll
  for (int it = 0; it < C::NLA; ++it) {
    const int q = it * kNT + tid, row = q / 8;
    const uint32_t c = (uint32_t)(((q % 8) ^ swz8(row)) << 4);
    voffA[it] = row < rowsA ? (uint32_t)row * ldaB + c : kOOB;
  }
#pragma unroll
  for (int it = 0; it < C::NLB; ++it) {
    const int q = it * kNT + tid, row = q / 8;
    const uint32_t c = (uint32_t)(((q % 8) ^ swz8(row)) << 4);
    voffB[it] = row < rowsB ? (uint32_t)row * ldbB + c : kOOB;
  }
  // scales: sa row-major [M][nkt], sb row-major [ceil(N/128)][nkt].  Waves
  // 0..3 copy the slice's 256 A-row scales, wave 4 the tile's BN/128 B
  // scales; waves 5..7 issue an out-of-range copy, so that every wave counts
  // the same loads.
  const int nbs = (int)min((int64_t)(BN / 128), (p.N + 127) / 128 - n0 / 128);
  __amdgpu_buffer_rsrc_t rS;
  uint32_t voffS;
  if (swave < 4) {
    rS = make_rsrc(p.sa + m0 * nkt, (int64_t)rowsA * nkt * 4);
    const int row = swave * 64 + lane;
    voffS = row < rowsA ? (uint32_t)row * (uint32_t)nkt * 4 : kOOB;
  } else {
    rS = make_rsrc(p.sb + (n0 / 128) * nkt, (int64_t)nbs * nkt * 4);
    voffS = swave == 4 && lane < nbs ? (uint32_t)lane * (uint32_t)nkt * 4 : kOOB;
  }
  const int soffS = swave < 4 ? C::SAOff + swave * 256 : C::SBOff + (swave - 4) * 256;

  // Copy idx (0 <= idx < NL) of slice kt into stage st.  Slices past the end
  // reload the last one into a stage nobody reads any more.
  auto issue_one = [&](int kt, int st, int idx) __attribute__((always_inline)) {
    const uint32_t koff = (uint32_t)min(kt, nkt - 1) * kRB;
    if (idx < C::NLA) {
      buffer_load_lds16(rA, smem + C::AOff + st * C::ABytes + (idx * kNT + swave * 64) * 16,
                        voffA[idx], koff);
    } else if (idx < C::NLD) {
      const int it = idx - C::NLA;
      buffer_load_lds16(rB, smem + C::BOff + st * C::BBytes + (it * kNT + swave * 64) * 16,
                        voffB[it], koff);
    } else {
      buffer_load_lds4(rS, smem + soffS + st * 1024, voffS, (uint32_t)min(kt, nkt - 1) * 4);
    }
  };

  // L2 prefetch of slice kt (see gemm.hip): the kGroupM x 8 block of tiles one
  // XCD runs together shares each A panel among 8 workgroups and each B panel
  // among kGroupM.  Wave 5 touches this workgroup's 1/8 of the A rows, waves 6
  // and 7 its 1/kGroupM of the B rows, one 4-byte copy per 64-byte half line;
  // the other waves' copies are out of range.
  __amdgpu_buffer_rsrc_t rP = rA;
  uint32_t voffP = kOOB;
  {
    const uint32_t cP = (uint32_t)(lane & 1) * 64;
    if (swave == 5) {
      const int row = (tn & 7) * (kBM / 8) + (lane >> 1);
      voffP = row < rowsA ? (uint32_t)row * ldaB + cP : kOOB;
    } else if (swave >= 6) {
      rP = rB;
      const int part = (swave - 6) * 32, row = (tm & (kGroupM - 1)) * (BN / kGroupM) + part + (lane >> 1);
      voffP = part < BN / kGroupM && row < rowsB ? (uint32_t)row * ldbB + cP : kOOB;
    }
  }
  auto issue_pf = [&](int kt) __attribute__((always_inline)) {
    buffer_load_lds4(rP, smem + C::PFOff + swave * 256, voffP, (uint32_t)min(kt, nkt - 1) * kRB);
  };

  // Fragments: lane l holds row l%16 of a 16-row block and the 32-byte K
  // group l/16 (two 16-byte chunks), for A and B alike.  Byte addresses: the
  // row block and the stage go into the instruction's offset.
  uint32_t aoff[2], boff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int ra = wm * C::WM + r16, rb = wn * C::WN + r16;
    aoff[h] = (uint32_t)(C::AOff + ra * kRB + (((2 * g16 + h) ^ swz8(ra)) << 4));
    boff[h] = (uint32_t)(C::BOff + rb * kRB + (((2 * g16 + h) ^ swz8(rb)) << 4));
  }
  i32x4_t fa[TM][2], fb[4][2];
  auto read_fa = [&](int st, int i) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      fa[i][h] = *(const i32x4_t*)(smem + aoff[h] + st * C::ABytes + i * 16 * kRB);
  };
  auto read_fb = [&](int st, int j) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      fb[j & 3][h] = *(const i32x4_t*)(smem + boff[h] + st * C::BBytes + j * 16 * kRB);
  };
  float sc[2][TM];  // by slice parity: sa(this lane's row of block i) * sb
  auto read_scales = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      sc[st][i] = *(const float*)(smem + C::SAOff + st * 1024 + (wm * C::WM + i * 16 + r16) * 4);
  };
  auto mul_scales = [&](int st) __attribute__((always_inline)) {
    const float sbv = *(const float*)(smem + C::SBOff + st * 1024 + (wn * C::WN / 128) * 4);
#pragma unroll
    for (int i = 0; i < TM; ++i) sc[st][i] *= sbv;
  };

  // ---- prologue: slice 0 and the first part of slice 1 in flight, slices
  // 2 .. kPD-1 prefetched; wait for slice 0
#pragma unroll
  for (int idx = 0; idx < C::NL; ++idx) issue_one(0, 0, idx);
#pragma unroll
  for (int idx = 0; idx < C::NP1; ++idx) issue_one(1, 1, idx);
#pragma unroll
  for (int t = 2; t < kPD; ++t) issue_pf(t);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<C::NP1 + kPD - 2>());
  stage_barrier();
#pragma unroll
  for (int i = 0; i < TM; ++i) read_fa(0, i);
#pragma unroll
  for (int j = 0; j < kFD; ++j) read_fb(0, j);
  read_scales(0);
  mul_scales(0);

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // partial products in flight: MFMA g writes part[g % 4]; the kLag left at
  // the end of a slice are promoted at the start of the next (before the
  // first slice: zeros times zero scales)
  f32x4_t part[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) part[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < TM; ++i) sc[1][i] = 0.f;
  if (swave >= 4) __builtin_amdgcn_s_setprio(1);

  auto mfma_one = [&](int g) __attribute__((always_inline)) {
    const int i = g % TM, j = g / TM;
    part[g & 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
        cat(fb[j & 3][0], fb[j & 3][1]), cat(fa[i][0], fa[i][1]), f32x4_t{0.f, 0.f, 0.f, 0.f}, FB,
        FA, 0, 0, 0, 0);
  };
  auto promote = [&](int g, float s) __attribute__((always_inline)) {
    const int i = g % TM, j = g / TM;
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(part[g & 3][v], s, acc[i][j][v]);
  };

  // One K slice kt in stage st = kt % 2.
  auto slice = [&](int kt, auto stc) __attribute__((always_inline)) {
    constexpr int st = decltype(stc)::value, nst = st ^ 1;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if (j == TN - kFD) {
        __builtin_amdgcn_sched_barrier(0);
        // slice kt+1 landed (only the newest prefetch may be in flight) and
        // this wave's reads of slice kt are done; then every wave's
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<1>());
        stage_barrier();
      }
      __builtin_amdgcn_sched_barrier(0);
      if (j + kFD < TN) read_fb(st, j + kFD);
      else read_fb(nst, j + kFD - TN);  // next slice, after the barrier
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int g = j * TM + i;
        __builtin_amdgcn_sched_barrier(0);
        mfma_one(g);
        if (g >= kLag) promote(g - kLag, sc[st][(g - kLag) % TM]);
        else promote(NM - kLag + g, sc[nst][(NM - kLag + g) % TM]);
        if (j == TN - 1) read_fa(nst, i);  // after this slice's last use
        if (j == TN - 1 && i == 0) read_scales(nst);
        if (j == TN - 1 && i == TM - 1) mul_scales(nst);
        // copies of slice kt+2 into this slice's stage, after the barrier
        const int k = g - (TN - kFD) * TM;
        if (k >= 0)
#pragma unroll
          for (int idx = k * C::NL / kNS2; idx < (k + 1) * C::NL / kNS2; ++idx)
            issue_one(kt + 2, st, idx);
        // the rest of slice kt+1's copies, then the prefetch (the newest load
        // at the next barrier)
        const int k2 = C::NS1 + g;
        if (k2 < kNS2)
#pragma unroll
          for (int idx = k2 * C::NL / kNS2; idx < (k2 + 1) * C::NL / kNS2; ++idx)
            issue_one(kt + 1, nst, idx);
        if (g == kNS2 - C::NS1 - 1) issue_pf(kt + kPD);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  int kt = 0;
  for (; kt + 1 < nkt; kt += 2) {
    slice(kt, IntConst<0>{});
    slice(kt + 1, IntConst<1>{});
  }
  if (kt < nkt) slice(kt, IntConst<0>{});
  __builtin_amdgcn_sched_barrier(0);
  if ((nkt - 1) & 1) {
#pragma unroll
    for (int g = NM - kLag; g < NM; ++g) promote(g, sc[1][g % TM]);
  } else {
#pragma unroll
    for (int g = NM - kLag; g < NM; ++g) promote(g, sc[0][g % TM]);
  }
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // every wave is done with the K-slice stages

  // ---- epilogue.  Lane l, register v of a transposed 16x16 accumulator is
  // D[row = l%16][col = 4*(l/16) + v].
  if (p.out_bf16 && !p.C) {
    // Round to BF16 and stage the wave's quadrant in LDS, 16-byte unit u of
    // row r at u ^ (r % units per row); read back whole row segments and
    // store 16 bytes (8 columns) per lane.
    constexpr int RBY = C::WN * 2, UPR = RBY / 16, RPI = 64 / UPR;
    uint8_t* wbase = smem + swave * (C::WM * RBY);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const f32x4_t x = acc[i][j];
        const uint32_t lo = pack2_bf16(x[0], x[1]);
        const uint32_t hi = pack2_bf16(x[2], x[3]);
        const int r = i * 16 + r16, u = 2 * j + (g16 >> 1);
        *(uint2*)(wbase + r * RBY + ((u ^ (r & (UPR - 1))) << 4) + (g16 & 1) * 8) =
            make_uint2(lo, hi);
      }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<0>());  // own region only
#pragma unroll
    for (int it = 0; it < C::WM / RPI; ++it) {
      const int r = it * RPI + lane / UPR, u = lane % UPR;
      const u32x4_t v = *(const u32x4_t*)(wbase + r * RBY + ((u ^ (r & (UPR - 1))) << 4));
      const int64_t row = m0 + wm * C::WM + r, col = n0 + wn * C::WN + u * 8;
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
    for (int i = 0; i < TM; ++i) {
      const int64_t row = m0 + wm * C::WM + i * 16 + r16;
#pragma unroll
      for (int j = 0; j < TN; ++j) store4(p, row, n0 + wn * C::WN + j * 16 + 4 * g16, acc[i][j]);
    }
  }
}

template <int FA, int FB>
hipError_t launch_fmt(const GemmArgs& a, hipStream_t s) {
  // 256 x 128 tiles when 256 x 256 ones would leave more than half of the 256
  // compute units idle
  const int64_t big = ((a.M + kBM - 1) / kBM) * ((a.N + 255) / 256);
  if (big < 128) {
    const int64_t tiles = ((a.M + kBM - 1) / kBM) * ((a.N + 127) / 128);
    hipLaunchKernelGGL((gemm_fp8_block_kernel<FA, FB, 128>), dim3((unsigned)tiles), dim3(kNT), 0,
                       s, a);
  } else {
    hipLaunchKernelGGL((gemm_fp8_block_kernel<FA, FB, 256>), dim3((unsigned)big), dim3(kNT), 0, s,
                       a);
  }
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
