// Tiled MFMA GEMM for gfx950 (CDNA4): BF16 and scaled FP8 inputs, FP32
// accumulation, FP32 or BF16 output.
//
// What is computed: D = A*B + C with the products accumulated in FP32 -- the
// operation of a matrix instruction as the page "Tensor Cores: Matrix
// Instructions, Swizzling and FP8, Measured" (vidyal.ai) defines it in Step 1,
// applied to whole matrices as in its Step 2 (B may be stored N x K so both
// operands are K-contiguous).  For FP8 the per-tensor scales are removed in
// the epilogue, and with per-block scales each 128-wide partial sum is formed
// from zero and promoted into the FP32 accumulator with its two scales (Step 5
// of the same page, promotion of partial results into FP32 registers; the
// "Tensor Cores" chapter of ai-infra-handbooks, "Precision" section, on
// per-tensor/per-row/per-block FP8 scaling factors).
//
// Structure (three-level tiling: workgroup tile staged in LDS, wave tile held
// in accumulator registers, one MFMA per 32x32 sub-tile):
//  * a 256-thread workgroup (4 waves, one per SIMD) owns a BM x BN tile of D;
//    each wave owns a (BM/2) x (BN/2) quarter as 32x32 MFMA sub-tiles;
//  * K advances in slices of 128 bytes per row (64 BF16 or 128 FP8 values);
//    two LDS stages: while the MFMAs consume one slice, the next slice is being
//    copied into the other stage;
//  * A and column-major B are copied global -> LDS by buffer loads that write
//    LDS directly (no VGPR round trip); a row-major B slice goes through VGPRs
//    and is transposed 8x8 in registers so that LDS always holds K-contiguous
//    rows;
//  * LDS rows are 128 bytes = eight 16-byte chunks; chunk c of row r is stored
//    at position c ^ ((r ^ (r >> 3)) & 7).  A wave's 16-byte fragment reads
//    (32 consecutive rows, one chunk column) then hit every bank once per 8 or
//    16 lanes.  The same XOR is applied when the slice is written, so no
//    padding is needed (the XOR-swizzle idea of the vidyal.ai page, Step 3,
//    re-derived for 128-byte rows and 16-byte reads);
//  * out-of-range rows and the K tail are fetched as zeros by giving their
//    buffer loads an out-of-range offset;
//  * workgroup ids are remapped so that the tiles one XCD runs together share
//    A row panels and B column panels in that XCD's L2.
#include "dmu_device.h"
#include "dmu_internal.h"

namespace dmu {
namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;  // bytes of K per tile row per stage

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

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

template <int FA, int FB>
__device__ __forceinline__ f32x16_t mfma_fp8_32x32x64(const i32x8_t& a, const i32x8_t& b,
                                                      const f32x16_t& c) {
  // cbsz / blgp select the A / B formats: 0 = E4M3, 1 = E5M2.  Zero scale
  // operands select the unscaled instruction.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
}

// D[row][col .. col+3] = x (+ C), masked to the matrix.
__device__ __forceinline__ void store4(const GemmArgs& p, int64_t row, int64_t col, f32x4_t x) {
  if (row >= p.M || col >= p.N) return;
  const bool full = col + 3 < p.N;
  if (p.C) {
    const float* c = p.C + row * p.ldc + col;
    if (full && ((p.ldc & 3) == 0)) {
      x += *(const f32x4_t*)c;
    } else {
      for (int r = 0; r < 4; ++r)
        if (col + r < p.N) x[r] += c[r];
    }
  }
  if (p.out_bf16) {
    uint16_t* d = (uint16_t*)p.D + row * p.ldd + col;
    const uint32_t lo = f32_to_bf16_bits(x[0]) | ((uint32_t)f32_to_bf16_bits(x[1]) << 16);
    const uint32_t hi = f32_to_bf16_bits(x[2]) | ((uint32_t)f32_to_bf16_bits(x[3]) << 16);
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

template <int KIND, int FA, int FB, bool BROW, int BM, int BN, int kGroupM>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs p) {
  constexpr int ESZ = KIND == kBF16 ? 2 : 1;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_BYTES = BM * kRowBytes, B_BYTES = BN * kRowBytes;
  constexpr int SA_BYTES = KIND == kFP8Block ? BM * 4 : 0;
  constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES;
  constexpr int NSTEP = KIND == kBF16 ? 4 : 2;  // MFMA K-steps per slice
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile");
  static_assert(!BROW || (KIND == kBF16 && BN == 256), "row-major B staging layout");
  static_assert(KIND != kFP8Block || BM == kThreads, "block-scale staging layout");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_m = (int)((p.M + BM - 1) / BM), tiles_n = (int)((p.N + BN - 1) / BN);
  int tm, tn;
  tile_coords<kGroupM>(tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t kbytes = p.K * ESZ;
  const int nkt = (int)((kbytes + kRowBytes - 1) / kRowBytes);
  const bool tail = (kbytes % kRowBytes) != 0;

  // ---- A: global -> LDS descriptors (rows beyond M read as zeros)
  const int rowsA = (int)min((int64_t)BM, p.M - m0);
  const uint32_t ldaB = (uint32_t)(p.lda * ESZ);
  const __amdgpu_buffer_rsrc_t rA =
      make_rsrc((const uint8_t*)p.A + m0 * p.lda * ESZ, (int64_t)(rowsA - 1) * ldaB + kbytes);
  uint32_t voffA[BM / 32];
  uint32_t cA[BM / 32];
#pragma unroll
  for (int it = 0; it < BM / 32; ++it) {
    const int q = it * kThreads + tid, row = q >> 3;
    const uint32_t c = (uint32_t)(((q & 7) ^ swz(row)) << 4);
    cA[it] = c;
    voffA[it] = row < rowsA ? (uint32_t)row * ldaB + c : kOOB;
  }

  // ---- B descriptors
  const int rowsB = (int)min((int64_t)BN, p.N - n0);
  const uint32_t ldbB = (uint32_t)(p.ldb * ESZ);
  __amdgpu_buffer_rsrc_t rB;
  constexpr int NB_IT = BROW ? 1 : BN / 32;
  uint32_t voffB[NB_IT];
  uint32_t cB[NB_IT];
  // row-major B: thread owns an 8 (k) x 8 (n) block of the slice
  const int kb8 = tid >> 5, nb8 = tid & 31;
  bool colok = true;
  if constexpr (BROW) {
    rB = make_rsrc((const uint8_t*)p.B + n0 * 2, (p.K * p.ldb - n0) * 2);
    colok = (int64_t)nb8 * 8 < rowsB;
    voffB[0] = ((uint32_t)(kb8 * 8) * (uint32_t)p.ldb + (uint32_t)nb8 * 8) * 2;
    cB[0] = 0;
  } else {
    rB = make_rsrc((const uint8_t*)p.B + n0 * p.ldb * ESZ, (int64_t)(rowsB - 1) * ldbB + kbytes);
#pragma unroll
    for (int it = 0; it < NB_IT; ++it) {
      const int q = it * kThreads + tid, row = q >> 3;
      const uint32_t c = (uint32_t)(((q & 7) ^ swz(row)) << 4);
      cB[it] = c;
      voffB[it] = row < rowsB ? (uint32_t)row * ldbB + c : kOOB;
    }
  }

  // ---- per-block scales of A (one float per row per K slice)
  const int nkb = (int)(p.K / 128);
  __amdgpu_buffer_rsrc_t rSA;
  uint32_t voffSA = kOOB;
  if constexpr (KIND == kFP8Block) {
    rSA = make_rsrc(p.sa + m0 * nkb, (int64_t)rowsA * nkb * 4);
    voffSA = tid < rowsA ? (uint32_t)tid * (uint32_t)nkb * 4 : kOOB;
  }

  u32x4_t breg[8];  // row-major B staging registers

  auto issue_loads = [&](int kt, int stage) __attribute__((always_inline)) {
    uint8_t* sA = smem + stage * STAGE;
    uint8_t* sB = sA + A_BYTES;
    const uint32_t koff = (uint32_t)kt * kRowBytes;
    const bool partial = tail && kt == nkt - 1;
#pragma unroll
    for (int it = 0; it < BM / 32; ++it) {
      uint32_t v = voffA[it];
      if (partial && koff + cA[it] >= (uint32_t)kbytes) v = kOOB;
      buffer_load_lds16(rA, sA + (it * kThreads + wave * 64) * 16, v, koff);
    }
    if constexpr (BROW) {
      const int k0 = kt * 64 + kb8 * 8;
      const bool ok = colok && k0 < p.K;
      const uint32_t soff = (uint32_t)kt * 64u * (uint32_t)p.ldb * 2u;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        breg[i] = buffer_load16(rB, ok ? voffB[0] + (uint32_t)(i * p.ldb * 2) : kOOB, soff);
    } else {
#pragma unroll
      for (int it = 0; it < NB_IT; ++it) {
        uint32_t v = voffB[it];
        if (partial && koff + cB[it] >= (uint32_t)kbytes) v = kOOB;
        buffer_load_lds16(rB, sB + (it * kThreads + wave * 64) * 16, v, koff);
      }
    }
    if constexpr (KIND == kFP8Block) {
      uint8_t* sSA = sB + B_BYTES;
      buffer_load_lds4(rSA, sSA + wave * 256, voffSA, (uint32_t)kt * 4);
    }
  };

  // row-major B: transpose the thread's 8x8 block in registers and store the
  // eight 16-byte K-chunks (one per n) into the swizzled K-contiguous layout.
  auto store_brow = [&](int stage) __attribute__((always_inline)) {
    if constexpr (BROW) {
      uint8_t* sB = smem + stage * STAGE + A_BYTES;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u32x4_t w;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = breg[2 * q][j >> 1], hi = breg[2 * q + 1][j >> 1];
          w[q] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
        }
        const int n = nb8 * 8 + j;
        *(u32x4_t*)(sB + n * kRowBytes + ((kb8 ^ swz(n)) << 4)) = w;
      }
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16_t{};

  const int rl = lane & 31, hl = lane >> 5;

  issue_loads(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  store_brow(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nkt) issue_loads(kt + 1, cur ^ 1);
    const uint8_t* sA = smem + cur * STAGE;
    const uint8_t* sB = sA + A_BYTES;

    if constexpr (KIND == kBF16) {
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        bf16x8_t a[TM], b[TN];
        const int c = 2 * s + hl;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int row = wm * WM + i * 32 + rl;
          a[i] = *(const bf16x8_t*)(sA + row * kRowBytes + ((c ^ swz(row)) << 4));
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int row = wn * WN + j * 32 + rl;
          b[j] = *(const bf16x8_t*)(sB + row * kRowBytes + ((c ^ swz(row)) << 4));
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
      }
    } else {
      // FP8: 32 bytes (two chunks) of K per lane per step
      auto frag = [&](const uint8_t* base, int row, int s) __attribute__((always_inline)) -> i32x8_t {
        const int c = 4 * s + 2 * hl;
        const i32x4_t lo = *(const i32x4_t*)(base + row * kRowBytes + ((c ^ swz(row)) << 4));
        const i32x4_t hi =
            *(const i32x4_t*)(base + row * kRowBytes + (((c + 1) ^ swz(row)) << 4));
        return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      };
      if constexpr (KIND == kFP8Tensor) {
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) {
          i32x8_t a[TM], b[TN];
#pragma unroll
          for (int i = 0; i < TM; ++i) a[i] = frag(sA, wm * WM + i * 32 + rl, s);
#pragma unroll
          for (int j = 0; j < TN; ++j) b[j] = frag(sB, wn * WN + j * 32 + rl, s);
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = mfma_fp8_32x32x64<FB, FA>(b[j], a[i], acc[i][j]);
        }
      } else {
        // per-block scales: partial = sum over this 128-wide K block, from zero
        const float* sSA = (const float*)(sB + B_BYTES);
        // a wave whose columns all lie beyond N has no scale row to read
        const int64_t ncol0 = n0 + wn * WN;
        const int nblk = __builtin_amdgcn_readfirstlane((int)(ncol0 >> 7));
        const float sbv = ncol0 < p.N ? p.sb[(int64_t)nblk * nkb + kt] : 0.0f;
        i32x8_t a0[TM], a1[TM], b0[TN], b1[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          a0[i] = frag(sA, wm * WM + i * 32 + rl, 0);
          a1[i] = frag(sA, wm * WM + i * 32 + rl, 1);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          b0[j] = frag(sB, wn * WN + j * 32 + rl, 0);
          b1[j] = frag(sB, wn * WN + j * 32 + rl, 1);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          // lane holds row (i*32 + lane%32) of the sub-tile: one A scale per lane
          const float sc = sSA[wm * WM + i * 32 + rl] * sbv;
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            f32x16_t part = mfma_fp8_32x32x64<FB, FA>(b0[j], a0[i], f32x16_t{});
            part = mfma_fp8_32x32x64<FB, FA>(b1[j], a1[i], part);
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = __builtin_fmaf(part[v], sc, acc[i][j][v]);
          }
        }
      }
    }

    if (kt + 1 < nkt) {
      __builtin_amdgcn_s_waitcnt(0);
      store_brow(cur ^ 1);
    }
    __syncthreads();
  }

  // ---- epilogue: scale, add C, round, store.  MFMAs were issued with the
  // B fragment as the instruction's first operand, so the accumulator holds
  // the transposed sub-tile: lane l, register 4q+r is D[row = l%32]
  // [col = 8q + 4*(l/32) + r] -- four consecutive columns of one row.
  float alpha = 1.0f;
  if constexpr (KIND == kFP8Tensor) alpha = p.sa[0] * p.sb[0];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t row = m0 + wm * WM + i * 32 + rl;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = n0 + wn * WN + j * 32 + 8 * q + 4 * hl;
        f32x4_t x = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                     acc[i][j][4 * q + 3]};
        if constexpr (KIND == kFP8Tensor) x *= alpha;
        store4(p, row, col, x);
      }
    }
  }
}

template <int KIND, int FA, int FB, bool BROW, int BM, int BN, int G>
hipError_t launch(const GemmArgs& a, hipStream_t s) {
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_kernel<KIND, FA, FB, BROW, BM, BN, G>), dim3((unsigned)tiles),
                     dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& a, int b_col_major, hipStream_t s) {
  if (b_col_major) return launch<kBF16, 0, 0, false, 256, 256, 4>(a, s);
  return launch<kBF16, 0, 0, true, 256, 256, 4>(a, s);
}

template <int FA, int FB>
static hipError_t launch_fp8_fmt(const GemmArgs& a, int block_scaled, hipStream_t s) {
  if (block_scaled) return launch<kFP8Block, FA, FB, false, 256, 256, 4>(a, s);
  return launch<kFP8Tensor, FA, FB, false, 256, 256, 4>(a, s);
}

hipError_t launch_gemm_fp8(const GemmArgs& a, int fmt_a, int fmt_b, int block_scaled,
                           hipStream_t s) {
  if (fmt_a == 0 && fmt_b == 0) return launch_fp8_fmt<0, 0>(a, block_scaled, s);
  if (fmt_a == 0 && fmt_b == 1) return launch_fp8_fmt<0, 1>(a, block_scaled, s);
  if (fmt_a == 1 && fmt_b == 0) return launch_fp8_fmt<1, 0>(a, block_scaled, s);
  return launch_fp8_fmt<1, 1>(a, block_scaled, s);
}

}  // namespace dmu
