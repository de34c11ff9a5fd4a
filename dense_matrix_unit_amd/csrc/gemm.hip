// Tiled MFMA GEMM for gfx950 (CDNA4): BF16, per-tensor-scaled FP8 and
// microscaled (MX) FP8 inputs, FP32 accumulation, FP32 or BF16 output.
// (Per-block FP32 scales of 1 x 128 / 128 x 128 blocks: gemm_block.hip.)
//
// What is computed: D = A*B + C with the products accumulated in FP32 -- the
// operation of a matrix instruction as the page "Tensor Cores: Matrix
// Instructions, Swizzling and FP8, Measured" (vidyal.ai) defines it in Step 1,
// applied to whole matrices as in its Step 2 (B may be stored N x K so both
// operands are K-contiguous).  For FP8 the two per-tensor scales are applied
// in the epilogue ("Tensor Cores" chapter of ai-infra-handbooks, "Precision"
// section, on per-tensor FP8 scaling factors).  MX: D = C + (A x SA)(B x SB)
// with one power-of-two (E8M0) scale per row and 32 values of K, the
// block-scaled product of "How Blackwell's Tensor Memory Actually Works",
// section "Quantization became an allocation problem"; gfx950's scaled MFMA
// applies the two scales itself, so they ride along with the K slices.
//
// Structure (three-level tiling: workgroup tile staged in LDS, wave tile held
// in accumulator registers, one MFMA per 32x32 sub-tile and K step):
//  * a 256-thread workgroup (4 waves, one per SIMD) owns a 256 x 256 tile of
//    D; each wave owns a 128 x 128 quadrant (4 x 4 sub-tiles, 256 AGPRs);
//  * K advances in 128-byte slices (64 BF16 or 128 FP8 values per row) held
//    in a 2-stage LDS ring: the copy of slice k+1 is issued while slice k is
//    multiplied, and an L2 prefetch brings slice k+3 close;
//  * A and B are copied global -> LDS by buffer loads that write LDS
//    directly (no VGPR round trip).  A row-major B slice stays row-major in
//    LDS (64 K rows of 512 bytes) and its fragments are read with gfx950's
//    transposing LDS read, which hands each lane 4 consecutive K values of
//    one column;
//  * LDS rows are 128 bytes of 16-byte chunks; chunk c of row r is stored at
//    position c ^ ((r ^ (r >> 3)) & 7).  A wave's 16-byte fragment reads
//    (consecutive rows, one chunk column) then touch every bank group once per
//    8 lanes.  The same XOR is applied when the slice is written, so no
//    padding is needed (the XOR-swizzle idea of the vidyal.ai page, Step 3,
//    re-derived for this row width and 16-byte reads);
//  * within a slice, the next step's fragment reads and the next slice's
//    copies are spread one or two per MFMA; half of the last step's MFMAs run
//    after the slice barrier, with the next slice's first reads between them;
//  * out-of-range rows and the K tail are fetched as zeros by giving their
//    buffer loads an out-of-range offset;
//  * workgroup ids are remapped so that the tiles one XCD runs together share
//    A row panels and B column panels in that XCD's L2;
//  * MX: a slice's scale codes are one 4-byte word (the 4 E8M0 codes of 128
//    K) per tile row of A and of B.  They sit in a two-buffer LDS ring beside
//    the stages, fetched for 4 slices at a time (16 bytes per row) when the
//    scale rows allow it.  After each slice barrier a lane reads the next
//    slice's words of its 4 A and 4 B rows; it supplies the scale of K block
//    lane / 32 of each 64-wide step, so it shifts each word right by
//    8 * (lane / 32), and step s selects byte 2 s with the instruction's
//    op_sel.
#include "gemm_common.h"

namespace dmu {
namespace {

// K slices between the L2 prefetch of a slice and its use (0 = no prefetch).
constexpr int kPrefetch = 3;
constexpr int kWavesBF16 = 4, kWavesFP8 = 4;  // waves per workgroup (4: one per SIMD)

template <int FA, int FB>
__device__ __forceinline__ f32x16_t mfma_fp8_32x32x64(const i32x8_t& a, const i32x8_t& b,
                                                      const f32x16_t& c) {
  // cbsz / blgp select the A / B formats: 0 = E4M3, 1 = E5M2.  Zero scale
  // operands select the unscaled instruction.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
}

// LDS layouts of a K slice: the XOR-swizzled rows every entry point uses, and
// two variants kept only for the layout ablation of the BF16 kernel
// (dmu_probe_gemm_bf16_layout): plain rows, and rows padded by 16 bytes.
enum LdsLayout { kSwizzled = 0, kPlain = 1, kPadded = 2 };

// A row-major B slice in LDS is K rows of 512 bytes (256 BF16 columns, 32
// chunks of 16 bytes); chunk c of K row r is stored at position c ^ bswz(r).
// One transposing fragment read covers 4 consecutive K rows and 64 bytes of
// each per 32 lanes; flipping bits 2-3 of the chunk index with r % 4 puts
// those 4 x 64 bytes in distinct banks.
__device__ __forceinline__ int bswz(int r) { return (r & 3) << 2; }

// gfx950 transposing LDS read (ds_read_b64_tr_b16): in each group of 16
// lanes, lane i names row i / 4 and 16-bit elements 4 (i % 4) .. +3 of a
// row-major 4 x 16 block; lane j receives element j of the 4 rows, in row
// order.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const uint8_t* p) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
  const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
  return __builtin_bit_cast(uint2, r);
}

template <int KIND, int FA, int FB, bool BROW, int BM, int BN, int RB, int S, int kGroupM, int PD,
          int NW, bool KT, int LAY = kSwizzled>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void
gemm_kernel(GemmArgs p) {
  constexpr int NT = NW * 64;   // threads; NW waves in a 2 x (NW/2) grid
  constexpr bool F4 = KIND == kMXF4;  // E2M1 operands: 32 bytes of a row per K step of 64
  constexpr bool GRP = KIND == kBF16G;                // grouped over experts
  constexpr bool EPI = KIND == kBF16F || KIND == kFP8TensorF;  // fused epilogue
  constexpr bool BF = KIND == kBF16 || GRP || KIND == kBF16F;  // BF16 operands
  constexpr bool F8T = KIND == kFP8Tensor || KIND == kFP8TensorF;  // per-tensor FP8
  constexpr int ESZ = BF ? 2 : 1;
  constexpr int CPR = RB / 16;  // 16-byte chunks of K per LDS row
  // LDS row stride and 16-byte positions per row: a padded row carries one
  // unused position after its chunks
  constexpr int RS = LAY == kPadded ? RB + 16 : RB;
  constexpr int CPRS = RS / 16;
  static_assert(LAY == kSwizzled || (KIND == kBF16 && !BROW && !KT),
                "the plain and padded layouts exist for the BF16 kernel's ablation only");
  constexpr int WM = BM / 2, WN = BN / (NW / 2);
  constexpr int TM = WM / 32, TN = WN / 32;      // 32x32 sub-tiles per wave
  constexpr int A_BYTES = BM * RS, B_BYTES = BN * RS;
  constexpr int STAGE = A_BYTES + B_BYTES;
  // MX: scale words are fetched XG slices at a time (4 * XG bytes per tile
  // row) into a two-buffer ring of their own after the stages
  constexpr bool MX = KIND == kMX || KIND == kMX4 || KIND == kMXF4;
  constexpr int XG = KIND == kMX4 ? 4 : F4 ? 2 : 1;
  constexpr int WPS = F4 ? 2 : 1;               // scale words per row and slice
  constexpr int XROW = 4 * WPS * XG;            // ring bytes per tile row
  constexpr int XBUF = (BM + BN) * XROW;        // one ring buffer (A rows, then B rows)
  constexpr int XOFF = S * STAGE;               // ring offset in LDS
  constexpr int XR = MX ? 2 * XBUF : 0;
  constexpr int NSTEP = BF || F4 ? RB / 32 : RB / 64;  // MFMA K-steps per slice
  constexpr int NLA = BM * CPRS / NT;                // A copies per thread per slice
  constexpr int NLB = BN * CPRS / NT;                // B copies per thread per slice
  constexpr int NLS = MX ? 2 : 0;                    // MX scale-group copies (A, B)
  constexpr int NL = NLA + NLB + NLS;
  static_assert(BM % 64 == 0 && BN % 64 == 0 && (BM * CPRS) % NT == 0, "tile");
  // row-major B in LDS: RB / 2 K rows of BROWB bytes (BN BF16 values)
  constexpr int BROWB = BN * 2;
  static_assert(!BROW || ((KIND == kBF16 || KIND == kBF16F) && BN == 256 && RB == 128 && S == 2 &&
                          NW == 4 && LAY == kSwizzled),
                "row-major B staging");
  static_assert(BF || F8T || MX,
                "per-block FP32 scales live in gemm_block.hip");
  static_assert(!MX || (!KT && !BROW && RB == 128 && NW == 4 && BM == 256 && BN == 256 && S == 2),
                "MX: whole 128-K slices, one scale row per thread and operand");
  static_assert(S >= 2 && NL * (S - 2) < 64, "vmcnt range");
  static_assert(PD == 0 || (S == 2 && BM == 256 && BN == 256 && kGroupM == 4 && PD >= 2),
                "L2 prefetch layout");
  // one landing area per wave for the L2 prefetch's 4-byte copies, and for
  // MX scale copies that have nothing to fetch (64 lanes x 4 * XG bytes)
  constexpr int PF_WAVE = MX ? 64 * XROW : 256;
  constexpr int PF_BYTES = PD > 0 || MX ? NW * PF_WAVE : 0;
  // Row-major B: every LDS buffer is an array of its own (A stages sa0, sa1,
  // B stages sb0, sb1, prefetch area spf).  The compiler cannot tell a
  // transposing read from the copies still writing LDS unless they touch
  // different arrays; in one array it would make every such read wait for all
  // outstanding copies.
  constexpr int SMEM = BROW ? 16 : S * STAGE + XR + PF_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];
  __shared__ __attribute__((aligned(1024))) uint8_t sa0[BROW ? A_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t sa1[BROW ? A_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t sb0[BROW ? B_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t sb1[BROW ? B_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t spf[BROW && PF_BYTES > 0 ? PF_BYTES : 16];
  // LDS stage st of A and of B (st is a constant at every call), and the
  // prefetch landing area
  auto stage_a = [&](int st) __attribute__((always_inline)) -> uint8_t* {
    if constexpr (BROW) return st == 0 ? sa0 : sa1;
    else return smem + st * STAGE;
  };
  auto stage_b = [&](int st) __attribute__((always_inline)) -> uint8_t* {
    if constexpr (BROW) return st == 0 ? sb0 : sb1;
    else return smem + st * STAGE + A_BYTES;
  };
  uint8_t* const pf_area = BROW ? spf : smem + S * STAGE + XR;

  const int tid = threadIdx.x, lane = tid & 63;
  const int swave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept scalar
  const int wm = swave / (NW / 2), wn = swave % (NW / 2);
  const int rl = lane & 31, hl = lane >> 5;
  // grouped: an upper bound of the experts' m-tile count, sum ceil(M_g / BM)
  const int tiles_m = GRP ? (int)((p.Mmax + BM - 1) / BM + p.G) : (int)((p.M + BM - 1) / BM);
  const int tiles_n = (int)((p.N + BN - 1) / BN);
  int tm, tn;
  tile_coords<kGroupM>(tiles_m, tiles_n, tm, tn);
  tm = __builtin_amdgcn_readfirstlane(tm);
  tn = __builtin_amdgcn_readfirstlane(tn);
  int64_t m0 = (int64_t)tm * BM;
  if constexpr (GRP) {
    // m-tile tm is tile t of expert g: walk the experts' tile counts (row
    // offsets written by routing on the device, read with scalar loads).
    // Offsets are clamped to [0, Mmax] and made non-decreasing, so no
    // workgroup touches rows outside A and D whatever they hold.
    int64_t lo = min(max(p.goff[0], (int64_t)0), p.Mmax);
    int t = tm, g = 0;
    for (; g < p.G; ++g) {
      const int64_t hi = min(max(p.goff[g + 1], lo), p.Mmax);
      const int nt = (int)((hi - lo + BM - 1) / BM);
      if (t < nt) {
        m0 = lo + (int64_t)t * BM;
        p.M = hi;  // the expert's last row bounds this tile's loads and stores
        break;
      }
      t -= nt;
      lo = hi;
    }
    if (g == p.G) return;  // past the last expert's tiles: the whole workgroup exits
    p.B = (const uint16_t*)p.B + g * p.gstride;
  }
  const int64_t n0 = (int64_t)tn * BN;
  const int64_t kbytes = F4 ? p.K / 2 : p.K * ESZ;
  const int nkt = (int)((kbytes + RB - 1) / RB);

  // ---- A: global -> LDS descriptors (rows beyond M read as zeros)
  const int rowsA = (int)min((int64_t)BM, p.M - m0);
  const uint32_t ldaB = (uint32_t)(p.lda * ESZ);
  const __amdgpu_buffer_rsrc_t rA =
      make_rsrc((const uint8_t*)p.A + m0 * p.lda * ESZ, (int64_t)(rowsA - 1) * ldaB + kbytes);
  // copy `it` of a thread fills LDS position q = it * NT + tid (16 bytes):
  // row q / CPRS, position q % CPRS, from the global chunk that belongs there
  // (the XOR applied on the source side; a padding position fetches zeros)
  auto src_chunk = [&](int row, int pos) __attribute__((always_inline)) -> int {
    return LAY == kSwizzled ? pos ^ swz<RB>(row) : pos;
  };
  uint32_t voffA[NLA], cA[NLA];
#pragma unroll
  for (int it = 0; it < NLA; ++it) {
    const int q = it * NT + tid, row = q / CPRS, pos = q % CPRS;
    const uint32_t c = (uint32_t)(src_chunk(row, pos) << 4);
    cA[it] = c;
    voffA[it] = row < rowsA && pos < CPR ? (uint32_t)row * ldaB + c : kOOB;
  }

  // ---- B descriptors
  const int rowsB = (int)min((int64_t)BN, p.N - n0);  // columns of D this tile covers
  const uint32_t ldbB = (uint32_t)(p.ldb * ESZ);
  __amdgpu_buffer_rsrc_t rB;
  // column-major B: as A.  Row-major B: copy `it` fills LDS position q = it *
  // NT + tid, K row q / 32, position q % 32 of that row's 32 16-byte chunks
  // (8 columns each), from chunk (q % 32) ^ bswz(row); cB holds the K row.
  uint32_t voffB[NLB], cB[NLB];
  if constexpr (BROW) {
    rB = make_rsrc((const uint8_t*)p.B + n0 * 2, (p.K * p.ldb - n0) * 2);
#pragma unroll
    for (int it = 0; it < NLB; ++it) {
      const int q = it * NT + tid, row = q / (BROWB / 16), pos = q % (BROWB / 16);
      const int c = pos ^ bswz(row);
      cB[it] = (uint32_t)row;
      voffB[it] = c * 8 < rowsB ? (uint32_t)row * ldbB + (uint32_t)(c << 4) : kOOB;
    }
  } else {
    rB = make_rsrc((const uint8_t*)p.B + n0 * p.ldb * ESZ, (int64_t)(rowsB - 1) * ldbB + kbytes);
#pragma unroll
    for (int it = 0; it < NLB; ++it) {
      const int q = it * NT + tid, row = q / CPRS, pos = q % CPRS;
      const uint32_t c = (uint32_t)(src_chunk(row, pos) << 4);
      cB[it] = c;
      voffB[it] = row < rowsB && pos < CPR ? (uint32_t)row * ldbB + c : kOOB;
    }
  }

  // A resource with no records: every load through it returns zeros.  When
  // K fills whole slices (!KT), a slice is either entirely in range or
  // entirely past the end, so the copies pick this resource with one scalar
  // select per slice instead of testing every lane's offset.
  const __amdgpu_buffer_rsrc_t rNull = make_rsrc(p.A, 0);

  // ---- MX scale words.  Group G holds slices XG*G .. XG*G+XG-1: the 4*XG
  // codes of each tile row, for A rows then B rows, in ring buffer G % 2.
  // Thread t copies row t of A and of B (4*XG bytes each; rows past the
  // matrix read zeros).  A row's codes for one slice are a single word, so
  // each copy instruction touches 64 rows, i.e. 64 cache lines: fetching XG
  // slices at once divides those line requests by XG.
  __amdgpu_buffer_rsrc_t rXA = rNull, rXB = rNull;
  uint32_t voffXA = kOOB, voffXB = kOOB;
  const int ngroups = nkt / XG;
  if constexpr (MX) {
    const int64_t kb = p.K / 32;  // scale bytes per row
    rXA = make_rsrc(p.xa + m0 * p.ldxa, (int64_t)(rowsA - 1) * p.ldxa + kb);
    rXB = make_rsrc(p.xb + n0 * p.ldxb, (int64_t)(rowsB - 1) * p.ldxb + kb);
    voffXA = tid < rowsA ? (uint32_t)(tid * p.ldxa) : kOOB;
    voffXB = tid < rowsB ? (uint32_t)(tid * p.ldxb) : kOOB;
  }
  // copy `which` (0: A, 1: B) of scale group G.  A copy with nothing to
  // fetch (no group G, or `on` false) still issues, through the null
  // resource into the wave's landing area: one instruction stream for every
  // slice, with no branch between the MFMAs.
  auto issue_xgroup = [&](int G, int which, bool on) __attribute__((always_inline)) {
    if constexpr (MX) {
      const bool act = on && G < ngroups;
      uint8_t* dst = act ? smem + XOFF + (G & 1) * XBUF + which * BM * XROW + swave * 64 * XROW
                         : pf_area + swave * PF_WAVE;
      const uint32_t koff = act ? (uint32_t)G * XROW : 0u;
      const __amdgpu_buffer_rsrc_t r = act ? (which == 0 ? rXA : rXB) : rNull;
      const uint32_t v = which == 0 ? voffXA : voffXB;
      static_assert(XROW == 16 || XROW == 4, "scale copy width");
      if constexpr (XROW == 16) buffer_load_lds16(r, dst, v, koff);
      else buffer_load_lds4(r, dst, v, koff);
    }
  };

  // ---- L2 prefetch of slice kt + PD.  With two LDS stages only one slice of
  // copies is in flight, so a copy that misses to HBM stalls the K loop.  A
  // 4-byte copy per 64-byte half line, into a scratch LDS area, brings the
  // slice into this XCD's L2 a few slices early; the real copy then hits.
  // The workgroups one XCD runs together form a kGroupM x 8 block of tiles
  // (tile_coords), so each A panel is shared by 8 of them and each B panel
  // by kGroupM: each workgroup fetches 1/8 of its A rows (wave 0) and
  // 1/kGroupM of its B rows (waves 1 and 2), so every line is fetched once.
  // Row-major B: a slice is RB / 2 K rows of BN columns, and each workgroup
  // fetches 1/kGroupM of those rows, 64 bytes per lane; prow is the K row
  // within the slice and pfs the byte distance between slices (RB for A).
  __amdgpu_buffer_rsrc_t rP = rA;
  uint32_t voffP = kOOB, cP = 0;
  uint32_t pfs = RB, prow = 0;
  if constexpr (PD > 0) {
    const int half = lane & 1;
    cP = (uint32_t)half * 64;
    if (swave == 0) {
      const int row = (tn & 7) * (BM / 8) + (lane >> 1);
      voffP = row < rowsA ? (uint32_t)row * ldaB + cP : kOOB;
    } else if (swave <= 2) {
      rP = rB;
      if constexpr (BROW) {
        constexpr int RPW = RB / 2 / kGroupM / 2;  // K rows per fetching wave
        constexpr int LPR = BROWB / 64;            // lanes per K row
        static_assert(RPW * LPR == 64, "one 64-byte fetch per lane");
        const int row = (tm & (kGroupM - 1)) * (2 * RPW) + (swave - 1) * RPW + lane / LPR;
        const int col = (lane % LPR) * 64;  // bytes
        prow = (uint32_t)row;
        pfs = (uint32_t)(RB / 2) * ldbB;
        voffP = col / 2 < rowsB ? (uint32_t)row * ldbB + (uint32_t)col : kOOB;
      } else {
        const int row = (tm & (kGroupM - 1)) * (BN / kGroupM) + (swave - 1) * 32 + (lane >> 1);
        voffP = row < rowsB ? (uint32_t)row * ldbB + cP : kOOB;
      }
    }
  }
  auto issue_pf = [&](int kt) __attribute__((always_inline)) {
    if constexpr (PD > 0) {
      const bool active = kt < nkt;
      if constexpr (BROW) {
        const uint32_t koff = active ? (uint32_t)kt * pfs : 0u;
        if constexpr (KT) {
          // past the end of K: the byte along A's row, or B's K row
          const bool in = swave == 0 ? koff + cP < (uint32_t)kbytes
                                     : (int64_t)kt * (RB / 2) + prow < p.K;
          buffer_load_lds4(rP, pf_area + swave * PF_WAVE, active && in ? voffP : kOOB, koff);
        } else {
          buffer_load_lds4(active ? rP : rNull, pf_area + swave * PF_WAVE, voffP, koff);
        }
      } else {
        const uint32_t koff = active ? (uint32_t)kt * RB : 0u;
        if constexpr (KT) {
          const uint32_t v = active && koff + cP < (uint32_t)kbytes ? voffP : kOOB;
          buffer_load_lds4(rP, pf_area + swave * PF_WAVE, v, koff);
        } else {
          buffer_load_lds4(active ? rP : rNull, pf_area + swave * PF_WAVE, voffP, koff);
        }
      }
    }
  };

  // Row-major B: copy `it` of slice kt into B stage sB.  The slice is RB / 2
  // K rows from row kt * RB / 2; rows past K read zeros.
  auto issue_brow = [&](uint8_t* sB, int kt, bool active, int it) __attribute__((always_inline)) {
    uint8_t* dst = sB + (it * NT + swave * 64) * 16;
    const uint32_t soff = active ? (uint32_t)kt * (uint32_t)(RB / 2) * ldbB : 0u;
    if constexpr (KT) {
      const bool in = active && (int64_t)kt * (RB / 2) + cB[it] < p.K;
      buffer_load_lds16(rB, dst, in ? voffB[it] : kOOB, soff);
    } else {
      buffer_load_lds16(active ? rB : rNull, dst, voffB[it], soff);
    }
  };

  // Copy K slice `kt` into LDS stage `st`.  With active == false every lane
  // gets an out-of-range offset (slices after the last one), so the
  // instruction stream is the same on every iteration.
  auto issue_loads = [&](int kt, int st, bool active) __attribute__((always_inline)) {
    uint8_t* sA = stage_a(st);
    uint8_t* sB = stage_b(st);
    // chunks at byte position >= klim along K are fetched as zeros: the K
    // tail of the last slice, or everything when inactive
    const uint32_t koff = active ? (uint32_t)kt * RB : 0u;
    const uint32_t klim = active ? (uint32_t)kbytes : 0u;
#pragma unroll
    for (int it = 0; it < NLA; ++it) {
      const uint32_t v = koff + cA[it] < klim ? voffA[it] : kOOB;
      buffer_load_lds16(rA, sA + (it * NT + swave * 64) * 16, v, koff);
    }
    if constexpr (BROW) {
#pragma unroll
      for (int it = 0; it < NLB; ++it) issue_brow(sB, kt, active, it);
    } else {
#pragma unroll
      for (int it = 0; it < NLB; ++it) {
        const uint32_t v = koff + cB[it] < klim ? voffB[it] : kOOB;
        buffer_load_lds16(rB, sB + (it * NT + swave * 64) * 16, v, koff);
      }
    }
  };

  // Copy number idx (0 <= idx < NLA + NLB) of slice kt into stage st; the
  // same copies issue_loads makes, one at a time, so they can be spread
  // between MFMAs.
  auto issue_one = [&](int kt, int st, bool active, int idx) __attribute__((always_inline)) {
    if (NLS > 0 && idx >= NLA + NLB) {
      // MX: kt is the slice being copied, one ahead of the slice being
      // multiplied (cur).  In the first slice of group G, the copy of group
      // G + 1: it lands by this slice's closing wait, and its buffer last
      // held group G - 1, whose reads all completed before the barrier that
      // closed the previous slice.
      const int cur = kt - (S - 1);
      issue_xgroup(cur / XG + 1, idx - NLA - NLB, cur % XG == 0);
      return;
    }
    uint8_t* sA = stage_a(st);
    uint8_t* sB = stage_b(st);
    const uint32_t koff = active ? (uint32_t)kt * RB : 0u;
    const uint32_t klim = active ? (uint32_t)kbytes : 0u;
    if (idx < NLA) {
      if constexpr (KT) {
        const uint32_t v = koff + cA[idx] < klim ? voffA[idx] : kOOB;
        buffer_load_lds16(rA, sA + (idx * NT + swave * 64) * 16, v, koff);
      } else {
        buffer_load_lds16(active ? rA : rNull, sA + (idx * NT + swave * 64) * 16, voffA[idx], koff);
      }
    } else if constexpr (BROW) {
      issue_brow(sB, kt, active, idx - NLA);
    } else {
      const int it = idx - NLA;
      if constexpr (KT) {
        const uint32_t v = koff + cB[it] < klim ? voffB[it] : kOOB;
        buffer_load_lds16(rB, sB + (it * NT + swave * 64) * 16, v, koff);
      } else {
        buffer_load_lds16(active ? rB : rNull, sB + (it * NT + swave * 64) * 16, voffB[it], koff);
      }
    }
  };

  // 16-byte LDS read of logical chunk c of tile row `row`.
  auto lds16 = [&](const uint8_t* base, int row, int c) __attribute__((always_inline)) -> i32x4_t {
    return *(const i32x4_t*)(base + row * RS + ((LAY == kSwizzled ? c ^ swz<RB>(row) : c) << 4));
  };

  // ---- prologue: slices 0 .. S-2 in flight, wait for slice 0
#pragma unroll
  for (int t = 0; t < S - 1; ++t) issue_loads(t, t, t < nkt);
#pragma unroll
  for (int w = 0; w < NLS; ++w) issue_xgroup(0, w, true);  // MX scale group 0
  // slices 1 .. PD-1 are prefetched here; the loop prefetches kt + PD
#pragma unroll
  for (int t = 1; t < PD; ++t) issue_pf(t);
  constexpr int NPF = PD > 0 ? 1 : 0;  // prefetches per slice per thread
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<NL * (S - 2) + (PD > 1 ? PD - 1 : 0)>());
  stage_barrier();

  {
    constexpr int CPL = BF || F4 ? 1 : 2;  // 16-byte chunks per lane per step
    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x16_t{};
    i32x4_t fa[2][TM][CPL], fb[2][TN][CPL];
    // 16-byte chunk (along K) that half h of this lane's step-s fragment
    // holds.  Unscaled products do not depend on which K positions a lane's
    // bytes stand for, so those read one contiguous run per lane.  The scaled
    // MFMA does: a lane's two halves are K positions 16 * (lane / 32) and
    // 32 + 16 * (lane / 32) of the 64-wide step, and lane group g's scale
    // covers K block g (32 values) of the step.
    auto chunk = [&](int s, int h) __attribute__((always_inline)) -> int {
      if constexpr (MX && !F4) return 4 * s + 2 * h + hl;
      else return (2 * s + hl) * CPL + h;
    };
    // MX: the next slice's scale words as read from the ring, and the
    // current slice's shifted to this lane's K block (WPS words per row)
    uint32_t xraw[TM + TN][WPS], xa[WPS][TM], xb[WPS][TN];
    auto read_scales = [&](int kt) __attribute__((always_inline)) {
      if constexpr (MX) {
        const uint8_t* x = smem + XOFF + ((kt / XG) & 1) * XBUF + 4 * WPS * (kt % XG);
#pragma unroll
        for (int r = 0; r < TM + TN; ++r) {
          const int row = r < TM ? wm * WM + r * 32 + rl : BM + wn * WN + (r - TM) * 32 + rl;
          if constexpr (WPS == 2) {
            const uint2 w = *(const uint2*)(x + row * XROW);
            xraw[r][0] = w.x;
            xraw[r][1] = w.y;
          } else {
            xraw[r][0] = *(const uint32_t*)(x + row * XROW);
          }
        }
      }
    };
    auto take_scales = [&]() __attribute__((always_inline)) {
      if constexpr (MX) {
        const uint32_t sh = 8u * (uint32_t)hl;
#pragma unroll
        for (int w = 0; w < WPS; ++w) {
#pragma unroll
          for (int i = 0; i < TM; ++i) xa[w][i] = xraw[i][w] >> sh;
#pragma unroll
          for (int j = 0; j < TN; ++j) xb[w][j] = xraw[TM + j][w] >> sh;
        }
      }
    };
    // Row-major B: the step-s fragment of sub-tile j (lane l: column l % 32,
    // K values 16 s + 8 (l / 32) + 0..7, as the A fragment's chunk) is two
    // transposing reads, K rows 16 s + 8 (l / 32) + 0..3 and + 4..7.  Lane i
    // of 16-lane group g names K row i / 4 of the four and columns
    // 16 (g % 2) + 4 (i % 4) .. +3 of the sub-tile; bswz of those rows is
    // (i / 4) << 2, so each sub-tile has one per-lane offset.
    uint32_t bro[BROW ? TN : 1];
    if constexpr (BROW) {
      const int i = lane & 15, g = (lane >> 4) & 1;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int c = (wn * WN + j * 32) / 8 + 2 * g + ((i & 3) >> 1);  // 16-byte chunk
        bro[j] = (uint32_t)((8 * hl + (i >> 2)) * BROWB + ((c ^ ((i >> 2) << 2)) << 4) +
                            ((i & 1) << 3));
      }
    }
    auto rd_b = [&](const uint8_t* sB, int j, int s, int h) __attribute__((always_inline)) -> i32x4_t {
      if constexpr (BROW) {
        const uint8_t* q = sB + bro[j] + 16 * s * BROWB;
        const uint2 lo = lds_read_tr16(q), hi = lds_read_tr16(q + 4 * BROWB);
        return i32x4_t{(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
      } else {
        return lds16(sB, wn * WN + j * 32 + rl, chunk(s, h));
      }
    };
    auto load_step = [&](int st, int s, int buf) __attribute__((always_inline)) {
      const uint8_t* sA = stage_a(st);
      const uint8_t* sB = stage_b(st);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int h = 0; h < CPL; ++h)
          fa[buf][i][h] = lds16(sA, wm * WM + i * 32 + rl, chunk(s, h));
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int h = 0; h < CPL; ++h) fb[buf][j][h] = rd_b(sB, j, s, h);
    };
    // Fragment read k (0 <= k < NR) of step s, in the order the step's MFMAs
    // first need them: A fragment 0, B fragments 0 .. TN-1, A fragments
    // 1 .. TM-1 (each CPL 16-byte chunks).  Spreading these reads between the
    // previous step's MFMAs keeps only a few LDS reads outstanding, so the
    // next step's first MFMAs never wait on a burst of reads.
    constexpr int NR = (TM + TN) * CPL;
    auto read_one = [&](int st, int s, int buf, int k) __attribute__((always_inline)) {
      const uint8_t* sA = stage_a(st);
      const uint8_t* sB = stage_b(st);
      const int c = chunk(s, k % CPL);
      const int slot = k / CPL, h = k % CPL;
      if (slot == 0)
        fa[buf][0][h] = lds16(sA, wm * WM + rl, c);
      else if (slot <= TN)
        fb[buf][slot - 1][h] = rd_b(sB, slot - 1, s, h);
      else
        fa[buf][slot - TN][h] = lds16(sA, wm * WM + (slot - TN) * 32 + rl, c);
    };
    // The B fragment is the instruction's first operand, so each accumulator
    // holds a transposed 32x32 sub-tile (see the epilogue).
    auto mfma_one = [&](int s, int i, int j) __attribute__((always_inline)) {
      const int buf = s & 1;
      if constexpr (BF)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, fb[buf][j][0]),
            __builtin_bit_cast(bf16x8_t, fa[buf][i][0]), acc[i][j], 0, 0, 0);
      else if constexpr (MX) {
        // step s covers K blocks 2 s and 2 s + 1 of the slice: scale word
        // s / 2, byte 2 (s % 2) (+ the lane group, already shifted in).  The
        // first operand is B's fragment, so its scale is the instruction's
        // first.  E2M1 fragments are 16 bytes, in the low half of the
        // operand registers.
        const int w = F4 ? s / 2 : 0;
        const i32x4_t z = {0, 0, 0, 0};
        const i32x8_t ob = F4 ? cat(fb[buf][j][0], z) : cat(fb[buf][j][0], fb[buf][j][CPL - 1]);
        const i32x8_t oa = F4 ? cat(fa[buf][i][0], z) : cat(fa[buf][i][0], fa[buf][i][CPL - 1]);
        constexpr int CF = F4 ? 4 : FB, CA = F4 ? 4 : FA;  // cbsz / blgp format codes
        if ((F4 ? s % 2 : s) == 0)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              ob, oa, acc[i][j], CF, CA, 0, (int)xb[w][j], 0, (int)xa[w][i]);
        else
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              ob, oa, acc[i][j], CF, CA, 2, (int)xb[w][j], 2, (int)xa[w][i]);
      } else
        acc[i][j] = mfma_fp8_32x32x64<FB, FA>(cat(fb[buf][j][0], fb[buf][j][1]),
                                              cat(fa[buf][i][0], fa[buf][i][1]), acc[i][j]);
    };
    // With two or more steps per slice, the fragment buffers alternate within
    // the slice and the last step ends on buffer 1, so the next slice's first
    // reads (buffer 0) can overlap the second half of the last step.  With
    // one step per slice all MFMAs are issued before the barrier and the
    // next slice's fragments are read after it.
    constexpr bool kSplitLast = NSTEP >= 2;
    // The next slice's copies are spread between this slice's MFMAs (one
    // every R MFMAs, all before the barrier): a burst of copies would stall
    // the wave at issue while the matrix pipe idles.
    // MX scale copies ride along with the first data copies, so the data
    // copies keep their slots and the last of them stays as far from the
    // slice's closing wait as without scales
    constexpr int NLD = NLA + NLB;  // data copies per slice
    constexpr int PRE = (NSTEP - 1) * TM * TN + (kSplitLast ? TM / 2 : TM) * TN;
    constexpr int R = PRE / NLD < 2 ? PRE / NLD : 2;
    static_assert(R >= 1, "every copy is issued before the slice barrier");
    // same order as in the loop, so the waits at the loop head stay exact
    read_scales(0);
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      read_one(0, 0, 0, k);
      __builtin_amdgcn_sched_barrier(0);
    }
    // One K slice in stage st.  The loop runs two slices per iteration so that
    // every stage index, hence every LDS address offset, is a constant.
    auto slice = [&](int kt, const int st) __attribute__((always_inline)) {
      const int ld_st = st == 0 ? S - 1 : st - 1;  // stage of slice kt+S-1
      const int nx_st = st == S - 1 ? 0 : st + 1;  // stage of slice kt+1
      const bool act = kt + S - 1 < nkt;
      take_scales();
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        const int buf = s & 1;
        const int iend = (s + 1 < NSTEP || !kSplitLast) ? TM : TM / 2;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if (i >= iend) continue;
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            mfma_one(s, i, j);
            const int gl = i * TN + j;  // MFMA index within the step
            const int g = s * TM * TN + gl;
            __builtin_amdgcn_sched_barrier(0);
            if (s + 1 < NSTEP) {
#pragma unroll
              for (int k = gl * NR / (TM * TN); k < (gl + 1) * NR / (TM * TN); ++k)
                read_one(st, s + 1, buf ^ 1, k);
            }
            if (g % R == R - 1 && g / R < NLD) {
              if (g / R < NLS) issue_one(kt + S - 1, ld_st, act, NLD + g / R);
              issue_one(kt + S - 1, ld_st, act, g / R);
              if (g / R == NLD - 1) issue_pf(kt + PD);  // after this slice's copies
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // slice kt+1 has landed; only the prefetch issued in this slice may
      // still be in flight (vector memory operations complete in order)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<NL * (S - 2) + NPF>());
      stage_barrier();
      __builtin_amdgcn_sched_barrier(0);
      read_scales(kt + 1);  // next slice's scale words; this slice's stay in xa / xb
      if constexpr (kSplitLast) {
        // next slice's first fragments, interleaved with the rest of this slice
        constexpr int NM = (TM - TM / 2) * TN;
#pragma unroll
        for (int i = TM / 2; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int gl = (i - TM / 2) * TN + j;
#pragma unroll
            for (int k = gl * NR / NM; k < (gl + 1) * NR / NM; ++k) read_one(nx_st, 0, 0, k);
            __builtin_amdgcn_sched_barrier(0);
            mfma_one(NSTEP - 1, i, j);
            __builtin_amdgcn_sched_barrier(0);
          }
      } else {
        load_step(nx_st, 0, 0);  // next slice's first reads (zeros after the last slice)
      }
    };
    static_assert(S == 2, "two slices per loop iteration");
    int kt = 0;
    for (; kt + 1 < nkt; kt += 2) {
      slice(kt, 0);
      slice(kt + 1, 1);
    }
    if (kt < nkt) slice(kt, 0);

    // ---- epilogue: scale, add C, round, store.  Lane l, register 4q+r of a
    // transposed 32x32 accumulator is D[row = l%32][col = 8q + 4*(l/32) + r].
    // Written straight to memory that is 16 B per lane spread over 32 rows;
    // instead each wave passes one 32-row band at a time through its own LDS
    // region, and reads it back so that every store covers whole row
    // segments (32 lanes x 16 B of FP32, or x 8 B of BF16, per row).  Rows
    // are padded by 16 bytes, which makes both the band writes (16 lanes at
    // the same column of 16 rows) and the row reads bank-conflict free.
    constexpr int ROWW = WN + 4;  // padded band row, in floats
    static_assert(NW * 32 * ROWW * 4 <= S * STAGE, "epilogue bands fit in LDS");
    static_assert(NW * TM * 32 * WN * 2 <= S * STAGE && (WN * 2) % 16 == 0 && 64 % (WN / 8) == 0,
                  "BF16 staging fits in LDS");
    static_assert(WN % 4 == 0 && 64 % (WN / 4) == 0, "band read shape");
    float alpha = 1.0f;
    if constexpr (F8T) alpha = p.sa[0] * p.sb[0];
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // every wave is done reading the K-slice stages
    // the wave's staging region of `bytes`; with row-major B the regions are
    // the two A stages and the two B stages, 32 KB each
    auto region = [&](int bytes) __attribute__((always_inline)) -> uint8_t* {
      if constexpr (BROW) {
        static_assert(NW == 4 && A_BYTES == 32768 && B_BYTES == 32768, "four 32 KB regions");
        return swave == 0 ? sa0 : swave == 1 ? sa1 : swave == 2 ? sb0 : sb1;
      } else {
        return smem + swave * bytes;
      }
    };
    if constexpr (EPI) {
      // Fused epilogue (the fused entry points take no C): scale, bias,
      // activation and conversion on the accumulators, one 32-row block row
      // of the wave at a time.  The block's converted bytes are staged in the
      // wave's own LDS region (16-byte unit u of staged row r at
      // u ^ (r % units-per-row), so neither the writes nor the reads collide
      // in the banks), read back a row segment per lane and stored 16 bytes
      // at a time.  Lane l, register 4q+r of sub-tile (i, j) is column
      // j*32 + 8q + 4*(l/32) + r of row i*32 + l%32.
      //
      // The lane's bias values are loaded once, before any is used, from
      // addresses clamped into the vector, so the loads carry no branch.
      f32x4_t bv[TN][4];
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) bv[j][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (p.bias) {
        const int64_t cb = n0 + wn * WN + 4 * hl;
        if (p.N % 4 == 0) {
          // a group of four columns is wholly inside or wholly outside
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int64_t c = cb + j * 32 + 8 * q;
              const f32x4_t v = *(const f32x4_t*)(p.bias + min(c, p.N - 4));
              bv[j][q] = c < p.N ? v : f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
        } else {
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int64_t c = cb + j * 32 + 8 * q + r;
                const float v = p.bias[min(c, p.N - 1)];
                bv[j][q][r] = c < p.N ? v : 0.0f;
              }
        }
      }
      // One copy of the loop per output type and activation (EB output
      // bytes, ACT, FMT the FP8 format): a test of the activation per element
      // would split the code into thousands of branches.  The block-row loop
      // stays rolled; a switch copies block row i out of the accumulators,
      // which are never indexed at run time.
      static_assert(TM == 4, "block-row switch");
      auto fused = [&](auto ob, auto ac, auto fc) __attribute__((always_inline)) {
        constexpr int EB = decltype(ob)::value;  // output bytes per element
        constexpr int ACT = decltype(ac)::value;
        constexpr int FMT = decltype(fc)::value;
        constexpr int RBS = WN * EB;             // staged row bytes
        constexpr int UPS = RBS / 16;            // 16-byte units per staged row
        constexpr int RPIS = 64 / UPS;           // staged rows per read instruction
        static_assert(NW * 32 * RBS <= S * STAGE && RBS % 16 == 0 && 64 % UPS == 0,
                      "block staging fits in LDS");
        const float m = EB == 1 ? 1.0f / p.out_scale[0] : 1.0f;
        static_assert(!BROW || 32 * RBS <= 32768, "staging region");
        uint8_t* wb = region(32 * RBS);
#pragma unroll 1
        for (int i = 0; i < TM; ++i) {
          f32x16_t cur[TN];
          switch (i) {
            case 0:
#pragma unroll
              for (int j = 0; j < TN; ++j) cur[j] = acc[0][j];
              break;
            case 1:
#pragma unroll
              for (int j = 0; j < TN; ++j) cur[j] = acc[1][j];
              break;
            case 2:
#pragma unroll
              for (int j = 0; j < TN; ++j) cur[j] = acc[2][j];
              break;
            default:
#pragma unroll
              for (int j = 0; j < TN; ++j) cur[j] = acc[3][j];
          }
          uint8_t* row = wb + rl * RBS;
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              f32x4_t x = {cur[j][4 * q], cur[j][4 * q + 1], cur[j][4 * q + 2], cur[j][4 * q + 3]};
              if constexpr (F8T) x *= alpha;
              x += bv[j][q];
              if constexpr (ACT != 0)
#pragma unroll
                for (int r = 0; r < 4; ++r) x[r] = activate(x[r], ACT);
              if constexpr (EB == 4) {
                const int u = j * 8 + 2 * q + hl;
                *(f32x4_t*)(row + ((u ^ (rl & (UPS - 1))) << 4)) = x;
              } else if constexpr (EB == 2) {
                const uint32_t lo =
                    pack2_bf16(x[0], x[1]);
                const uint32_t hi =
                    pack2_bf16(x[2], x[3]);
                const int u = j * 4 + q;
                *(uint2*)(row + ((u ^ (rl & (UPS - 1))) << 4) + hl * 8) = make_uint2(lo, hi);
              } else {
                const int u = j * 2 + q / 2;
                *(uint32_t*)(row + ((u ^ (rl & (UPS - 1))) << 4) + 8 * (q & 1) + 4 * hl) =
                    cvt4_fp8<FMT>(x * m);
              }
            }
          // own region only: no barrier, and no wait for earlier blocks'
          // stores; the next block's writes cannot pass these reads, as the
          // LDS work of one wave stays in order.  All reads go out before the
          // first store waits for its data.
          __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<63>());
          u32x4_t v[32 / RPIS];
#pragma unroll
          for (int it = 0; it < 32 / RPIS; ++it) {
            const int r = it * RPIS + lane / UPS, u = lane % UPS;
            v[it] = *(const u32x4_t*)(wb + r * RBS + ((u ^ (r & (UPS - 1))) << 4));
          }
#pragma unroll
          for (int it = 0; it < 32 / RPIS; ++it) {
            const int r = it * RPIS + lane / UPS, u = lane % UPS;
            const int64_t grow = m0 + wm * WM + i * 32 + r, col = n0 + wn * WN + u * (16 / EB);
            if (grow < p.M && col < p.N) {
              uint8_t* d = (uint8_t*)p.D + (grow * p.ldd + col) * EB;
              if (col + 16 / EB - 1 < p.N) {
                *(u32x4_t*)d = v[it];
              } else {
                for (int e = 0; e < 16; ++e)
                  if (col + e / EB < p.N) d[e] = (uint8_t)(v[it][e >> 2] >> (8 * (e & 3)));
              }
            }
          }
        }
      };
      auto by_act = [&](auto ob, auto fc) __attribute__((always_inline)) {
        if (p.act == 1) fused(ob, IntConst<1>{}, fc);
        else if (p.act == 2) fused(ob, IntConst<2>{}, fc);
        else if (p.act == 3) fused(ob, IntConst<3>{}, fc);
        else fused(ob, IntConst<0>{}, fc);
      };
      if (p.out_fp8 == 0) by_act(IntConst<1>{}, IntConst<0>{});
      else if (p.out_fp8 == 1) by_act(IntConst<1>{}, IntConst<1>{});
      else if (p.out_bf16) by_act(IntConst<2>{}, IntConst<0>{});
      else by_act(IntConst<4>{}, IntConst<0>{});
    } else if (p.out_bf16 && !p.C) {
      // BF16 output: round first, then stage all four bands of the wave at
      // once (4 x 32 rows x 256 B = 32 KB per wave), so the LDS traffic is
      // halved and no band waits for the previous one.  16-byte unit u of
      // staged row r sits at u ^ (r % 16): the 8-byte writes of 16 rows at
      // one column then fall in distinct bank groups.  Each read instruction
      // covers 4 rows x 256 B and each store writes 16 B (8 columns) per lane.
      static_assert(!BROW || TM * 32 * WN * 2 <= 32768, "staging region");
      uint8_t* wbase = region(TM * 32 * WN * 2);
      constexpr int RB16 = WN * 2;    // staged row bytes
      constexpr int UPR = RB16 / 16;  // 16-byte units per row
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4_t x = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                         acc[i][j][4 * q + 3]};
            if constexpr (F8T) x *= alpha;
            const uint32_t lo = pack2_bf16(x[0], x[1]);
            const uint32_t hi = pack2_bf16(x[2], x[3]);
            const int u = j * 4 + q;  // 16-byte unit of the staged row
            *(uint2*)(wbase + (i * 32 + rl) * RB16 + ((u ^ (rl & (UPR - 1))) << 4) + hl * 8) =
                make_uint2(lo, hi);
          }
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<0>());  // own region only: no barrier
      constexpr int RPI16 = 64 / UPR;  // rows per read instruction
#pragma unroll
      for (int it = 0; it < TM * 32 / RPI16; ++it) {
        const int r = it * RPI16 + lane / UPR, u = lane % UPR;
        const u32x4_t v = *(const u32x4_t*)(wbase + r * RB16 + ((u ^ (r & (UPR - 1))) << 4));
        const int64_t row = m0 + wm * WM + r, col = n0 + wn * WN + u * 8;
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
      static_assert(!BROW || 32 * ROWW * 4 <= 32768, "staging region");
      float* band = (float*)region(32 * ROWW * 4);
      constexpr int LPR = WN / 4;       // lanes per band row on the read side
      constexpr int RPI = 64 / LPR;     // band rows per read instruction
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4_t x = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                         acc[i][j][4 * q + 3]};
            if constexpr (F8T) x *= alpha;
            *(f32x4_t*)(band + rl * ROWW + j * 32 + 8 * q + 4 * hl) = x;
          }
#pragma unroll
        for (int it = 0; it < 32 / RPI; ++it) {
          const int br = it * RPI + lane / LPR, bc = (lane % LPR) * 4;
          const f32x4_t x = *(const f32x4_t*)(band + br * ROWW + bc);
          store4(p, m0 + wm * WM + i * 32 + br, n0 + wn * WN + bc, x);
        }
      }
    }
  }
}

template <int KIND, int FA, int FB, bool BROW, int BM, int BN, int RB, int S, int G, int PD = 0,
          int NW = 4>
hipError_t launch(const GemmArgs& a, hipStream_t s) {
  const int64_t tiles_m = KIND == kBF16G ? (a.Mmax + BM - 1) / BM + a.G : (a.M + BM - 1) / BM;
  const int64_t tiles = tiles_m * ((a.N + BN - 1) / BN);
  // K tail: the last slice is partial and its lanes are range-checked one by
  // one (MX requires whole slices and has no such variant)
  if constexpr (KIND != kMX && KIND != kMX4 && KIND != kMXF4) {
    if ((a.K * (KIND == kBF16 || KIND == kBF16G || KIND == kBF16F ? 2 : 1)) % RB != 0) {
      hipLaunchKernelGGL((gemm_kernel<KIND, FA, FB, BROW, BM, BN, RB, S, G, PD, NW, true>),
                         dim3((unsigned)tiles), dim3(NW * 64), 0, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_kernel<KIND, FA, FB, BROW, BM, BN, RB, S, G, PD, NW, false>),
                     dim3((unsigned)tiles), dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16_fused(const GemmArgs& a, int b_col_major, hipStream_t s) {
  if (b_col_major) return launch<kBF16F, 0, 0, false, 256, 256, 128, 2, 4, kPrefetch, kWavesBF16>(a, s);
  return launch<kBF16F, 0, 0, true, 256, 256, 128, 2, 4, kPrefetch, kWavesBF16>(a, s);
}

hipError_t launch_gemm_fp8_fused(const GemmArgs& a, int fmt_a, int fmt_b, hipStream_t s) {
#define DMU_F8F(FA, FB) launch<kFP8TensorF, FA, FB, false, 256, 256, 128, 2, 4, kPrefetch, kWavesFP8>(a, s)
  if (fmt_a == 0 && fmt_b == 0) return DMU_F8F(0, 0);
  if (fmt_a == 0 && fmt_b == 1) return DMU_F8F(0, 1);
  if (fmt_a == 1 && fmt_b == 0) return DMU_F8F(1, 0);
  return DMU_F8F(1, 1);
#undef DMU_F8F
}

hipError_t launch_gemm_grouped_bf16(const GemmArgs& a, hipStream_t s) {
  return launch<kBF16G, 0, 0, false, 256, 256, 128, 2, 4, kPrefetch, kWavesBF16>(a, s);
}

hipError_t launch_gemm_bf16_layout(const GemmArgs& a, int layout, hipStream_t s) {
  // the headline kernel (B stored N x K, whole K slices) with each LDS layout
  const dim3 grid((unsigned)(((a.M + 255) / 256) * ((a.N + 255) / 256)));
  if (layout == kPlain)
    hipLaunchKernelGGL((gemm_kernel<kBF16, 0, 0, false, 256, 256, 128, 2, 4, kPrefetch, kWavesBF16,
                                    false, kPlain>),
                       grid, dim3(kWavesBF16 * 64), 0, s, a);
  else if (layout == kPadded)
    hipLaunchKernelGGL((gemm_kernel<kBF16, 0, 0, false, 256, 256, 128, 2, 4, kPrefetch, kWavesBF16,
                                    false, kPadded>),
                       grid, dim3(kWavesBF16 * 64), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_kernel<kBF16, 0, 0, false, 256, 256, 128, 2, 4, kPrefetch, kWavesBF16,
                                    false, kSwizzled>),
                       grid, dim3(kWavesBF16 * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const GemmArgs& a, int b_col_major, hipStream_t s) {
  if (b_col_major && skinny_applies(a)) return launch_gemm_bf16_skinny(a, s);
  if (b_col_major) return launch<kBF16, 0, 0, false, 256, 256, 128, 2, 4, kPrefetch, kWavesBF16>(a, s);
  return launch<kBF16, 0, 0, true, 256, 256, 128, 2, 4, kPrefetch, kWavesBF16>(a, s);
}

template <int FA, int FB>
static hipError_t launch_fp8_fmt(const GemmArgs& a, int block_scaled, hipStream_t s) {
  if (block_scaled) return launch_gemm_fp8_block(a, FA, FB, s);
  return launch<kFP8Tensor, FA, FB, false, 256, 256, 128, 2, 4, kPrefetch, kWavesFP8>(a, s);
}

hipError_t launch_gemm_fp8(const GemmArgs& a, int fmt_a, int fmt_b, int block_scaled,
                           hipStream_t s) {
  if (fmt_a == 0 && fmt_b == 0) return launch_fp8_fmt<0, 0>(a, block_scaled, s);
  if (fmt_a == 0 && fmt_b == 1) return launch_fp8_fmt<0, 1>(a, block_scaled, s);
  if (fmt_a == 1 && fmt_b == 0) return launch_fp8_fmt<1, 0>(a, block_scaled, s);
  return launch_fp8_fmt<1, 1>(a, block_scaled, s);
}

template <int KIND>
static hipError_t launch_mx_kind(const GemmArgs& a, int fmt_a, int fmt_b, hipStream_t s) {
#define DMU_MX(FA, FB) launch<KIND, FA, FB, false, 256, 256, 128, 2, 4, kPrefetch, kWavesFP8>(a, s)
  if (fmt_a == 0 && fmt_b == 0) return DMU_MX(0, 0);
  if (fmt_a == 0 && fmt_b == 1) return DMU_MX(0, 1);
  if (fmt_a == 1 && fmt_b == 0) return DMU_MX(1, 0);
  return DMU_MX(1, 1);
#undef DMU_MX
}

hipError_t launch_gemm_mxfp4(const GemmArgs& a, hipStream_t s) {
  return launch<kMXF4, 4, 4, false, 256, 256, 128, 2, 4, kPrefetch, kWavesFP8>(a, s);
}

hipError_t launch_gemm_mxfp8(const GemmArgs& a, int fmt_a, int fmt_b, hipStream_t s) {
  // scale groups of 4 slices (16 bytes per row) when they are whole and
  // 16-byte aligned, else one slice (4 bytes) at a time
  const bool g4 = a.K % 512 == 0 && a.ldxa % 16 == 0 && a.ldxb % 16 == 0 &&
                  (uintptr_t)a.xa % 16 == 0 && (uintptr_t)a.xb % 16 == 0;
  if (g4) return launch_mx_kind<kMX4>(a, fmt_a, fmt_b, s);
  return launch_mx_kind<kMX>(a, fmt_a, fmt_b, s);
}

}  // namespace dmu
