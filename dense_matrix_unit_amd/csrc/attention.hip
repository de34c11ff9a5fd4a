// Attention chain for gfx950: O = softmax(scale * Q K^T) V per head, BF16
// inputs, FP32 accumulation, BF16 output.  Two products are chained through
// a row-wise softmax without the scores ever leaving the chip: the chain the
// "Tensor Cores" chapter (ai-infra-handbooks), section "mma.sync: the register
// layout is explicit", names as FlashAttention's, where one product's output
// is worked on in registers and fed to the next.  The softmax is taken online
// over blocks of 64 keys: a reference maximum m and a running sum l per row,
// the partial output rescaled by exp(m_old - m_new) when m moves, which it
// does only when a block's maximum exceeds it by more than 2^8 in weight.
//
// Layout on the chip, per workgroup of 4 waves and 128 query rows:
//  * each wave owns 32 query rows; its Q rows sit in registers for the whole
//    kernel (B operand of the first product);
//  * both products use the swapped form (K or V^T first), so a lane always
//    holds one query row: lane l has row l % 32 and, of each 32-wide tile, the
//    columns 8q + 4(l/32) + r (register 4q + r).  The scores of a 16-key step
//    are then exactly the B operand the second product needs, so P goes from
//    the score registers straight into the next MFMA, rounded to BF16;
//  * a block of 64 keys is staged in LDS by direct copies: K rows in two
//    128-byte halves when d = 128, V rows whole, the 16-byte chunks of both
//    XOR-swizzled by row so that the fragment reads meet no bank conflict;
//  * the second product needs V transposed (keys along the lane's operand):
//    gfx950's transposing LDS read, ds_read_b64_tr_b16, gives each lane four
//    keys of its column from four rows, so V is never transposed in
//    registers; two such reads, of keys 4h..4h+3 and 8+4h..8+4h+3 of a 16-key
//    step, match the order of the weights in the score registers;
//  * each stage of K and of V is an LDS array of its own: the compiler then
//    sees that a stage's reads and the copies into the other stage touch
//    different arrays, and waits only for the reads (in one array it would
//    make every transposing read wait for all copies in flight);
//  * two stages of K and V (64 KB for d = 128), so two workgroups share a
//    CU and one wave's softmax arithmetic can run beside another's MFMAs;
//    alternate runs of 256 workgroup ids run at a higher wave priority, which
//    keeps the two on a CU from running in step;
//  * the copies of block t+2 go out right after the barrier that ends block
//    t, one barrier per block;
//  * with the causal mask a workgroup takes two query blocks, the i-th from
//    the end and the i-th from the start of its head, one after the other:
//    their key counts add up to the same for every pair, so all workgroups
//    carry the same work.
#include <utility>

#include "dmu_device.h"
#include "dmu_internal.h"
#include "gemm_common.h"

namespace dmu {
namespace {

constexpr int kBM = 128;  // query rows per workgroup (32 per wave)
constexpr int kBN = 64;   // keys per block
constexpr int kThreads = 256;
constexpr float kMinusBig = -1.0e30f;  // running maximum before the first key

// Physical 16-byte chunk of logical chunk c of a 128-byte LDS row r: c ^ aswz(r).
__device__ __forceinline__ int aswz(int r) { return (r ^ (r >> 3)) & 7; }

// Swizzle of the 16-byte chunks of V row j (d * 2 bytes): a transposing read
// covers 4 consecutive rows and 64 bytes of each per 32 lanes; flipping bits
// 2-3 of the chunk index with the row puts those 4 x 64 bytes in distinct
// banks.
template <int D>
__device__ __forceinline__ int vswz(int j) {
  return D == 128 ? (j & 3) << 2 : ((j >> 1) & 1) << 2;
}

// gfx950 transposing LDS read (ds_read_b64_tr_b16): in each group of 16
// lanes, lane i names row i / 4 and 16-bit elements 4 (i % 4) .. +3 of a
// row-major 4 x 16 block; lane j receives element j of the 4 rows, in row
// order.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 read_tr16(const uint8_t* q) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
  const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)q);
  return __builtin_bit_cast(uint2, r);
}

// Compile-time loop: f(Idx<0>{}), ..., f(Idx<N-1>{}), so that an index can
// feed a template argument (an instruction's immediate offset).
template <int V>
struct Idx {
  static constexpr int value = V;
};
template <typename F, int... I>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(Idx<I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll_n(F&& f) {
  unroll_seq(f, std::make_integer_sequence<int, N>{});
}

// The reference maximum of a row moves only when a block's maximum exceeds
// it by more than this (in exp2 units): weights then stay below 2^8, and the
// output is rescaled rarely instead of after nearly every block.
constexpr float kRescaleSlack = 8.0f;

// The two halves of a query row (lanes l and l ^ 32) side by side, with
// gfx950's v_permlane32_swap_b32 (lanes 32-63 of the first register trade
// places with lanes 0-31 of the second): on two copies of x it leaves the
// first holding lanes 0-31 of x twice and the second lanes 32-63 twice.  It
// is issued as inline assembly: the compiler's builtin, given the same value
// twice, folds its two results into one.  The s_nop gives the two wait
// states a VALU write needs before v_permlane32_swap reads the register.
__device__ __forceinline__ void halves(float x, float& lo, float& hi) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  lo = __builtin_bit_cast(float, a);
  hi = __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float half_max(float x) {
  float lo, hi;
  halves(x, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float half_sum(float x) {
  float lo, hi;
  halves(x, lo, hi);
  return lo + hi;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void
attention_kernel(AttnArgs p) {
  static_assert(D == 64 || D == 128, "head dimension");
  constexpr int NSTEP = D / 16;              // 16-wide d steps of the first product
  constexpr int NT = D / 32;                 // 32-column tiles of the output
  constexpr int KROW = 128;                  // bytes of a K half-row
  constexpr int VROW = D * 2;                // bytes of a V row
  constexpr int K_BYTES = kBN * D * 2;       // one K stage: D/64 halves of 64 x 128 B
  constexpr int V_BYTES = kBN * VROW;        // one V stage: 64 rows
  constexpr int KCOPY = K_BYTES / 16 / kThreads;  // 16-byte copies per thread per block, K
  constexpr int VCOPY = V_BYTES / 16 / kThreads;  // and V
  constexpr int CPR = D / 8;                 // 16-byte chunks of a V row
  constexpr int OB = 32 * D * 2;             // one wave's staged output rows
  static_assert(4 * OB <= 2 * K_BYTES + 2 * V_BYTES, "output staging fits");
  __shared__ __attribute__((aligned(1024))) uint8_t sK0[K_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sK1[K_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sV0[V_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sV1[V_BYTES];
  static_assert(2 * OB == K_BYTES, "two waves' output rows per K stage");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rl = lane & 31, hl = lane >> 5;
  // Two workgroups share a CU, so each SIMD runs one wave of each; when they
  // run in step, both want the matrix unit, then both the VALU.  Workgroups
  // in alternate runs of 256 ids (one per CU on this chip, the two that share
  // a CU in the first dispatch round) run at different wave priority, which
  // keeps them out of step: 2-4% faster across the measured shapes.
  if (((blockIdx.x >> 8) & 1) != 0) __builtin_amdgcn_s_setprio(2);

  // Workgroup -> (head, work item).  Dispatch goes round robin over the 8
  // XCDs; give each XCD a contiguous run of ids, so the query blocks of one
  // head (which read the same K and V) share an L2.  A work item is one query
  // block; with the causal mask it is a pair, blocks nqb-1-pb and pb, whose
  // key counts add up to the same for every pair, so every workgroup has the
  // same work (an odd middle block runs alone).
  const int nqb = (int)((p.Sq + kBM - 1) / kBM);
  const int npq = CAUSAL ? (nqb + 1) / 2 : nqb;  // work items per head
  int logical;
  {
    const int b = blockIdx.x, T = gridDim.x;
    const int x = b & 7, per = T >> 3, rem = T & 7;
    logical = __builtin_amdgcn_readfirstlane(x * per + (x < rem ? x : rem) + (b >> 3));
  }
  const int64_t bh = logical / npq;
  const int pb = logical - (int)(bh * npq);
  const int64_t off = p.Sk - p.Sq;  // causal: row i sees keys j <= i + off

  const uint16_t* Qh = p.Q + bh * p.hq;
  const uint16_t* Kh = p.K + bh * p.hk;
  const uint16_t* Vh = p.V + bh * p.hv;

  // ---- per-thread parts of the block copies (the block start moves the resource base)
  // K: copy unit u = it * 256 + tid -> half st = u / 512, row j, slot c of that
  // half; it fetches logical chunk c ^ aswz(j) of the row's half st.
  uint32_t kvo[KCOPY];
#pragma unroll
  for (int it = 0; it < KCOPY; ++it) {
    const int u = it * kThreads + tid, st = u >> 9, j = (u >> 3) & 63, c = u & 7;
    kvo[it] = (uint32_t)j * (uint32_t)(p.ldk * 2) + (uint32_t)st * KROW +
              (uint32_t)((c ^ aswz(j)) << 4);
  }
  // V: copy unit u -> row j = u / CPR, slot c, fetching chunk c ^ vswz(j)
  uint32_t vvo[VCOPY];
#pragma unroll
  for (int it = 0; it < VCOPY; ++it) {
    const int u = it * kThreads + tid, j = u / CPR, c = u % CPR;
    vvo[it] = (uint32_t)j * (uint32_t)(p.ldv * 2) + (uint32_t)((c ^ vswz<D>(j)) << 4);
  }

  auto issue_block = [&](int t, int stage) __attribute__((always_inline)) {
    const int64_t k0 = (int64_t)t * kBN;
    const int64_t rows = p.Sk - k0;  // >= 1
    const __amdgpu_buffer_rsrc_t rK = make_rsrc(Kh + k0 * p.ldk, ((rows - 1) * p.ldk + D) * 2);
#pragma unroll
    for (int it = 0; it < KCOPY; ++it)
      buffer_load_lds16(rK, (stage ? sK1 : sK0) + (it * kThreads + wave * 64) * 16, kvo[it], 0);
    const __amdgpu_buffer_rsrc_t rV = make_rsrc(Vh + k0 * p.ldv, ((rows - 1) * p.ldv + D) * 2);
#pragma unroll
    for (int it = 0; it < VCOPY; ++it)
      buffer_load_lds16(rV, (stage ? sV1 : sV0) + (it * kThreads + wave * 64) * 16, vvo[it], 0);
  };
  // Fragment reads.  Row 32t + l%32 of a K half-tile has
  // aswz = aswz(l%32) ^ (4t & 7), and the chunk a lane half h reads at d step
  // s is (2s + h) ^ aswz = ((2s ^ 4t) & 7) ^ (h ^ aswz(l%32)): one of four
  // per-lane offsets (k = 0, 2, 4, 6) plus a constant, which the LDS read
  // takes as its immediate offset.
  int foff[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) foff[k] = rl * KROW + (((2 * k) ^ hl ^ aswz(rl)) << 4);
  // V operand of output tile nt: lane i of 16-lane group g reads row 4h + i/4
  // (+ the step's first key, + 8 for the second read), columns
  // 32 nt + 16 (g % 2) + 4 (i % 4) .. +3; the swizzle depends on the row only
  // through i / 4, so each tile has one per-lane offset (bytes into a V
  // stage); key step and half are constants added to it.
  int voff[NT];
  {
    const int g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      voff[nt] = (4 * hl + (i >> 2)) * VROW +
                 (((4 * nt + 2 * (g & 1) + ((i & 3) >> 1)) ^ vswz<D>(i >> 2)) << 4) +
                 ((i & 1) << 3);
  }

  const float c = p.scale * kLog2e;  // exp(scale * x) = exp2(c * x)

  const int npass = CAUSAL && 2 * pb + 1 < nqb ? 2 : 1;
#pragma unroll 1
  for (int pass = 0; pass < npass; ++pass) {
    const int qb = CAUSAL ? (pass == 0 ? nqb - 1 - pb : pb) : pb;  // the longer block first
    const int64_t q0 = (int64_t)qb * kBM;
    const int64_t i0 = q0 + wave * 32;  // the wave's first query row
    int64_t kend = p.Sk;
    if constexpr (CAUSAL) kend = min(p.Sk, q0 + kBM + off);
    const int nblk = (int)((kend + kBN - 1) / kBN);
    if (pass > 0) __syncthreads();  // every wave has read its output staging back

    // ---- Q rows of this wave, in registers: lane holds row i0 + l%32, d = 16s + 8h .. +7
    u32x4_t qf[NSTEP];
    {
      const __amdgpu_buffer_rsrc_t rQ = make_rsrc(Qh, ((p.Sq - 1) * p.ldq + D) * 2);
      const int64_t i = i0 + rl;
      const uint32_t vo = i < p.Sq ? (uint32_t)(i * p.ldq * 2) + (uint32_t)hl * 16u : kOOB;
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) qf[s] = buffer_load16(rQ, vo, (uint32_t)s * 32u);
    }

    // ---- prologue: block 0 staged, block 1 in flight
    issue_block(0, 0);
    if (nblk > 1) {
      issue_block(1, 1);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<KCOPY + VCOPY>());  // block 0 (and Q) in
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<0>());
    }
    stage_barrier();

    f32x16_t o[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[nt] = f32x16_t{};
    float m = kMinusBig;  // running row maximum of the raw scores (both lane halves agree)
    float l = 0.0f;       // this lane's part of the running row sum
    const int64_t irow = i0 + rl;
    const int64_t lim_row = CAUSAL ? min(p.Sk - 1, irow + off) : p.Sk - 1;  // last key the row sees

    // One block; ST (0 or 1) is its stage, a constant, so every LDS offset is.
    auto blk = [&](int t, auto ST) __attribute__((always_inline)) {
      constexpr int stage = decltype(ST)::value;
      const int64_t k0 = (int64_t)t * kBN;
      bool visible = true, masked = k0 + kBN > p.Sk;
      if constexpr (CAUSAL) {
        visible = k0 <= i0 + 31 + off;
        masked = masked || k0 + kBN - 1 > i0 + off;
      }
      if (visible) {
        // ---- scores S^T = K Q^T, two 32-key tiles
        // (fragment reads run two MFMAs ahead of their use: a ring of three)
        const uint8_t* kb = stage ? sK1 : sK0;
        auto kread = [&](int x) __attribute__((always_inline)) {
          const int s = x >> 1, jt = x & 1;  // d step, key tile
          const int half = s >> 2, k = ((2 * s) ^ (4 * jt)) & 7;
          return *(const u32x4_t*)(kb + foff[k >> 1] + half * (kBN * KROW) + jt * 32 * KROW);
        };
        f32x16_t sc[2] = {f32x16_t{}, f32x16_t{}};
        u32x4_t kr[3];
        kr[0] = kread(0);
        kr[1] = kread(1);
#pragma unroll
        for (int x = 0; x < 2 * NSTEP; ++x) {
          if (x + 2 < 2 * NSTEP) kr[(x + 2) % 3] = kread(x + 2);
          __builtin_amdgcn_sched_barrier(0);
          sc[x & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, kr[x % 3]), __builtin_bit_cast(bf16x8_t, qf[x >> 1]),
              sc[x & 1], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        // ---- keys past the end, or past the row's causal limit
        if (masked) {
          const int lim = (int)max(min(lim_row - k0, (int64_t)kBN), (int64_t)-1);
#pragma unroll
          for (int jt = 0; jt < 2; ++jt)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int j = jt * 32 + (v >> 2) * 8 + hl * 4 + (v & 3);
              if (j > lim) sc[jt][v] = -__builtin_huge_valf();
            }
        }
        // ---- online softmax: row maximum over both lane halves
        float mx = sc[0][0];
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[jt][v]);
        mx = half_max(mx);
        const bool move = (mx - m) * c > kRescaleSlack;  // false for an all-masked row (-inf)
        const float mnew = move ? mx : m;
        const float alpha = move ? __builtin_amdgcn_exp2f((m - mnew) * c) : 1.0f;
        m = mnew;
        const float mc = mnew * c;
        uint32_t pk[2][8];
        float rs = 0.0f;
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[jt][2 * w], c, -mc));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[jt][2 * w + 1], c, -mc));
            rs += p0 + p1;
            pk[jt][w] = pack2_bf16(p0, p1);
          }
        l = l * alpha + rs;
        if (__builtin_amdgcn_ballot_w64(move)) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) o[nt] *= alpha;
        }
        // ---- O^T += V^T P^T, four 16-key steps
        // (reads two MFMAs ahead, each fragment two transposing reads)
        const uint8_t* vb = stage ? sV1 : sV0;
        auto vread = [&](auto X) __attribute__((always_inline)) {
          constexpr int x = decltype(X)::value;
          constexpr int ks = x / NT, nt = x % NT;  // key step, output tile
          const uint8_t* q = vb + voff[nt] + ks * 16 * VROW;
          const uint2 lo = read_tr16(q), hi = read_tr16(q + 8 * VROW);
          return u32x4_t{lo.x, lo.y, hi.x, hi.y};
        };
        u32x4_t vq[3];
        vq[0] = vread(Idx<0>{});
        vq[1] = vread(Idx<1>{});
        unroll_n<4 * NT>([&](auto X) __attribute__((always_inline)) {
          constexpr int x = decltype(X)::value;
          if constexpr (x + 2 < 4 * NT) vq[(x + 2) % 3] = vread(Idx<x + 2>{});
          constexpr int ks = x / NT, nt = x % NT, jt = ks >> 1, w0 = (ks & 1) * 4;
          const u32x4_t pf = {pk[jt][w0], pk[jt][w0 + 1], pk[jt][w0 + 2], pk[jt][w0 + 3]};
          __builtin_amdgcn_sched_barrier(0);
          o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vq[x % 3]),
                                                          __builtin_bit_cast(bf16x8_t, pf), o[nt],
                                                          0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      // ---- block t+1's copies are in; then start block t+2.  The wait is
      // unconditional (nothing is in flight after the last block), so the
      // compiler knows no copy is outstanding past the barrier but those
      // issued after it, into the stage the next block does not read.
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<0>());
      stage_barrier();  // block t's stage is free; block t+1's is complete
      if (t + 2 < nblk) issue_block(t + 2, stage);
    };
    // Blocks in pairs, so that every pass round the loop has run both stages:
    // the copies in flight at the top of the loop are then only those into
    // stage 1, which the compiler can see (an odd last block runs after it).
    int t = 0;
    for (; t + 1 < nblk; t += 2) {
      blk(t, Idx<0>{});
      blk(t + 1, Idx<1>{});
    }
    if (t < nblk) blk(t, Idx<0>{});

    // ---- epilogue: O / l, rounded to BF16, staged per wave and stored in row segments
    l = half_sum(l);
    const float inv = 1.0f / l;
    {
      constexpr int RB = D * 2;       // staged row bytes
      constexpr int UPR = RB / 16;    // 16-byte units per row
      constexpr int RPI = 64 / UPR;   // rows per read instruction
      uint8_t* wb = (wave < 2 ? sK0 : sK1) + (wave & 1) * OB;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4_t x = {o[nt][4 * q] * inv, o[nt][4 * q + 1] * inv, o[nt][4 * q + 2] * inv,
                             o[nt][4 * q + 3] * inv};
          const int u = nt * 4 + q;  // unit of columns 8u .. 8u+7; this lane half's are 8u + 4h ..
          *(uint2*)(wb + rl * RB + ((u ^ (rl & (UPR - 1))) << 4) + hl * 8) =
              make_uint2(pack2_bf16(x[0], x[1]), pack2_bf16(x[2], x[3]));
        }
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0<63>());  // own region: no barrier
      uint16_t* Oh = p.O + bh * p.ho;
#pragma unroll
      for (int it = 0; it < 32 / RPI; ++it) {
        const int r = it * RPI + lane / UPR, u = lane % UPR;
        const u32x4_t v = *(const u32x4_t*)(wb + r * RB + ((u ^ (r & (UPR - 1))) << 4));
        const int64_t i = i0 + r;
        if (i < p.Sq) *(u32x4_t*)(Oh + i * p.ldo + u * 8) = v;
      }
    }
    if (p.lse && hl == 0 && irow < p.Sq) p.lse[bh * p.Sq + irow] = m * p.scale + __logf(l);
  }  // pass
}

template <int D, bool CAUSAL>
hipError_t launch(const AttnArgs& a, hipStream_t s) {
  const int64_t nqb = (a.Sq + kBM - 1) / kBM;
  const int64_t wgs = (CAUSAL ? (nqb + 1) / 2 : nqb) * a.BH;
  hipLaunchKernelGGL((attention_kernel<D, CAUSAL>), dim3((unsigned)wgs), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_bf16(const AttnArgs& a, int d, int causal, hipStream_t s) {
  if (d == 64) return causal ? launch<64, true>(a, s) : launch<64, false>(a, s);
  return causal ? launch<128, true>(a, s) : launch<128, false>(a, s);
}

}  // namespace dmu
