/*
 * CPU oracle for the dense matrix-unit GEMM path (test infrastructure only).
 *
 * This file is the plain, slow, obviously-correct definition that the HIP
 * kernels are checked against.  Nothing in the product library links it; only
 * the test suite, the smoke check and the CPU-baseline leg of the benchmark
 * load it.  It shares no source, header, table or helper with the GPU path.
 *
 * Sources for what is computed (cited by page title and section):
 *  - "Tensor Cores: Matrix Instructions, Swizzling and FP8, Measured"
 *    (vidyal.ai), Step 1: an MMA instruction computes D = A*B + C; Step 2:
 *    B stored N x K, inputs rounded to BF16, FP32 results, error measured
 *    against an FP64 product; Step 5: FP8 E4M3 inputs with an FP32
 *    accumulator, promotion of partial sums per block of K.
 *  - "Tensor Cores" chapter (ai-infra-handbooks), section "Precision: FP16,
 *    BF16, TF32, FP8": bit splits BF16 1/8/7, E4M3 1/4/3, E5M2 1/5/2; FP8 GEMMs
 *    carry per-tensor, per-row or per-block scaling factors.
 *  - "Tensor cores and low precision" (learn-kernels.com), opening
 *    paragraphs: E4M3 has no infinity and a largest normal of 448, E5M2 keeps
 *    IEEE specials and reaches 57,344; a tensor is scaled so its largest
 *    values sit near that maximum, cast down, and the scale is removed after
 *    the multiply.
 *
 * Readings where the pages leave a step open (each also listed in the design
 * notes): E4M3 is the OCP "FN" variant (no Inf, NaN = S.1111.111); FP8 encode
 * saturates to +-max instead of producing Inf/NaN; the quantizer multiplies by
 * m = fl32(FMAX/amax) and stores the dequantisation factor s = fl32(amax/FMAX);
 * an all-zero block uses m = s = 1; a block holding a NaN has amax = NaN, one
 * holding an Inf (and no NaN) has amax = +Inf; NaN encodes to 0x7F/0xFF.
 *
 * Everything is FP64 with exact decoding.  Each output element is summed in
 * increasing k order; no blocking or reordering of the sums.
 * Build: gcc -O2 -fopenmp -ffp-contract=off (never -ffast-math).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_FMT_E4M3 0
#define ORC_FMT_E5M2 1
#define ORC_FMT_E2M1 4 /* FP4 element format of MXFP4, two per byte */
#define ORC_B_ROW_MAJOR 0 /* B(k,j) at B[k*ldb + j] */
#define ORC_B_COL_MAJOR 1 /* B(k,j) at B[j*ldb + k], i.e. B stored N x K */
#define ORC_SCALE_TENSOR 0
#define ORC_SCALE_BLOCK 1
#define ORC_BLOCK 128

/* Number of OpenMP threads the oracle's parallel loops use. */
int orc_num_threads(void) { return omp_get_max_threads(); }

/* ---------------------------------------------------------------- decoders */

/* BF16 is the upper half of an IEEE binary32 (1 sign, 8 exponent, 7 fraction
 * bits); widening is exact. */
double orc_decode_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* FP8 E4M3 (OCP FN, exponent bias 7) and E5M2 (IEEE-like, bias 15), decoded
 * from the sign/exponent/mantissa fields. */
double orc_decode_fp8(uint8_t v, int fmt) {
  int s = v >> 7;
  double sign = s ? -1.0 : 1.0;
  if (fmt == ORC_FMT_E4M3) {
    int e = (v >> 3) & 15, m = v & 7;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) return sign * ldexp((double)m, -9);        /* m/8 * 2^(1-7) */
    return sign * ldexp((double)(8 + m), e - 10);          /* (1+m/8) * 2^(e-7) */
  } else {
    int e = (v >> 2) & 31, m = v & 3;
    if (e == 31) return m == 0 ? sign * INFINITY : NAN;
    if (e == 0) return sign * ldexp((double)m, -16);       /* m/4 * 2^(1-15) */
    return sign * ldexp((double)(4 + m), e - 17);          /* (1+m/4) * 2^(e-15) */
  }
}

void orc_decode_bf16_array(const uint16_t* h, int64_t n, double* out) {
  for (int64_t i = 0; i < n; i++) out[i] = orc_decode_bf16(h[i]);
}

void orc_decode_fp8_array(const uint8_t* v, int64_t n, int fmt, double* out) {
  for (int64_t i = 0; i < n; i++) out[i] = orc_decode_fp8(v[i], fmt);
}

/* E2M1 (FP4 of the microscaling formats): sign, 2 exponent bits with bias 1,
 * 1 mantissa bit, no Inf or NaN.  Exponent field 0 is subnormal (m * 2^-1),
 * so the magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.  The low 4 bits of `v`
 * are the code. */
double orc_decode_fp4(uint8_t v) {
  double sign = (v & 8) ? -1.0 : 1.0;
  int e = (v >> 1) & 3, m = v & 1;
  if (e == 0) return sign * 0.5 * m;
  return sign * ldexp(2.0 + m, e - 2); /* (1 + m/2) * 2^(e-1) */
}

/* ---------------------------------------------------------------- encoders */

/* Round a finite, non-negative double a to the grid of a binary format with
 * `mbits` fraction bits and smallest normal exponent `emin` (no upper limit),
 * ties to even.  Works on values: the quantum of a's binade (or of the
 * subnormal range) divides a exactly in FP64, and rint() rounds half to even
 * in the default rounding mode. */
static double round_to_grid(double a, int mbits, int emin) {
  if (a == 0.0) return 0.0;
  int e2;
  frexp(a, &e2);          /* a = f * 2^e2, f in [0.5, 1) */
  int E = e2 - 1;         /* a in [2^E, 2^(E+1)) */
  if (E < emin) E = emin; /* subnormal range shares the smallest normal quantum */
  double q = ldexp(1.0, E - mbits);
  return rint(a / q) * q;
}

/* FP32 -> BF16, round to nearest even; overflow goes to Inf (BF16 has Inf);
 * NaN becomes the quiet NaN 0x7FC0 with the input's sign; no flush to zero. */
uint16_t orc_encode_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  if (isnan(x)) return (uint16_t)(sign | 0x7FC0u);
  double a = fabs((double)x);
  if (isinf(x)) return (uint16_t)(sign | 0x7F80u);
  double v = round_to_grid(a, 7, -126);
  if (v >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
  /* v is exactly a BF16 value, hence exactly an FP32 value whose low 16 bits
   * are zero. */
  float fv = (float)v;
  uint32_t w;
  memcpy(&w, &fv, sizeof w);
  return (uint16_t)(sign | (w >> 16));
}

/* A finite or infinite double -> FP8 with round to nearest even and
 * saturation: magnitudes at or above the format's largest finite value (Inf
 * included) become +-max; NaN becomes 0x7F / 0xFF. */
static uint8_t encode_fp8_d(double x, int fmt) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return (uint8_t)(sign | 0x7F);
  const int mbits = fmt == ORC_FMT_E4M3 ? 3 : 2;
  const int bias = fmt == ORC_FMT_E4M3 ? 7 : 15;
  const int emin = 1 - bias;
  const double fmax = fmt == ORC_FMT_E4M3 ? 448.0 : 57344.0;
  const uint8_t maxcode = fmt == ORC_FMT_E4M3 ? 0x7E : 0x7B;
  double a = fabs(x);
  if (a >= fmax) return (uint8_t)(sign | maxcode);
  double v = round_to_grid(a, mbits, emin);
  if (v == 0.0) return sign;
  /* Recover the fields of the representable value v. */
  int e2;
  frexp(v, &e2);
  int E = e2 - 1;
  int efield, mfield;
  if (E < emin) {
    efield = 0;
    mfield = (int)(v / ldexp(1.0, emin - mbits));
  } else {
    efield = E + bias;
    mfield = (int)(v / ldexp(1.0, E - mbits)) - (1 << mbits);
  }
  return (uint8_t)(sign | (efield << mbits) | mfield);
}

/* A finite or infinite double -> E2M1 with round to nearest even and
 * saturation at +-6 (the format has no Inf); -0 keeps its sign.  NaN input
 * has no code: it gives the signed zero, and the MX quantizer marks its block
 * with the NaN scale instead. */
static uint8_t encode_fp4_d(double x) {
  uint8_t sign = signbit(x) ? 0x8 : 0x0;
  if (isnan(x)) return sign;
  double a = fabs(x);
  if (a >= 6.0) return (uint8_t)(sign | 0x7);
  double v = round_to_grid(a, 1, 0);
  if (v == 0.0) return sign;
  if (v < 1.0) return (uint8_t)(sign | 0x1); /* the subnormal 0.5 */
  int e2;
  frexp(v, &e2);
  int E = e2 - 1; /* v in [2^E, 2^(E+1)), E in 0..2 */
  int mfield = (int)(v / ldexp(1.0, E - 1)) - 2;
  return (uint8_t)(sign | ((E + 1) << 1) | mfield);
}

uint8_t orc_encode_fp4(float x) { return encode_fp4_d((double)x); }

/* FP32 -> FP8 with round to nearest even and saturation (see encode_fp8_d;
 * the FP32 value widens exactly). */
uint8_t orc_encode_fp8(float x, int fmt) { return encode_fp8_d((double)x, fmt); }

void orc_encode_bf16_array(const float* x, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = orc_encode_bf16(x[i]);
}

void orc_encode_fp8_array(const float* x, int64_t n, int fmt, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = orc_encode_fp8(x[i], fmt);
}

/* One E2M1 code per output byte (unpacked), for tests. */
void orc_encode_fp4_array(const float* x, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = orc_encode_fp4(x[i]);
}

void orc_decode_fp4_array(const uint8_t* v, int64_t n, double* out) {
  for (int64_t i = 0; i < n; i++) out[i] = orc_decode_fp4(v[i]);
}

/* ---------------------------------------------------------------- quantize */

/* Per-block FP8 quantisation: amax over the block, m = fl32(FMAX/amax),
 * q = encode(fl32(x*m)), stored scale s = fl32(amax/FMAX) so x ~ decode(q)*s.
 * Blocks are block_rows x block_cols; scales are row-major
 * [rows/block_rows][cols/block_cols].  Returns 0, or -1 on bad arguments. */
int orc_quantize_fp8(const float* X, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                     int64_t block_rows, int64_t block_cols, uint8_t* Q, int64_t ldq,
                     float* scales) {
  if (rows <= 0 || cols <= 0 || block_rows <= 0 || block_cols <= 0) return -1;
  if (rows % block_rows || cols % block_cols || ldx < cols || ldq < cols) return -1;
  if (fmt != ORC_FMT_E4M3 && fmt != ORC_FMT_E5M2) return -1;
  const float fmax = fmt == ORC_FMT_E4M3 ? 448.0f : 57344.0f;
  const int64_t nbr = rows / block_rows, nbc = cols / block_cols;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t bi = 0; bi < nbr; bi++) {
    for (int64_t bj = 0; bj < nbc; bj++) {
      float amax = 0.0f;
      int has_nan = 0;
      for (int64_t r = bi * block_rows; r < (bi + 1) * block_rows; r++)
        for (int64_t c = bj * block_cols; c < (bj + 1) * block_cols; c++) {
          float x = X[r * ldx + c];
          if (isnan(x)) has_nan = 1;
          else if (fabsf(x) > amax) amax = fabsf(x);
        }
      if (has_nan) amax = NAN;
      float m, s;
      if (amax == 0.0f) {
        m = 1.0f;
        s = 1.0f;
      } else {
        m = fmax / amax;
        s = amax / fmax;
      }
      for (int64_t r = bi * block_rows; r < (bi + 1) * block_rows; r++)
        for (int64_t c = bj * block_cols; c < (bj + 1) * block_cols; c++) {
          float y = X[r * ldx + c] * m;
          Q[r * ldq + c] = orc_encode_fp8(y, fmt);
        }
      scales[bi * nbc + bj] = s;
    }
  }
  return 0;
}

/* ---------------------------------------------------------------- GEMMs */

/* Selected rows of D = A*B + C in FP64, plus S = sum_k |a_ik * b_kj| (the
 * magnitude that the tolerance scales with).  A is M x K row-major BF16, B is
 * K x N given row-major or column-major (= stored N x K).  C (FP32 M x N,
 * row-major) may be NULL.  rows == NULL means all M rows.  Outputs D and S are
 * [nrows][N] row-major doubles (S may be NULL). */
int orc_gemm_bf16(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int b_layout,
                  const float* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                  const int64_t* rows, int64_t nrows, double* D, double* S) {
  if (M <= 0 || N <= 0 || K <= 0) return -1;
  if (b_layout != ORC_B_ROW_MAJOR && b_layout != ORC_B_COL_MAJOR) return -1;
  if (!rows) nrows = M;
  double* tab = (double*)malloc(65536 * sizeof(double));
  if (!tab) return -2;
  for (int h = 0; h < 65536; h++) tab[h] = orc_decode_bf16((uint16_t)h);
  int bad = 0;
#pragma omp parallel for schedule(dynamic)
  for (int64_t r = 0; r < nrows; r++) {
    int64_t i = rows ? rows[r] : r;
    if (i < 0 || i >= M) { bad = 1; continue; }
    double* d = D + r * N;
    double* s = S ? S + r * N : NULL;
    if (b_layout == ORC_B_COL_MAJOR) {
      for (int64_t j = 0; j < N; j++) {
        double acc = 0.0, sacc = 0.0;
        for (int64_t k = 0; k < K; k++) {
          double p = tab[A[i * lda + k]] * tab[B[j * ldb + k]];
          acc += p;
          sacc += fabs(p);
        }
        d[j] = acc;
        if (s) s[j] = sacc;
      }
    } else {
      for (int64_t j = 0; j < N; j++) d[j] = 0.0;
      if (s) for (int64_t j = 0; j < N; j++) s[j] = 0.0;
      for (int64_t k = 0; k < K; k++) {
        double a = tab[A[i * lda + k]];
        const uint16_t* brow = B + k * ldb;
        for (int64_t j = 0; j < N; j++) {
          double p = a * tab[brow[j]];
          d[j] += p;
          if (s) s[j] += fabs(p);
        }
      }
    }
    if (C)
      for (int64_t j = 0; j < N; j++) d[j] += (double)C[i * ldc + j];
  }
  free(tab);
  return bad ? -1 : 0;
}

/* Selected rows of the scaled FP8 product.  A is M x K row-major, B is stored
 * N x K (column-major B), both FP8 codes in formats fmt_a / fmt_b.
 *  per-tensor: D = sa[0]*sb[0]*sum_k a_ik b_jk + C
 *  per-block:  D = sum_kb sa[i][kb]*sb[j/128][kb]*(sum_{k in kb} a_ik b_jk) + C,
 *              sa is [M][K/128], sb is [ceil(N/128)][K/128], both row-major;
 *              each 128-wide partial sum is formed first and then scaled
 *              (promotion of per-block partial sums).
 * S receives sum |a*scale_a| * |b*scale_b| over k. */
int orc_gemm_fp8(const uint8_t* A, int64_t lda, int fmt_a, const uint8_t* B, int64_t ldb,
                 int fmt_b, const float* sa, const float* sb, int scale_mode, const float* C,
                 int64_t ldc, int64_t M, int64_t N, int64_t K, const int64_t* rows,
                 int64_t nrows, double* D, double* S) {
  if (M <= 0 || N <= 0 || K <= 0) return -1;
  if (scale_mode != ORC_SCALE_TENSOR && scale_mode != ORC_SCALE_BLOCK) return -1;
  if (scale_mode == ORC_SCALE_BLOCK && K % ORC_BLOCK) return -1;
  if (!rows) nrows = M;
  double ta[256], tb[256];
  for (int v = 0; v < 256; v++) {
    ta[v] = orc_decode_fp8((uint8_t)v, fmt_a);
    tb[v] = orc_decode_fp8((uint8_t)v, fmt_b);
  }
  const int64_t nkb = K / ORC_BLOCK;
  int bad = 0;
#pragma omp parallel for schedule(dynamic)
  for (int64_t r = 0; r < nrows; r++) {
    int64_t i = rows ? rows[r] : r;
    if (i < 0 || i >= M) { bad = 1; continue; }
    for (int64_t j = 0; j < N; j++) {
      const uint8_t* arow = A + i * lda;
      const uint8_t* bcol = B + j * ldb;
      double out, sabs;
      if (scale_mode == ORC_SCALE_TENSOR) {
        double acc = 0.0, sacc = 0.0;
        for (int64_t k = 0; k < K; k++) {
          double p = ta[arow[k]] * tb[bcol[k]];
          acc += p;
          sacc += fabs(p);
        }
        double sc = (double)sa[0] * (double)sb[0];
        out = acc * sc;
        sabs = sacc * fabs(sc);
      } else {
        out = 0.0;
        sabs = 0.0;
        for (int64_t kb = 0; kb < nkb; kb++) {
          double part = 0.0, spart = 0.0;
          for (int64_t k = kb * ORC_BLOCK; k < (kb + 1) * ORC_BLOCK; k++) {
            double p = ta[arow[k]] * tb[bcol[k]];
            part += p;
            spart += fabs(p);
          }
          double sc = (double)sa[i * nkb + kb] * (double)sb[(j / ORC_BLOCK) * nkb + kb];
          out += part * sc;
          sabs += spart * fabs(sc);
        }
      }
      if (C) out += (double)C[i * ldc + j];
      D[r * N + j] = out;
      if (S) S[r * N + j] = sabs;
    }
  }
  return bad ? -1 : 0;
}

/* ---------------------------------------------------------------- MX (microscaling) */

/* Microscaling block formats: every group of 32 consecutive elements along a
 * row shares one scale that is a bare power of two stored as an 8-bit
 * exponent (E8M0: code c means 2^(c-127), code 255 is NaN), and a block-scaled
 * product multiplies every element by its group's scale ("How Blackwell's
 * Tensor Memory Actually Works", section "Quantization became an allocation
 * problem": D = C + (A x SFA)(B x SFB) with one scale per 16 or 32 elements
 * along K; the 32-element, E8M0 variant follows the Open Compute
 * microscaling specification). */
#define ORC_MX_BLOCK 32

double orc_decode_e8m0(uint8_t c) { return c == 255 ? NAN : ldexp(1.0, (int)c - 127); }

/* Quantise rows x cols FP32 (row-major, cols % 32 == 0) to FP8 or FP4 (E2M1)
 * with one E8M0 scale per 1 x 32 block.  Scale choice, read from the
 * microscaling specification: X = 2^(floor(log2 amax) - emax), emax the
 * largest exponent of the element format (8 for E4M3, 15 for E5M2, 2 for
 * E2M1), the exponent clamped to the E8M0 range [-127, 127]; elements q =
 * saturating RNE of x / X (exact: X is a power of two).  Readings where the
 * pages say nothing: an all-zero block takes the smallest scale 2^-127; a
 * block holding a NaN or an infinity gets the NaN scale 255 and NaN element
 * codes (FP8) or signed zeros (FP4, which has no NaN).  Q has ldq bytes per
 * row: one code per byte (FP8), or two (FP4: element k in the low nibble of
 * byte k/2 when k is even, the high nibble when odd).  S is row-major
 * [rows][lds], lds >= cols/32. */
int orc_quantize_mx(const float* X, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* Q,
                    int64_t ldq, uint8_t* S, int64_t lds) {
  const int fp4 = fmt == ORC_FMT_E2M1;
  if (rows <= 0 || cols <= 0 || cols % ORC_MX_BLOCK || ldx < cols) return -1;
  if (ldq < (fp4 ? cols / 2 : cols) || lds < cols / ORC_MX_BLOCK) return -1;
  if (fmt != ORC_FMT_E4M3 && fmt != ORC_FMT_E5M2 && !fp4) return -1;
  const int emax = fmt == ORC_FMT_E4M3 ? 8 : fmt == ORC_FMT_E5M2 ? 15 : 2;
  const int64_t nb = cols / ORC_MX_BLOCK;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t r = 0; r < rows; r++) {
    for (int64_t b = 0; b < nb; b++) {
      const float* x = X + r * ldx + b * ORC_MX_BLOCK;
      uint8_t* q = Q + r * ldq + b * (fp4 ? ORC_MX_BLOCK / 2 : ORC_MX_BLOCK);
      uint8_t c[ORC_MX_BLOCK];
      double amax = 0.0;
      int nonfinite = 0;
      for (int k = 0; k < ORC_MX_BLOCK; k++) {
        if (!isfinite(x[k])) nonfinite = 1;
        else if (fabs((double)x[k]) > amax) amax = fabs((double)x[k]);
      }
      if (nonfinite) {
        S[r * lds + b] = 255;
        for (int k = 0; k < ORC_MX_BLOCK; k++)
          c[k] = fp4 ? (uint8_t)(signbit(x[k]) ? 0x8 : 0x0)
                     : (uint8_t)(signbit(x[k]) ? 0xFF : 0x7F);
      } else {
      int e;
      if (amax == 0.0) {
        e = -127;
      } else {
        int e2;
        frexp(amax, &e2); /* amax = f * 2^e2, f in [0.5, 1): floor(log2 amax) = e2 - 1 */
        e = e2 - 1 - emax;
        if (e < -127) e = -127;
        if (e > 127) e = 127;
      }
      S[r * lds + b] = (uint8_t)(e + 127);
      for (int k = 0; k < ORC_MX_BLOCK; k++) {
        const double y = ldexp((double)x[k], -e);
        c[k] = fp4 ? encode_fp4_d(y) : encode_fp8_d(y, fmt);
      }
      }
      if (fp4)
        for (int k = 0; k < ORC_MX_BLOCK; k += 2) q[k / 2] = (uint8_t)(c[k] | (c[k + 1] << 4));
      else
        for (int k = 0; k < ORC_MX_BLOCK; k++) q[k] = c[k];
    }
  }
  return 0;
}

/* Element k of a row of codes: a byte (FP8) or a nibble (FP4, packed as in
 * orc_quantize_mx). */
static int code_at(const uint8_t* row, int64_t k, int fmt) {
  if (fmt == ORC_FMT_E2M1) return (row[k >> 1] >> ((k & 1) * 4)) & 15;
  return row[k];
}

/* Selected rows of the MX product: A is M x K row-major, B stored N x K, FP8
 * or FP4 codes (fmt_a, fmt_b; lda, ldb in bytes); SA [M][ldsa] and SB [N][ldsb]
 * hold one E8M0 code per 32-element group along K.  D = C + sum_k (a_ik * sa_i,k/32) * (b_jk *
 * sb_j,k/32) in FP64, k ascending; S = sum_k of the magnitudes. */
int orc_gemm_mx(const uint8_t* A, int64_t lda, int fmt_a, const uint8_t* B, int64_t ldb, int fmt_b,
                const uint8_t* SA, int64_t ldsa, const uint8_t* SB, int64_t ldsb, const float* C,
                int64_t ldc, int64_t M, int64_t N, int64_t K, const int64_t* rows, int64_t nrows,
                double* D, double* S) {
  if (M <= 0 || N <= 0 || K <= 0 || K % ORC_MX_BLOCK) return -1;
  if (!rows) nrows = M;
  const int ok = (fmt_a == ORC_FMT_E4M3 || fmt_a == ORC_FMT_E5M2 || fmt_a == ORC_FMT_E2M1) &&
                 (fmt_b == ORC_FMT_E4M3 || fmt_b == ORC_FMT_E5M2 || fmt_b == ORC_FMT_E2M1);
  if (!ok) return -1;
  double ta[256], tb[256];
  for (int v = 0; v < 256; v++) {
    ta[v] = fmt_a == ORC_FMT_E2M1 ? orc_decode_fp4((uint8_t)v) : orc_decode_fp8((uint8_t)v, fmt_a);
    tb[v] = fmt_b == ORC_FMT_E2M1 ? orc_decode_fp4((uint8_t)v) : orc_decode_fp8((uint8_t)v, fmt_b);
  }
  /* every scale decoded once (exact powers of two, or NaN) */
  const int64_t ng = K / ORC_MX_BLOCK;
  double* sB = (double*)malloc((size_t)N * ng * sizeof(double));
  if (!sB) return -1;
  for (int64_t j = 0; j < N; j++)
    for (int64_t g = 0; g < ng; g++) sB[j * ng + g] = orc_decode_e8m0(SB[j * ldsb + g]);
  int bad = 0;
#pragma omp parallel for schedule(dynamic)
  for (int64_t r = 0; r < nrows; r++) {
    int64_t i = rows ? rows[r] : r;
    if (i < 0 || i >= M) { bad = 1; continue; }
    double sA[ng > 0 ? ng : 1];
    for (int64_t g = 0; g < ng; g++) sA[g] = orc_decode_e8m0(SA[i * ldsa + g]);
    for (int64_t j = 0; j < N; j++) {
      double acc = 0.0, sacc = 0.0;
      for (int64_t k = 0; k < K; k++) {
        const int64_t g = k / ORC_MX_BLOCK;
        double p = (ta[code_at(A + i * lda, k, fmt_a)] * sA[g]) *
                   (tb[code_at(B + j * ldb, k, fmt_b)] * sB[j * ng + g]);
        acc += p;
        sacc += fabs(p);
      }
      if (C) acc += (double)C[i * ldc + j];
      D[r * N + j] = acc;
      if (S) S[r * N + j] = sacc;
    }
  }
  free(sB);
  return bad ? -1 : 0;
}

/* ---------------------------------------------------------------- grouped (MoE) */

/* Grouped product of a mixture-of-experts layer ("How Blackwell's Tensor
 * Memory Actually Works", section "What this does to serving economics", the
 * third consequence: each expert multiplies the rows routing sent it, so every
 * expert's GEMM has its own M, which changes from step to step).  Rows
 * off[g] .. off[g+1]-1 of A (row-major BF16, lda) belong to expert g, whose
 * weight is the N x K BF16 matrix stored N x K (ldb) at B + g * stride_b;
 * D[r][j] = sum_k A[r][k] * B_g[j][k] in FP64, k ascending; S the same sum of
 * magnitudes.  off holds G + 1 non-decreasing entries, off[0] >= 0.  `rows`
 * (nrows entries) selects which rows of A / D to compute, else all rows
 * off[0] .. off[G]-1 (nrows is then ignored); a selected row outside every
 * group is an error. */
int orc_gemm_grouped_bf16(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                          int64_t stride_b, const int64_t* off, int64_t G, int64_t N, int64_t K,
                          const int64_t* rows, int64_t nrows, double* D, double* S) {
  if (G <= 0 || N <= 0 || K <= 0 || off[0] < 0) return -1;
  for (int64_t g = 0; g < G; g++)
    if (off[g + 1] < off[g]) return -1;
  if (!rows) nrows = off[G] - off[0];
  double* tab = (double*)malloc(65536 * sizeof(double));
  if (!tab) return -2;
  for (int h = 0; h < 65536; h++) tab[h] = orc_decode_bf16((uint16_t)h);
  int bad = 0;
#pragma omp parallel for schedule(dynamic)
  for (int64_t q = 0; q < nrows; q++) {
    const int64_t r = rows ? rows[q] : off[0] + q;
    int64_t g = 0;
    while (g < G && !(off[g] <= r && r < off[g + 1])) g++;
    if (g == G) { bad = 1; continue; }
    const uint16_t* Bg = B + g * stride_b;
    for (int64_t j = 0; j < N; j++) {
      double acc = 0.0, sacc = 0.0;
      for (int64_t k = 0; k < K; k++) {
        double p = tab[A[r * lda + k]] * tab[Bg[j * ldb + k]];
        acc += p;
        sacc += fabs(p);
      }
      D[q * N + j] = acc;
      if (S) S[q * N + j] = sacc;
    }
  }
  free(tab);
  return bad ? -1 : 0;
}

/* ---------------------------------------------------------------- fused epilogue */

/* The epilogue applied to the accumulator while it is still at hand ("How
 * Blackwell's Tensor Memory Actually Works", section "The cost of getting the
 * answer back": scale it, add a bias, apply an activation, cast down):
 * Y[i][j] = act(alpha * D[i][j] + bias[j]) in FP64 for a rows x N block of
 * FP64 products (bias may be NULL).  act: 0 none; 1 ReLU, x > 0 ? x : 0 (so
 * NaN gives 0); 2 GELU, x * Phi(x) with Phi the standard normal distribution
 * function 0.5 * (1 + erf(x / sqrt 2)); 3 SiLU, x / (1 + exp(-x)).  The cast
 * is left to the caller. */
int orc_epilogue(const double* D, int64_t rows, int64_t N, double alpha, const float* bias,
                 int act, double* Y) {
  if (rows < 0 || N <= 0 || act < 0 || act > 3) return -1;
  for (int64_t i = 0; i < rows; i++) {
    for (int64_t j = 0; j < N; j++) {
      double x = alpha * D[i * N + j] + (bias ? (double)bias[j] : 0.0);
      if (act == 1) x = x > 0.0 ? x : 0.0;
      else if (act == 2) x = x * 0.5 * (1.0 + erf(x / sqrt(2.0)));
      else if (act == 3) x = x / (1.0 + exp(-x));
      Y[i * N + j] = x;
    }
  }
  return 0;
}

/* ---------------------------------------------------------------- attention chain */

/* Two products chained through an elementwise step: the scores of the first
 * feed, after a row-wise softmax, the second.  The "Tensor Cores" chapter
 * (ai-infra-handbooks), section "mma.sync: the register layout is explicit",
 * names this as the case FlashAttention needs (one product's output consumed
 * by the next, elementwise work done on the result in between), and
 * "Tensor Cores: Matrix Instructions, Swizzling and FP8, Measured"
 * (vidyal.ai), section "In the real world", cites FlashAttention as the
 * kernel built that way.  The pages do not restate attention itself; this is
 * its textbook definition, per head bh and query row i:
 *
 *   s_j = scale * sum_k q[i][k] * k[j][k]      for the keys j the row sees
 *   w_j = exp(s_j - max_j s_j),  l = sum_j w_j
 *   O[i][n]   = sum_j w_j * v[j][n] / l
 *   lse[i]    = max_j s_j + log l              (log of sum_j exp(s_j))
 *   Aabs[i][n] = sum_j w_j * |v[j][n]| / l      (for error bounds)
 *
 * Non-causal rows see every key; causal rows see keys j <= i + (Sk - Sq)
 * (the last query row sees every key), which needs Sq <= Sk.  Q is
 * [BH][Sq][d], K and V [BH][Sk][d], all BF16 bit patterns, contiguous;
 * outputs are FP64 [BH][Sq][d] and [BH][Sq]; lse and Aabs may be NULL.
 * Inputs are decoded exactly and every sum runs in increasing index order. */
int orc_attention_bf16(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int64_t BH,
                       int64_t Sq, int64_t Sk, int64_t d, double scale, int causal, double* O,
                       double* lse, double* Aabs) {
  if (BH < 1 || Sq < 1 || Sk < 1 || d < 1 || (causal && Sq > Sk)) return -1;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
  for (int64_t bh = 0; bh < BH; bh++) {
    for (int64_t i = 0; i < Sq; i++) {
      const uint16_t* q = Q + (bh * Sq + i) * d;
      const int64_t nk = causal ? i + (Sk - Sq) + 1 : Sk;
      double* s = (double*)malloc((size_t)nk * sizeof(double));
      if (!s) {
#pragma omp atomic write
        bad = 1;
        continue;
      }
      double m = -INFINITY;
      /* s_j = scale * sum_k q_k k_jk, each sum in increasing k; four keys at a
       * time, their four sums kept apart */
      int64_t j = 0;
      for (; j + 4 <= nk; j += 4) {
        const uint16_t* k0 = K + (bh * Sk + j) * d;
        double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
        for (int64_t k = 0; k < d; k++) {
          const double qk = orc_decode_bf16(q[k]);
          a0 += qk * orc_decode_bf16(k0[k]);
          a1 += qk * orc_decode_bf16(k0[d + k]);
          a2 += qk * orc_decode_bf16(k0[2 * d + k]);
          a3 += qk * orc_decode_bf16(k0[3 * d + k]);
        }
        s[j] = scale * a0, s[j + 1] = scale * a1, s[j + 2] = scale * a2, s[j + 3] = scale * a3;
      }
      for (; j < nk; j++) {
        const uint16_t* kr = K + (bh * Sk + j) * d;
        double acc = 0.0;
        for (int64_t k = 0; k < d; k++) acc += orc_decode_bf16(q[k]) * orc_decode_bf16(kr[k]);
        s[j] = scale * acc;
      }
      for (j = 0; j < nk; j++)
        if (s[j] > m) m = s[j];
      double l = 0.0;
      for (int64_t j = 0; j < nk; j++) {
        s[j] = exp(s[j] - m);
        l += s[j];
      }
      double* o = O + (bh * Sq + i) * d;
      double* a = Aabs ? Aabs + (bh * Sq + i) * d : NULL;
      /* o[n] = sum_j s[j] v[j][n] / l, each sum taken in increasing j (the
       * rows of V are walked in memory order, one accumulator per column) */
      double* acc = (double*)calloc((size_t)(2 * d), sizeof(double));
      if (!acc) {
#pragma omp atomic write
        bad = 1;
        free(s);
        continue;
      }
      double* aa = acc + d;
      for (int64_t j = 0; j < nk; j++) {
        const uint16_t* vr = V + (bh * Sk + j) * d;
        for (int64_t n = 0; n < d; n++) {
          const double v = orc_decode_bf16(vr[n]);
          acc[n] += s[j] * v;
          aa[n] += s[j] * fabs(v);
        }
      }
      for (int64_t n = 0; n < d; n++) {
        o[n] = acc[n] / l;
        if (a) a[n] = aa[n] / l;
      }
      if (lse) lse[bh * Sq + i] = m + log(l);
      free(acc);
      free(s);
    }
  }
  return bad ? -1 : 0;
}
