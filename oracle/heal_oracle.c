/*
 * heal_oracle.c -- the plain CPU oracle for the HEAL hot path.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg load this library.  The
 * product path (the HIP library) never calls it, and the two share no source, header or table.
 *
 * Everything here is written for a reader who checks it against the pages by eye: straight loops in the
 * order of the definitions, FP64 wherever the pages leave the precision open, and the 16-bit conversions
 * written out from the IEEE 754 definition instead of taken from a compiler intrinsic.  OpenMP is used
 * only to run independent output elements on several cores; it never changes an order of summation.
 *
 * Sources (cited by page title and section, never by file position):
 *   [TS]  gist.science explainer "Demystifying Numerical Instability in LLM Inference: Achieving
 *         Reproducible Inference for Mission-Critical Tasks with HEAL", section "Technical Summary".
 *         [TS 2A] = "A. Mitigating Attention Truncation via INT16 Quantization" (Solution, Mechanism);
 *         [TS 2B] = "B. Mitigating GEMM Truncation via Algebraic Error Compensation" (Mechanism,
 *         Overflow Handling).
 *   [ABS] the authors' abstract, arXiv 2606.21023 v2 (paperdot listing).
 *
 * Readings adopted where the pages are silent (each is listed with its reason in the design notes):
 *   R-split   16-bit parts are FP16 after an exact power-of-two prescale per row, e = 14 - ilogb(max|x|),
 *             so the row maximum lands in [2^14, 2^15).  The outlier rescaling of [TS 2B Overflow
 *             Handling] read as an always-on, exact per-row scale.
 *   R-prod    the compensated product sums hi*hi + hi*lo + lo*hi (lo*lo dropped) when both operands are
 *             split, hi*hi + lo*hi when only the activations are ([TS 2B Mechanism] names two products).
 *   R-quant   symmetric INT16 per (token, head): s = fl32(max|x| / 32767), q = clamp(rint(fl32(x / s)),
 *             -32767, 32767); s = 0 (an all-zero row, or max|x| so small that s underflows) gives q = 0
 *             ([TS 2A Solution] names INT16 and no scheme).
 *   R-dual    Dual-FP16 unpack is the byte split hi = q >> 8 (floor), lo = q & 0xFF, q = 256*hi + lo;
 *             the pages write the pair with a 2^10 shift ([TS 2A Mechanism]); any shift that keeps both
 *             halves integer is exact, and 8 keeps every FP32 partial sum exact at head_dim 128.  Two
 *             other readings are built as variants: the pages' formula taken as a bit split at 10,
 *             q = 1024*hi + lo, and as a float-float pair, hi = fp16_rn(q), lo = 2^10 (q - hi), so that
 *             q = hi + lo / 2^10.
 *   R-attn    attention is graded on the dequantised inputs s*q; causal masking is bottom-right aligned
 *             (key j visible to query i when j <= i + kv_len - q_len); GQA maps query head h to key/value
 *             head h / (n_q_heads / n_kv_heads).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F16 2
#define ORC_BF16 1

/* ------------------------------------------------------------------------------------------------------
 * 16-bit conversions, written from IEEE 754-2008: round to nearest, ties to even; gradual underflow;
 * overflow to infinity; NaN stays NaN.  A finite magnitude a is rounded to the grid of its binade: the
 * spacing is 2^(e - p + 1) for a in [2^e, 2^(e+1)) with p significant bits, and never finer than the
 * subnormal spacing 2^(emin - p + 1).  Dividing by a power of two is exact in double, and nearbyint()
 * rounds to the nearest integer with ties to even under the default rounding mode.
 * ---------------------------------------------------------------------------------------------------- */
static uint16_t round_to_16bit(float x, int p /* significant bits */, int emin, int emax_bias,
                               int frac_bits) {
  uint32_t u;
  memcpy(&u, &x, 4);
  const uint16_t sign = (uint16_t)((u >> 31) << 15);
  const uint16_t exp_all_ones = (uint16_t)(((1u << (15 - frac_bits)) - 1u) << frac_bits);
  if (isnan(x)) return (uint16_t)(sign | exp_all_ones | (1u << (frac_bits - 1)));
  if (isinf(x)) return (uint16_t)(sign | exp_all_ones);
  double a = fabs((double)x);
  if (a == 0.0) return sign;
  int e = ilogb(a);
  if (e < emin) e = emin;
  const double spacing = ldexp(1.0, e - (p - 1));
  const double m = nearbyint(a / spacing);
  const double v = m * spacing; /* the rounded magnitude, exact in double */
  /* overflow: the largest finite value is (2^p - 1) * 2^(emax - p + 1); anything that rounds past it
     is >= 2^(emax + 1) and becomes infinity. */
  const int emax = emax_bias;
  if (v >= ldexp(1.0, emax + 1)) return (uint16_t)(sign | exp_all_ones);
  if (v < ldexp(1.0, emin)) {
    /* subnormal: the stored fraction is v / 2^(emin - p + 1) */
    return (uint16_t)(sign | (uint16_t)(v / ldexp(1.0, emin - (p - 1))));
  }
  const int ev = ilogb(v);
  const uint32_t frac = (uint32_t)(v / ldexp(1.0, ev - (p - 1))) - (1u << (p - 1));
  return (uint16_t)(sign | (uint16_t)((uint32_t)(ev + emax_bias) << frac_bits) | (uint16_t)frac);
}

/* binary16: p = 11, emin = -14, emax = 15 (bias 15), 10 fraction bits */
uint16_t orc_f16_bits(float x) { return round_to_16bit(x, 11, -14, 15, 10); }
/* bfloat16: p = 8, emin = -126, emax = 127 (bias 127), 7 fraction bits */
uint16_t orc_bf16_bits(float x) { return round_to_16bit(x, 8, -126, 127, 7); }

static double decode_16bit(uint16_t b, int p, int bias, int frac_bits) {
  const int sign = b >> 15;
  const int ebits = (b >> frac_bits) & ((1 << (15 - frac_bits)) - 1);
  const uint32_t frac = b & ((1u << frac_bits) - 1u);
  double v;
  if (ebits == (1 << (15 - frac_bits)) - 1) v = frac ? NAN : INFINITY;
  else if (ebits == 0) v = ldexp((double)frac, 1 - bias - (p - 1));
  else v = ldexp((double)(frac | (1u << frac_bits)), ebits - bias - (p - 1));
  return sign ? -v : v;
}
double orc_f16_value(uint16_t b) { return decode_16bit(b, 11, 15, 10); }
double orc_bf16_value(uint16_t b) { return decode_16bit(b, 8, 127, 7); }

void orc_f16_bits_array(const float* x, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_bits(x[i]);
}
void orc_bf16_bits_array(const float* x, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_bits(x[i]);
}

static uint16_t to_part(float v, int part) { return part == ORC_F16 ? orc_f16_bits(v) : orc_bf16_bits(v); }
static double part_value(uint16_t b, int part) {
  return part == ORC_F16 ? orc_f16_value(b) : orc_bf16_value(b);
}

/* ------------------------------------------------------------------------------------------------------
 * Split of an FP32 (or bf16-valued) matrix into a 16-bit leading part and the 16-bit remainder of what that
 * part could not hold: [TS 2B Mechanism], with an exact power-of-two row prescale standing for
 * [TS 2B Overflow Handling].
 *
 *   e_r = 14 - ilogb(max_c |x_rc|)   (0 when the row is all zero, or when prescale == 0)
 *   x'  = fl32(x * 2^e_r)
 *   hi  = round16(x')
 *   lo  = round16(x' - hi)           (x' - hi is exact in fp32; lo == NULL drops the residual)
 * ---------------------------------------------------------------------------------------------------- */
void orc_split_f32(const float* x, int64_t rows, int64_t cols, int64_t ld, int part, int prescale,
                   uint16_t* hi, uint16_t* lo, int64_t ld_part, int32_t* exps) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const float* row = x + r * ld;
    float amax = 0.0f;
    for (int64_t c = 0; c < cols; ++c) {
      const float a = fabsf(row[c]);
      if (a > amax) amax = a;
    }
    const int e = (prescale && amax > 0.0f) ? 14 - ilogbf(amax) : 0;
    if (exps) exps[r] = e;
    for (int64_t c = 0; c < cols; ++c) {
      const float xs = (float)((double)row[c] * ldexp(1.0, e)); /* one rounding to fp32 */
      const uint16_t h = to_part(xs, part);
      hi[r * ld_part + c] = h;
      if (lo) {
        const float resid = xs - (float)part_value(h, part);
        lo[r * ld_part + c] = to_part(resid, part);
      }
    }
  }
}

/* the same split applied to a bf16 matrix (bits in, R-split on the widened value) */
void orc_split_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int part, int prescale,
                    uint16_t* hi, uint16_t* lo, int64_t ld_part, int32_t* exps) {
  float* tmp = (float*)malloc(sizeof(float) * (size_t)(rows * cols > 0 ? rows * cols : 1));
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) tmp[r * cols + c] = (float)orc_bf16_value(x[r * ld + c]);
  orc_split_f32(tmp, rows, cols, cols, part, prescale, hi, lo, ld_part, exps);
  free(tmp);
}

/* ------------------------------------------------------------------------------------------------------
 * Dual-FP16 unpack of an INT16 tensor, [TS 2A Mechanism], byte-split reading R-dual:
 *   hi = q >> 8 (floor division by 256), lo = q & 0xFF,  q = 256*hi + lo, both halves exact in FP16.
 * Output is the FP16 bit pattern of each half.
 * ---------------------------------------------------------------------------------------------------- */
void orc_split_i16(const int16_t* q, int64_t rows, int64_t cols, int64_t ld, uint16_t* hi, uint16_t* lo,
                   int64_t ld_part) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      const int v = q[r * ld + c];
      const int h = (v - (v & 0xFF)) / 256; /* floor(v / 256): v - (v mod 256) is a multiple of 256 */
      const int l = v & 0xFF;
      hi[r * ld_part + c] = orc_f16_bits((float)h);
      lo[r * ld_part + c] = orc_f16_bits((float)l);
    }
}

/* ------------------------------------------------------------------------------------------------------
 * Dual-FP16 unpack under the three readings of R-dual ([TS 2A Mechanism]), FP16 bit patterns out:
 *   reading 0 (byte):     hi = floor(q / 256),  lo = q - 256*hi    (0 <= lo < 256)
 *   reading 1 (shift-10): hi = floor(q / 1024), lo = q - 1024*hi   (0 <= lo < 1024)
 *   reading 2 (float):    hi = q rounded to FP16 (nearest, ties to even), lo = 1024 * (q - hi)
 * Every value written is an integer (times 2^10 for the float lo) of at most 11 significant bits, so
 * its FP16 encoding is exact; the only rounding is the one that defines the float reading's hi.
 * ---------------------------------------------------------------------------------------------------- */
void orc_unpack_i16(const int16_t* q, int64_t rows, int64_t cols, int64_t ld, int reading, uint16_t* hi,
                    uint16_t* lo, int64_t ld_part) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      const int v = q[r * ld + c];
      double h, l;
      if (reading == 0 || reading == 1) {
        const int base = reading == 0 ? 256 : 1024;
        const int m = ((v % base) + base) % base; /* v mod base in [0, base) */
        h = (double)((v - m) / base);              /* exact division: v - m is a multiple of base */
        l = (double)m;
      } else {
        const uint16_t hb = orc_f16_bits((float)v);
        h = orc_f16_value(hb);
        l = 1024.0 * ((double)v - h);
      }
      hi[r * ld_part + c] = orc_f16_bits((float)h);
      lo[r * ld_part + c] = orc_f16_bits((float)l);
    }
}

/* ------------------------------------------------------------------------------------------------------
 * INT16 quantisation of Q/K/V, [TS 2A Solution] and [ABS], reading R-quant.  x is [tokens, heads, d]
 * with a token stride of ld_token floats and heads packed at stride d; q has the same shape packed, s is
 * [tokens, heads].  All arithmetic is IEEE fp32 (this file is built without contraction or fast-math).
 * ---------------------------------------------------------------------------------------------------- */
void orc_quant_i16(const float* x, int64_t tokens, int64_t heads, int64_t d, int64_t ld_token, int16_t* q,
                   float* s) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < tokens; ++t)
    for (int64_t h = 0; h < heads; ++h) {
      const float* row = x + t * ld_token + h * d;
      int16_t* qrow = q + (t * heads + h) * d;
      float amax = 0.0f;
      for (int64_t i = 0; i < d; ++i) {
        const float a = fabsf(row[i]);
        if (a > amax) amax = a;
      }
      const float sc = amax / 32767.0f;
      s[t * heads + h] = sc;
      if (sc == 0.0f) { /* an all-zero row (or one whose scale underflows) codes every element as 0 */
        for (int64_t i = 0; i < d; ++i) qrow[i] = 0;
        continue;
      }
      for (int64_t i = 0; i < d; ++i) {
        float r = rintf(row[i] / sc);
        if (r > 32767.0f) r = 32767.0f;
        if (r < -32767.0f) r = -32767.0f;
        qrow[i] = (int16_t)r;
      }
    }
}

/* ------------------------------------------------------------------------------------------------------
 * The quantity the compensated GEMM approximates: C = A * B in FP64, with A [M, K] (row stride lda) and
 * B given as its transpose Bt [N, K] (row stride ldb), both already widened exactly to double.  This is
 * the definition the method reaches up to rounding ([TS 2B Solution]: "high-precision matrix
 * multiplications").  k runs in increasing order.
 * ---------------------------------------------------------------------------------------------------- */
void orc_gemm_f64(int64_t M, int64_t N, int64_t K, const double* A, int64_t lda, const double* Bt,
                  int64_t ldb, double* C, int64_t ldc) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < M; ++i)
    for (int64_t j = 0; j < N; ++j) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += A[i * lda + k] * Bt[j * ldb + k];
      C[i * ldc + j] = acc;
    }
}

/* the same, for a list of (i, j) output positions: what a full-size check can afford */
void orc_gemm_f64_points(int64_t K, const double* A, int64_t lda, const double* Bt, int64_t ldb,
                         int64_t npts, const int64_t* ii, const int64_t* jj, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < npts; ++p) {
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) acc += A[ii[p] * lda + k] * Bt[jj[p] * ldb + k];
    out[p] = acc;
  }
}

/* ------------------------------------------------------------------------------------------------------
 * Emulation level of the compensated GEMM: the exact sum, in FP64, of the same 16-bit products the
 * method forms ([TS 2B Mechanism], reading R-prod), undone by the row/column prescales:
 *   C_e[i,j] = 2^-(ea_i + eb_j) * sum_k (ah*bh + ah*bl + al*bh)
 * and the magnitude sum  G[i,j] = 2^-(ea_i + eb_j) * sum_k (|ah*bh| + |ah*bl| + |al*bh|),
 * the factor in the rigorous bound of an FP32 accumulation of those products.  Absent lo parts are 0.
 * Parts are 16-bit patterns of `part` (F16 or BF16); exps may be NULL (no prescale).
 * ---------------------------------------------------------------------------------------------------- */
void orc_gemm_emul(int64_t M, int64_t N, int64_t K, const uint16_t* ah, const uint16_t* al,
                   const int32_t* ea, int64_t lda, const uint16_t* bh, const uint16_t* bl,
                   const int32_t* eb, int64_t ldb, int part, double* C, double* G, int64_t ldc) {
  /* the values of the parts, decoded once (an absent lo part is 0) */
  double* xa = (double*)malloc(sizeof(double) * (size_t)(M * K > 0 ? 2 * M * K : 1));
  double* ya = (double*)malloc(sizeof(double) * (size_t)(N * K > 0 ? 2 * N * K : 1));
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M; ++i)
    for (int64_t k = 0; k < K; ++k) {
      xa[2 * (i * K + k)] = part_value(ah[i * lda + k], part);
      xa[2 * (i * K + k) + 1] = al ? part_value(al[i * lda + k], part) : 0.0;
    }
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < N; ++j)
    for (int64_t k = 0; k < K; ++k) {
      ya[2 * (j * K + k)] = part_value(bh[j * ldb + k], part);
      ya[2 * (j * K + k) + 1] = bl ? part_value(bl[j * ldb + k], part) : 0.0;
    }
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < M; ++i)
    for (int64_t j = 0; j < N; ++j) {
      const double* x = xa + 2 * i * K;
      const double* y = ya + 2 * j * K;
      double acc = 0.0, mag = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const double xh = x[2 * k], xl = x[2 * k + 1], yh = y[2 * k], yl = y[2 * k + 1];
        acc += xh * yh + xh * yl + xl * yh;
        mag += fabs(xh * yh) + fabs(xh * yl) + fabs(xl * yh);
      }
      const int e = (ea ? ea[i] : 0) + (eb ? eb[j] : 0);
      C[i * ldc + j] = ldexp(acc, -e);
      if (G) G[i * ldc + j] = ldexp(mag, -e);
    }
  free(xa);
  free(ya);
}

/* ------------------------------------------------------------------------------------------------------
 * Attention in FP64 on real-valued Q, K, V (the definition), for a list of query rows.
 *   q  : [B, Lq, Hq, D] element strides qs[3] (batch, token, head), d contiguous
 *   k,v: [B, Lkv, Hkv, D] strides ks[3]
 *   row list: (b, i, h) triples; out[r*D + d] receives O for row r.
 * S_ij = scale * sum_d q_i,d k_j,d ; causal keeps j <= i + (Lkv - Lq) (reading R-attn);
 * P = softmax over the kept j with the row maximum subtracted; O_i = sum_j P_ij v_j.
 * ---------------------------------------------------------------------------------------------------- */
void orc_attn_f64(int64_t Lq, int64_t Lkv, int64_t Hq, int64_t Hkv, int64_t D, const double* q,
                  const int64_t* qs, const double* k, const double* v, const int64_t* ks, int causal,
                  double scale, int64_t nrows, const int64_t* rb, const int64_t* ri, const int64_t* rh,
                  double* out) {
  const int64_t group = Hq / Hkv;
#pragma omp parallel
  {
    double* sc = (double*)malloc(sizeof(double) * (size_t)(Lkv > 0 ? Lkv : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
      const int64_t b = rb[r], i = ri[r], h = rh[r], hk = h / group;
      const double* qi = q + b * qs[0] + i * qs[1] + h * qs[2];
      int64_t jmax = Lkv - 1;
      if (causal) jmax = i + (Lkv - Lq);
      if (jmax > Lkv - 1) jmax = Lkv - 1;
      double m = -INFINITY;
      for (int64_t j = 0; j <= jmax; ++j) {
        const double* kj = k + b * ks[0] + j * ks[1] + hk * ks[2];
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += qi[d] * kj[d];
        sc[j] = scale * dot;
        if (sc[j] > m) m = sc[j];
      }
      double l = 0.0;
      for (int64_t j = 0; j <= jmax; ++j) {
        sc[j] = exp(sc[j] - m);
        l += sc[j];
      }
      double* o = out + r * D;
      for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
      for (int64_t j = 0; j <= jmax; ++j) {
        const double* vj = v + b * ks[0] + j * ks[1] + hk * ks[2];
        for (int64_t d = 0; d < D; ++d) o[d] += sc[j] * vj[d];
      }
      for (int64_t d = 0; d < D; ++d) o[d] = (jmax >= 0) ? o[d] / l : 0.0;
    }
    free(sc);
  }
}

/* Dequantise an INT16 tensor with per-(b, token, head) fp32 scales into doubles: x = s * q, exact in
   double (24-bit scale times a 16-bit integer).  q strides qs[3], scale strides ss[3], both in elements;
   the output is packed [B, L, H, D]. */
void orc_dequant_i16(int64_t B, int64_t L, int64_t H, int64_t D, const int16_t* q, const int64_t* qs,
                     const float* s, const int64_t* ss, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < B; ++b)
    for (int64_t t = 0; t < L; ++t)
      for (int64_t h = 0; h < H; ++h) {
        const double sc = (double)s[b * ss[0] + t * ss[1] + h * ss[2]];
        const int16_t* src = q + b * qs[0] + t * qs[1] + h * qs[2];
        double* dst = out + ((b * L + t) * H + h) * D;
        for (int64_t d = 0; d < D; ++d) dst[d] = sc * (double)src[d];
      }
}
