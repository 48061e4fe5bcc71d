/*
 * aq_oracle.c -- CPU oracle for group-wise affine weight-only
 * quantization and the matmul that consumes the packed form.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is used by the test-suite, by the
 * smoke check and by the benchmark's CPU-baseline leg.  Nothing on the
 * product path links, loads or calls it; it shares no code, header, table
 * or helper with the HIP library.  It is deliberately plain and slow:
 * every rounding decision is taken by exact comparisons in binary64, and
 * every result follows the definitions below step by step.
 *
 * Sources (web pages; cited by title and section):
 *  [MLXQ]  "Quantization" (metalworking, MLX notes): opening paragraph
 *          (groups of 32/64/128 along a row, one scale + one bias +
 *          2-8 bit codes), "Mechanics" (w ~= codes*scale + bias per group).
 *  [QMLX]  "Quantizing a Model for MLX", section "What MLX quantization
 *          stores" (contiguous groups, scale and offset chosen per group,
 *          integers packed several to a machine word, fp16 scale and fp16
 *          bias, 4.5 bits/weight at G=64, 4 bits).
 *  [GPTQ]  "mlx-gptq", section "How it works" (the round-to-nearest grid
 *          spans each group's min-max range).
 *  [T10]   "Tutorial 10: Quantization", section 3 "Packing Multiple
 *          Weights into One Word" (codes extracted with right shifts by
 *          multiples of `bits` and a (1<<bits)-1 mask, i.e. least
 *          significant bits first; dequantize = values*scales + biases in
 *          float32, then cast), section 4 (container shapes
 *          [out_features, in_features/group_size]), section 5 "Approach 1:
 *          Dequantize Then Multiply" (y = x @ W^T on the dequantized W),
 *          section 6 "Quantized Embeddings" (rows selected by token id,
 *          then dequantized).
 *
 * Readings taken where the pages are silent (each is repeated in the
 * design notes):
 *  R1  bias = the group minimum rounded DOWN to fp16, so the bias never
 *      exceeds a group member; scale = the smallest non-negative fp16 for
 *      which the top grid point bias + (2^b-1)*scale reaches the group
 *      maximum (i.e. the quotient (max-bias)/(2^b-1) rounded UP to fp16).
 *  R2  code = index of the nearest grid point bias + q*scale,
 *      q in [0, 2^b-1]; an exact tie goes to the even q.  scale == 0
 *      (constant group) gives q = 0.  A group minimum of -0 is taken as +0.
 *  R3  packing is one least-significant-bit-first bitstream per row: code
 *      k of a row occupies bits [k*b, k*b+b) of the row, bit i of the
 *      stream being bit (i mod 32) of little-endian uint32 word i/32.  For
 *      b in {2,4,8} this is exactly the shift/mask decoder of [T10] s.3;
 *      for b=3 eight codes fill three bytes.
 *  R4  dequantize follows [T10] s.3 operation order: q*scale + bias
 *      evaluated in binary32 (q*scale is exact, so only the add rounds),
 *      then a round-to-nearest-even cast to the output type.
 *  R5  matmul oracle: y[m,n] = sum_k x[m,k] * w^[n,k] with w^ the exact
 *      value q*scale + bias, products and sums in binary64; the companion
 *      A[m,n] = sum_k |x[m,k] * w^[n,k]| scales the tolerance.
 *  R6  gather (MoE): y[t,j,:] = x[t,:] @ W_{ids[t,j]}^T, one output per
 *      (token, slot), no routing-weight combine.
 *  R13 embedding ([T10] s.6): out[t,:] is row ids[t] dequantized as in R4;
 *      an id outside the table gives a zero row.
 *  R14 range search ([GPTQ] "How it works", the --mse option: a group may
 *      be quantized over a range narrower than its min-max span, trading
 *      error on its outermost members for a finer step on the others).
 *      The pages give no grid and no error measure; taken here: candidate
 *      i = 0..steps-1 keeps the fraction p_i = (100 - i)/100 of the width,
 *      centred, i.e. both ends move inwards by the same amount
 *        d_i = (max - min) * (i / 200)            (binary64, left to right)
 *        range_i = [min + d_i, max - d_i]         (binary64)
 *      so every candidate lies inside [min, max] whatever the signs of the
 *      members (candidate 0 is [min, max] itself).  Bias and scale come
 *      from range_i by R1, codes by R2 against them (members outside the
 *      range clip to 0 or 2^b-1), error = sum over the group, in member
 *      order, of (w - (q*s + b))^2 in binary64.  The least error wins; an
 *      equal error keeps the earlier (wider) candidate.  steps = 1 is
 *      R1/R2.
 *  R15 integer zero point ([GPTQ] "On NVIDIA: the same recipe in AWQ
 *      format", --zero-point int: every group's offset is a whole number of
 *      steps, so the grid converts to a layout with integer zero points
 *      without loss).  The zero point z is an integer in [0, 2^b-1] (it is
 *      stored as a b-bit unsigned integer in such a layout), so every grid
 *      -z*s + q*s, q = 0..2^b-1, contains 0.  Taken here: the scale is the
 *      smallest fp16 s >= 0 for which some integer z in [0, 2^b-1] gives
 *      -z*s <= min, (2^b-1-z)*s >= max and -z*s exactly an fp16 value;
 *      z is the smallest such integer for that s; bias = -z*s (exact, +0
 *      when z = 0); codes by R2 against that bias and scale.  Hence every
 *      member lies on the grid's span and |w - w^| <= s/2, and w^ =
 *      (q - z)*s exactly.
 *  R16 mxfp4 ([MLXQ] newer-modes paragraph and [QMLX] "Modes, bits and
 *      mixed recipes": a block-scaled float mode with groups of 32 and
 *      4-bit codes that keeps one exponent per group instead of a scale and
 *      a bias).  The pages give no bit layout; taken here, the microscaling
 *      (MX) definition of that name: a code is an E2M1 float -- bit 3 the
 *      sign, bits 2..1 an exponent e with bias 1, bit 0 a mantissa m; value
 *      (1 + m/2) * 2^(e-1) for e > 0 and m/2 for e = 0, so the magnitudes
 *      of codes 0..7 are 0, 0.5, 1, 1.5, 2, 3, 4, 6 -- and the group's
 *      scale is 2^X, stored as the byte X + 127.  X = floor(log2(max|w|))
 *      - 2 (2 = the exponent of E2M1's largest value), clamped to
 *      [-127, 127], and -127 for an all-zero group.  A member's code is
 *      its sign bit with the magnitude code nearest to |w| / 2^X (ties to
 *      the even mantissa; above 6 that is 6); codes are packed as in R3
 *      with b = 4.  Dequantized value: code value * 2^X.
 *  R17 mxfp8 (the same passages: a block-scaled float mode with groups of
 *      32 and 8-bit codes).  Taken, again from the microscaling definition:
 *      a code is an E4M3 float -- bit 7 the sign, bits 6..3 an exponent e
 *      with bias 7, bits 2..0 a mantissa m; value (1 + m/8) * 2^(e-7) for
 *      e > 0 and (m/8) * 2^-6 for e = 0; the pattern e = 15, m = 7 is not a
 *      number, so the largest finite magnitude is 448 = 1.75 * 2^8.  The
 *      group scale is 2^X, byte X + 127, with X = floor(log2(max|w|)) - 8
 *      (8 = the exponent of 448), clamped to [-127, 127], -127 for an
 *      all-zero group.  A member's code is its sign bit with the finite
 *      magnitude code nearest to |w| / 2^X (ties to the even code, i.e. the
 *      even mantissa; above 448 that is 448); codes are bytes in row order
 *      (R3 with b = 8).  Dequantized value: code value * 2^X.
 *  R18 nvfp4 ([ET] configuration table and CLI options: NVIDIA's FP4
 *      format for weights, group size 16; the same MLX passages: groups of
 *      16, 4-bit codes).  Taken from the
 *      NVFP4 format of that name: codes are E2M1 as in R16, packed as in
 *      R16; each group of 16 stores one scale s, an E4M3 value (as in R17,
 *      sign bit 0) written as its byte; the whole matrix shares a second
 *      scale, here a power of two 2^T with T an integer in [-100, 100]
 *      chosen by the caller (0: no second scale), which lets the group
 *      scales use E4M3's normal range whatever the weights' magnitude.
 *      s = the E4M3 magnitude nearest to max|w| / (6 * 2^T) (6 = the
 *      largest E2M1 value; ties to the even code, above 448 that is 448),
 *      and a member's code is its sign bit with the magnitude code nearest
 *      to |w| / (s * 2^T) (ties to the even mantissa, above 6 that is 6),
 *      or magnitude 0 when s = 0.  Dequantized value: code value * s * 2^T.
 *      Exactness: an E4M3 value has at most 4 significant bits and an E2M1
 *      one at most 2, so every midpoint of either grid times 6, times a
 *      power of two or times s has at most 8 significant bits; the
 *      nearest-value decisions below compare a weight with such products,
 *      which binary64 holds exactly.
 *
 * Exactness of the binary64 comparisons used below.  Every finite fp16
 * value is an integer multiple of 2^-24 of magnitude < 2^16; q*s with
 * q <= 255 is a multiple of 2^-24 below 2^24; (q+1/2)*s is a multiple of
 * 2^-25 below 2^25.  Hence b + q*s and b + (q+1/2)*s are multiples of
 * 2^-25 below 2^26 and fit in 51 significant bits: binary64 holds them
 * exactly, and comparing them with a binary32 weight (also exact in
 * binary64) is an exact comparison of real numbers.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_ERR_ARG (-1)
#define OR_ERR_UNSUPPORTED (-2)
#define OR_ERR_RANGE (-5)
#define OR_ERR_INDEX (-6)

/* output type tags (same meaning as the library's, defined independently) */
#define OR_F32 0
#define OR_F16 1
#define OR_BF16 2

#define HALF_MAX_FINITE_MAG 0x7BFFu /* 65504 */

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* threads of the parallel loops from now on (the single-thread timing) */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ---------------------------------------------------------------------
 * IEEE-754 binary16 and bfloat16, from their definitions.
 * ------------------------------------------------------------------- */

/* value of a binary16 bit pattern: 1 sign, 5 exponent (bias 15), 10
 * fraction bits; exponent 0 = subnormal (fraction * 2^-24). */
double oracle_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int f = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25);
  return sign ? -v : v;
}

/* value of a bfloat16 bit pattern: the upper half of a binary32. */
double oracle_bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Non-negative binary16 magnitudes 0x0000..0x7BFF are ordered like their
 * patterns, so the searches below are bisections over patterns. */

/* largest finite fp16 <= x.  Returns OR_ERR_RANGE if x < -65504. */
static int half_round_down(double x, uint16_t *out) {
  if (!(x == x)) return OR_ERR_RANGE;
  if (x >= 0.0) { /* -0.0 lands here too and becomes +0 */
    /* largest p in [0, 0x7BFF] with value(p) <= x */
    uint32_t lo = 0, hi = HALF_MAX_FINITE_MAG;
    while (lo < hi) {
      uint32_t mid = (lo + hi + 1) / 2;
      if (oracle_half_to_double((uint16_t)mid) <= x) lo = mid; else hi = mid - 1;
    }
    *out = (uint16_t)lo;
    return OR_OK;
  }
  /* x < 0: smallest magnitude p with value(p) >= -x, returned negated */
  double mag = -x;
  if (mag > oracle_half_to_double(HALF_MAX_FINITE_MAG)) return OR_ERR_RANGE;
  uint32_t lo = 1, hi = HALF_MAX_FINITE_MAG;
  while (lo < hi) {
    uint32_t mid = (lo + hi) / 2;
    if (oracle_half_to_double((uint16_t)mid) >= mag) hi = mid; else lo = mid + 1;
  }
  *out = (uint16_t)(0x8000u | lo);
  return OR_OK;
}

/* Round-to-nearest-even of a finite double to binary16 (overflow to inf
 * at and above 65520, the midpoint past the largest finite value). */
uint16_t oracle_double_to_half_rne(double x) {
  if (isnan(x)) return (uint16_t)(signbit(x) ? 0xFE00u : 0x7E00u); /* a quiet NaN stays NaN */
  uint16_t sign = (x < 0 || (x == 0 && signbit(x))) ? 0x8000u : 0;
  double mag = fabs(x);
  if (mag >= 65520.0) return sign | 0x7C00u;
  /* p = largest pattern with value(p) <= mag */
  uint32_t lo = 0, hi = HALF_MAX_FINITE_MAG;
  while (lo < hi) {
    uint32_t mid = (lo + hi + 1) / 2;
    if (oracle_half_to_double((uint16_t)mid) <= mag) lo = mid; else hi = mid - 1;
  }
  double below = oracle_half_to_double((uint16_t)lo);
  if (below == mag || lo == 0x7C00u) return sign | (uint16_t)lo;
  double above = (lo + 1 == 0x7C00u) ? 65536.0 : oracle_half_to_double((uint16_t)(lo + 1));
  double d_lo = mag - below, d_hi = above - mag; /* exact: all on a fine grid */
  uint32_t p;
  if (d_lo < d_hi) p = lo;
  else if (d_hi < d_lo) p = lo + 1;
  else p = (lo & 1u) ? lo + 1 : lo; /* tie: even pattern */
  return sign | (uint16_t)p;
}

/* Round-to-nearest-even of a binary32 value to bfloat16.  The two
 * candidates are the binary32 values with the low 16 bits cleared (toward
 * zero) and the next bfloat16 magnitude; past the largest finite bfloat16
 * the next magnitude is 2^128 (infinity), as IEEE overflow rounding has it. */
uint16_t oracle_float_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7F800000u) == 0x7F800000u) /* inf stays inf, nan stays a quiet nan */
    return (uint16_t)((u >> 16) | ((u & 0x007FFFFFu) ? 0x40u : 0));
  uint32_t down = u & 0xFFFF0000u;
  uint32_t up = down + 0x10000u;
  float fd;
  memcpy(&fd, &down, sizeof fd);
  double vd = fabs((double)fd), vu;
  if ((up & 0x7F800000u) == 0x7F800000u) {
    vu = ldexp(1.0, 128);
  } else {
    float fu;
    memcpy(&fu, &up, sizeof fu);
    vu = fabs((double)fu);
  }
  double mag = fabs((double)f);
  double dd = mag - vd, du = vu - mag; /* exact in binary64 */
  if (dd < du) return (uint16_t)(down >> 16);
  if (du < dd) return (uint16_t)(up >> 16);
  return (uint16_t)(((down >> 16) & 1u) ? (up >> 16) : (down >> 16));
}

/* ---------------------------------------------------------------------
 * Format arithmetic ([QMLX] "What MLX quantization stores"): per group of
 * G weights, G*b bits of codes plus a 16-bit scale and a 16-bit bias.
 * ------------------------------------------------------------------- */
int64_t oracle_packed_words_per_row(int64_t K, int bits) { return K * bits / 32; }

int64_t oracle_qweight_bytes(int64_t N, int64_t K, int group_size, int bits) {
  return N * K * bits / 8 + N * (K / group_size) * 4;
}

static int check_shape(int64_t N, int64_t K, int G, int bits) {
  if (N < 0 || K < 0) return OR_ERR_ARG;
  if (G != 32 && G != 64 && G != 128) return OR_ERR_ARG;
  if (bits < 2 || bits > 8) return OR_ERR_ARG;
  if (K % G) return OR_ERR_ARG;
  return OR_OK;
}

/* ---------------------------------------------------------------------
 * Bitstream packing (reading R3), one bit at a time.
 * ------------------------------------------------------------------- */
static void put_code(uint32_t *row, int64_t k, int bits, uint32_t q) {
  for (int i = 0; i < bits; ++i) {
    int64_t pos = k * bits + i;
    if ((q >> i) & 1u) row[pos / 32] |= (1u << (pos % 32));
  }
}

static uint32_t get_code(const uint32_t *row, int64_t k, int bits) {
  uint32_t q = 0;
  for (int i = 0; i < bits; ++i) {
    int64_t pos = k * bits + i;
    q |= ((row[pos / 32] >> (pos % 32)) & 1u) << i;
  }
  return q;
}

/* pack an [N, K] array of codes (one per uint8) into [N, K*b/32] words */
int oracle_pack(const uint8_t *q, int64_t N, int64_t K, int bits, uint32_t *codes) {
  if (bits < 2 || bits > 8 || (K * bits) % 32) return OR_ERR_ARG;
  int64_t wpr = K * bits / 32;
  memset(codes, 0, (size_t)(N * wpr) * sizeof(uint32_t));
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      if (q[n * K + k] >> bits) return OR_ERR_RANGE;
      put_code(codes + n * wpr, k, bits, q[n * K + k]);
    }
  return OR_OK;
}

int oracle_unpack(const uint32_t *codes, int64_t N, int64_t K, int bits, uint8_t *q) {
  if (bits < 2 || bits > 8 || (K * bits) % 32) return OR_ERR_ARG;
  int64_t wpr = K * bits / 32;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) q[n * K + k] = (uint8_t)get_code(codes + n * wpr, k, bits);
  return OR_OK;
}

/* ---------------------------------------------------------------------
 * Quantize one group (readings R1, R2).
 * ------------------------------------------------------------------- */

/* scale: smallest fp16 s >= 0 with bias + L*s >= hi (exact test). */
static int group_scale(double bias, double hi, int L, uint16_t *s_out) {
  if (bias >= hi) { *s_out = 0; return OR_OK; }
  if (bias + L * oracle_half_to_double(HALF_MAX_FINITE_MAG) < hi) return OR_ERR_RANGE;
  uint32_t lo = 0, up = HALF_MAX_FINITE_MAG;
  while (lo < up) {
    uint32_t mid = (lo + up) / 2;
    if (bias + L * oracle_half_to_double((uint16_t)mid) >= hi) up = mid; else lo = mid + 1;
  }
  *s_out = (uint16_t)lo;
  return OR_OK;
}

/* code: nearest grid index.  The grid points b + q*s increase with q, so
 * the nearest one is the number of midpoints b + (j+1/2)*s (j = 0..L-1)
 * lying strictly below w; found by bisection.  If w sits exactly on a
 * midpoint between j and j+1, the even one of the two is taken. */
static uint32_t group_code(double w, double b, double s, int L) {
  if (s == 0.0) return 0;
  int lo = 0, hi = L; /* answer = count of j in [0,L) with mid_j < w */
  while (lo < hi) {
    int j = (lo + hi) / 2;
    double mid = b + (j + 0.5) * s;
    if (mid < w) lo = j + 1; else hi = j;
  }
  uint32_t q = (uint32_t)lo;
  if (q < (uint32_t)L && b + (q + 0.5) * s == w && (q & 1u)) q += 1;
  return q;
}

/* Quantize W fp32 [N, K] row-major into codes [N, K*b/32] uint32, scales
 * and biases [N, K/G] fp16 bits.  Returns OR_ERR_RANGE for a non-finite
 * weight or a group whose bias/scale leave the fp16 range. */
int oracle_quantize(const float *w, int64_t N, int64_t K, int G, int bits,
                    uint32_t *codes, uint16_t *scales, uint16_t *biases) {
  int st = check_shape(N, K, G, bits);
  if (st) return st;
  const int L = (1 << bits) - 1;
  const int64_t wpr = K * bits / 32, ng = K / G;
  int err = OR_OK;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    uint32_t *row = codes + n * wpr;
    memset(row, 0, (size_t)wpr * sizeof(uint32_t));
    for (int64_t g = 0; g < ng; ++g) {
      const float *grp = w + n * K + g * G;
      double lo = INFINITY, hi = -INFINITY;
      int bad = 0;
      for (int i = 0; i < G; ++i) {
        double v = (double)grp[i];
        if (!isfinite(v)) bad = 1;
        if (v < lo) lo = v;
        if (v > hi) hi = v;
      }
      uint16_t b16 = 0, s16 = 0;
      if (!bad && half_round_down(lo, &b16) != OR_OK) bad = 1;
      double b = oracle_half_to_double(b16);
      if (!bad && group_scale(b, hi, L, &s16) != OR_OK) bad = 1;
      if (bad) {
#pragma omp critical
        err = OR_ERR_RANGE;
        continue;
      }
      double s = oracle_half_to_double(s16);
      scales[n * ng + g] = s16;
      biases[n * ng + g] = b16;
      for (int i = 0; i < G; ++i)
        put_code(row, g * G + i, bits, group_code((double)grp[i], b, s, L));
    }
  }
  return err;
}

/* Range search (R14).  Same outputs as oracle_quantize, plus, when not
 * NULL: chosen [N, K/G] (index of the winning candidate) and errs
 * [N, K/G, steps] (every candidate's error).  only >= 0 evaluates that one
 * candidate alone (for checking a result that picked it).  The range
 * check of oracle_quantize applies to the full range (candidate 0); the
 * narrower candidates then stay in range. */
int oracle_quantize_mse(const float *w, int64_t N, int64_t K, int G, int bits, int steps, int only,
                        uint32_t *codes, uint16_t *scales, uint16_t *biases, int32_t *chosen,
                        double *errs) {
  int st = check_shape(N, K, G, bits);
  if (st) return st;
  if (steps < 1 || steps > 50 || only >= steps) return OR_ERR_ARG;
  const int L = (1 << bits) - 1;
  const int64_t wpr = K * bits / 32, ng = K / G;
  int err = OR_OK;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    uint32_t *row = codes + n * wpr;
    memset(row, 0, (size_t)wpr * sizeof(uint32_t));
    for (int64_t g = 0; g < ng; ++g) {
      const float *grp = w + n * K + g * G;
      double lo = INFINITY, hi = -INFINITY;
      int bad = 0;
      for (int i = 0; i < G; ++i) {
        double v = (double)grp[i];
        if (!isfinite(v)) bad = 1;
        if (v < lo) lo = v;
        if (v > hi) hi = v;
      }
      uint16_t b0 = 0, s0 = 0;
      if (!bad && half_round_down(lo, &b0) != OR_OK) bad = 1;
      if (!bad && group_scale(oracle_half_to_double(b0), hi, L, &s0) != OR_OK) bad = 1;
      if (bad) {
#pragma omp critical
        err = OR_ERR_RANGE;
        continue;
      }
      double best = INFINITY;
      int best_i = -1;
      uint16_t best_b = 0, best_s = 0;
      const double width = hi - lo;
      for (int i = (only >= 0 ? only : 0); i < (only >= 0 ? only + 1 : steps); ++i) {
        /* both ends move inwards by d; the range keeps (100 - i)% of its width */
        const double d = width * ((double)i / 200.0);
        const double clo = lo + d, chi = hi - d;
        uint16_t b16 = 0, s16 = 0;
        half_round_down(clo, &b16);
        const double b = oracle_half_to_double(b16);
        group_scale(b, chi, L, &s16);
        const double s = oracle_half_to_double(s16);
        double e = 0.0;
        for (int k = 0; k < G; ++k) {
          const double v = (double)grp[k];
          const double d = v - (b + group_code(v, b, s, L) * s);
          e += d * d;
        }
        if (errs) errs[(n * ng + g) * steps + i] = e;
        if (e < best) { best = e; best_i = i; best_b = b16; best_s = s16; }
      }
      const double b = oracle_half_to_double(best_b), s = oracle_half_to_double(best_s);
      scales[n * ng + g] = best_s;
      biases[n * ng + g] = best_b;
      if (chosen) chosen[n * ng + g] = best_i;
      for (int i = 0; i < G; ++i)
        put_code(row, g * G + i, bits, group_code((double)grp[i], b, s, L));
    }
  }
  return err;
}

/* Integer zero point (R15).  For one group with members in [lo, hi]:
 * the smallest fp16 scale s admitting an integer z in [0, L] with
 * -z*s <= lo, (L - z)*s >= hi and -z*s exactly an fp16 value, and the
 * smallest such z.  Scales are tried in increasing order from the smallest
 * one whose L steps span [min(lo, 0), max(hi, 0)] (no smaller scale can
 * cover a grid that contains 0); for each, every z in [0, L] is checked with
 * exact binary64 comparisons (z*s has at most 19 significant bits).
 * Returns OR_ERR_RANGE when no fp16 scale admits one. */
static int group_zero_point(double lo, double hi, int L, uint16_t *s_out, int *z_out) {
  const double lo0 = lo < 0.0 ? lo : 0.0, hi0 = hi > 0.0 ? hi : 0.0;
  uint16_t s0 = 0;
  if (group_scale(lo0, hi0, L, &s0) != OR_OK) return OR_ERR_RANGE;
  for (uint32_t p = s0; p <= HALF_MAX_FINITE_MAG; ++p) {
    const double sv = oracle_half_to_double((uint16_t)p);
    for (int z = 0; z <= L; ++z) {
      const double bottom = -(double)z * sv, top = (double)(L - z) * sv;
      if (bottom > lo || top < hi) continue;
      if (oracle_half_to_double(oracle_double_to_half_rne(bottom)) != bottom) continue;
      *s_out = (uint16_t)p;
      *z_out = z;
      return OR_OK;
    }
  }
  return OR_ERR_RANGE;
}

/* Quantize with integer zero points (R15): same outputs as oracle_quantize
 * plus zeros [N, K/G] (the integer z of each group; may be NULL). */
int oracle_quantize_zp(const float *w, int64_t N, int64_t K, int G, int bits, uint32_t *codes,
                       uint16_t *scales, uint16_t *biases, uint8_t *zeros) {
  int st = check_shape(N, K, G, bits);
  if (st) return st;
  const int L = (1 << bits) - 1;
  const int64_t wpr = K * bits / 32, ng = K / G;
  int err = OR_OK;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    uint32_t *row = codes + n * wpr;
    memset(row, 0, (size_t)wpr * sizeof(uint32_t));
    for (int64_t g = 0; g < ng; ++g) {
      const float *grp = w + n * K + g * G;
      double lo = INFINITY, hi = -INFINITY;
      int bad = 0;
      for (int i = 0; i < G; ++i) {
        double v = (double)grp[i];
        if (!isfinite(v)) bad = 1;
        if (v < lo) lo = v;
        if (v > hi) hi = v;
      }
      uint16_t s16 = 0;
      int z = 0;
      if (bad || group_zero_point(lo, hi, L, &s16, &z) != OR_OK) {
#pragma omp critical
        err = OR_ERR_RANGE;
        continue;
      }
      const double s = oracle_half_to_double(s16);
      const double b = -(double)z * s;
      const uint16_t b16 = z == 0 ? (uint16_t)0 : oracle_double_to_half_rne(b);
      scales[n * ng + g] = s16;
      biases[n * ng + g] = b16;
      if (zeros) zeros[n * ng + g] = (uint8_t)z;
      for (int i = 0; i < G; ++i)
        put_code(row, g * G + i, bits, group_code((double)grp[i], b, s, L));
    }
  }
  return err;
}

/* ---------------------------------------------------------------------
 * Dequantize ([MLXQ] "Mechanics", [T10] s.3 and s.7; reading R4).
 * ------------------------------------------------------------------- */

/* exact dequantized values w^ = q*s + b as binary64, [N, K] */
int oracle_dequantize_exact(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                            int64_t N, int64_t K, int G, int bits, double *out) {
  int st = check_shape(N, K, G, bits);
  if (st) return st;
  const int64_t wpr = K * bits / 32, ng = K / G;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      double s = oracle_half_to_double(scales[n * ng + k / G]);
      double b = oracle_half_to_double(biases[n * ng + k / G]);
      out[n * K + k] = (double)get_code(codes + n * wpr, k, bits) * s + b;
    }
  return OR_OK;
}

/* dequantize to fp32 / fp16 / bf16 in the pages' order: binary32 result
 * of q*s + b, then a round-to-nearest-even cast. */
/* One row: out_row[k] = q*s + b in binary32 (R4), then cast to out_dtype. */
static void dequantize_row(const uint32_t *row, const uint16_t *srow, const uint16_t *brow,
                           int64_t K, int G, int bits, int out_dtype, void *out, int64_t off) {
  for (int64_t k = 0; k < K; ++k) {
    double s = oracle_half_to_double(srow[k / G]);
    double b = oracle_half_to_double(brow[k / G]);
    /* q*s is exact in binary32; the binary32 sum rounds once, which is
     * the binary64 exact value rounded to binary32 */
    float v32 = (float)((double)get_code(row, k, bits) * s + b);
    if (out_dtype == OR_F32)
      ((float *)out)[off + k] = v32;
    else if (out_dtype == OR_F16)
      ((uint16_t *)out)[off + k] = oracle_double_to_half_rne((double)v32);
    else
      ((uint16_t *)out)[off + k] = oracle_float_to_bf16_rne(v32);
  }
}

int oracle_dequantize(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                      int64_t N, int64_t K, int G, int bits, int out_dtype, void *out) {
  int st = check_shape(N, K, G, bits);
  if (st) return st;
  if (out_dtype != OR_F32 && out_dtype != OR_F16 && out_dtype != OR_BF16) return OR_ERR_ARG;
  const int64_t wpr = K * bits / 32, ng = K / G;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    dequantize_row(codes + n * wpr, scales + n * ng, biases + n * ng, K, G, bits, out_dtype, out,
                   n * K);
  return OR_OK;
}

/* ---------------------------------------------------------------------
 * Quantized embedding ([T10] s.6 "Quantized Embeddings"): a lookup by
 * token id selects the packed row, its scales and its biases, and that row
 * is dequantized as above.  out[t, :] = dequantize(row ids[t]).
 * Reading R13: an id outside [0, V) selects no row and gives a zero row.
 * ------------------------------------------------------------------- */
int oracle_embedding(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                     int64_t V, int64_t K, int G, int bits, const int32_t *ids, int64_t T,
                     int out_dtype, void *out) {
  int st = check_shape(V, K, G, bits);
  if (st) return st;
  if (T < 0) return OR_ERR_ARG;
  if (out_dtype != OR_F32 && out_dtype != OR_F16 && out_dtype != OR_BF16) return OR_ERR_ARG;
  const int64_t wpr = K * bits / 32, ng = K / G;
  const size_t esz = out_dtype == OR_F32 ? 4 : 2;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    const int64_t id = ids[t];
    if (id < 0 || id >= V)
      memset((char *)out + (size_t)(t * K) * esz, 0, (size_t)K * esz);
    else
      dequantize_row(codes + id * wpr, scales + id * ng, biases + id * ng, K, G, bits, out_dtype,
                     out, t * K);
  }
  return OR_OK;
}

/* ---------------------------------------------------------------------
 * Matmul oracle ([T10] s.5 Approach 1: dequantize then multiply;
 * reading R5).  x holds the exact activation values as binary64.
 * Only the output columns listed in `cols` (nc of them) are computed, so
 * large shapes can be checked on a sample; y and A are [M, nc].
 * ------------------------------------------------------------------- */
int oracle_matmul_cols(const double *x, int64_t M, const uint32_t *codes, const uint16_t *scales,
                       const uint16_t *biases, int64_t N, int64_t K, int G, int bits,
                       const int64_t *cols, int64_t nc, double *y, double *A) {
  int st = check_shape(N, K, G, bits);
  if (st) return st;
  for (int64_t c = 0; c < nc; ++c)
    if (cols[c] < 0 || cols[c] >= N) return OR_ERR_INDEX;
  const int64_t wpr = K * bits / 32, ng = K / G;
  int err = OR_OK;
#pragma omp parallel
  {
    double *wrow = (double *)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
    if (!wrow) {
#pragma omp critical
      err = OR_ERR_ARG;
    } else {
#pragma omp for schedule(static)
      for (int64_t c = 0; c < nc; ++c) {
        int64_t n = cols[c];
        /* dequantize row n on use */
        for (int64_t k = 0; k < K; ++k) {
          double s = oracle_half_to_double(scales[n * ng + k / G]);
          double b = oracle_half_to_double(biases[n * ng + k / G]);
          wrow[k] = (double)get_code(codes + n * wpr, k, bits) * s + b;
        }
        for (int64_t m = 0; m < M; ++m) {
          double acc = 0.0, mag = 0.0;
          for (int64_t k = 0; k < K; ++k) {
            double p = x[m * K + k] * wrow[k];
            acc += p;
            mag += fabs(p);
          }
          y[m * nc + c] = acc;
          A[m * nc + c] = mag;
        }
      }
      free(wrow);
    }
  }
  return err;
}

int oracle_matmul(const double *x, int64_t M, const uint32_t *codes, const uint16_t *scales,
                  const uint16_t *biases, int64_t N, int64_t K, int G, int bits, double *y,
                  double *A) {
  int64_t *cols = (int64_t *)malloc((size_t)(N > 0 ? N : 1) * sizeof(int64_t));
  if (!cols) return OR_ERR_ARG;
  for (int64_t n = 0; n < N; ++n) cols[n] = n;
  int st = oracle_matmul_cols(x, M, codes, scales, biases, N, K, G, bits, cols, N, y, A);
  free(cols);
  return st;
}

/* ---------------------------------------------------------------------
 * Gather (MoE experts; [MLXQ] "gather variants"; reading R6).
 * codes [E, N, K*b/32], scales/biases [E, N, K/G], ids [T, topk],
 * x [T, K] exact values; y and A are [T, topk, N].
 * ------------------------------------------------------------------- */
int oracle_gather_matmul(const double *x, int64_t T, const uint32_t *codes, const uint16_t *scales,
                         const uint16_t *biases, int64_t E, int64_t N, int64_t K,
                         const int32_t *ids, int64_t topk, int G, int bits, double *y, double *A) {
  int st = check_shape(N, K, G, bits);
  if (st) return st;
  for (int64_t i = 0; i < T * topk; ++i)
    if (ids[i] < 0 || ids[i] >= E) return OR_ERR_INDEX;
  const int64_t wpe = N * (K * bits / 32), spe = N * (K / G);
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < topk; ++j) {
      int64_t e = ids[t * topk + j];
      st = oracle_matmul(x + t * K, 1, codes + e * wpe, scales + e * spe, biases + e * spe, N, K,
                         G, bits, y + (t * topk + j) * N, A + (t * topk + j) * N);
      if (st) return st;
    }
  return OR_OK;
}

/* ---------------------------------------------------------------------
 * mxfp4 (reading R16).  codes [N, K/8] words (R3 with b = 4), scales
 * [N, K/32] bytes holding X + 127; K a multiple of 32.
 * ------------------------------------------------------------------- */
/* magnitude of E2M1 code c (0..7): m/2 for e = 0, (1 + m/2) 2^(e-1) else */
static double e2m1_magnitude(int c) {
  const int e = (c >> 1) & 3, m = c & 1;
  return e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
}

double oracle_e2m1_to_double(int code) {
  const double v = e2m1_magnitude(code & 7);
  return (code & 8) ? -v : v;
}

/* the magnitude code nearest to t >= 0 (ties to the even mantissa) */
static int e2m1_nearest(double t) {
  int best = 0;
  for (int c = 1; c < 8; ++c) {
    const double d = fabs(t - e2m1_magnitude(c)), db = fabs(t - e2m1_magnitude(best));
    if (d < db || (d == db && (c & 1) == 0 && (best & 1) == 1)) best = c;
  }
  return best;
}

/* the group's scale exponent X (R16) */
static int mx_exponent(const float *g, int n) {
  double amax = 0.0;
  for (int i = 0; i < n; ++i) {
    const double a = fabs((double)g[i]);
    if (a > amax) amax = a;
  }
  if (amax == 0.0) return -127;
  int ex;
  frexp(amax, &ex);  /* amax = f * 2^ex, f in [0.5, 1): floor(log2(amax)) = ex - 1 */
  int X = ex - 1 - 2;
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

int oracle_quantize_mxfp4(const float *w, int64_t N, int64_t K, uint32_t *codes,
                          uint8_t *scales) {
  if (N < 0 || K < 0 || K % 32) return OR_ERR_ARG;
  for (int64_t i = 0; i < N * K; ++i)
    if (!isfinite(w[i])) return OR_ERR_RANGE;
  const int64_t wpr = K / 8, ng = K / 32;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    uint32_t *row = codes + n * wpr;
    memset(row, 0, (size_t)wpr * sizeof(uint32_t));
    for (int64_t g = 0; g < ng; ++g) {
      const float *grp = w + n * K + g * 32;
      const int X = mx_exponent(grp, 32);
      scales[n * ng + g] = (uint8_t)(X + 127);
      for (int i = 0; i < 32; ++i) {
        const double t = ldexp(fabs((double)grp[i]), -X);  /* exact: a power-of-two scaling */
        const int code = (signbit(grp[i]) ? 8 : 0) | e2m1_nearest(t);
        const int64_t k = g * 32 + i;
        row[k / 8] |= (uint32_t)code << (4 * (k % 8));
      }
    }
  }
  return OR_OK;
}

/* exact dequantized values (binary64 holds every code value times 2^X) */
int oracle_dequantize_mxfp4_exact(const uint32_t *codes, const uint8_t *scales, int64_t N,
                                  int64_t K, double *out) {
  if (N < 0 || K < 0 || K % 32) return OR_ERR_ARG;
  const int64_t wpr = K / 8, ng = K / 32;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      const int code = (int)((codes[n * wpr + k / 8] >> (4 * (k % 8))) & 15u);
      out[n * K + k] = ldexp(oracle_e2m1_to_double(code), (int)scales[n * ng + k / 32] - 127);
    }
  return OR_OK;
}

/* ---------------------------------------------------------------------
 * E4M3 (readings R17, R18).
 * ------------------------------------------------------------------- */
/* magnitude of E4M3 code c (0..126): (m/8) 2^-6 for e = 0, (1 + m/8) 2^(e-7) else */
static double e4m3_magnitude(int c) {
  const int e = (c >> 3) & 15, m = c & 7;
  return e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
}

double oracle_e4m3_to_double(int code) {
  if ((code & 0x7F) == 0x7F) return NAN;
  const double v = e4m3_magnitude(code & 0x7F);
  return (code & 0x80) ? -v : v;
}

/* the finite E4M3 magnitude code (0..126) nearest to a / d (a >= 0, d > 0),
 * ties to the even code.  t > m  <=>  a > m * d, and m * d is exact (R18),
 * so every decision is exact.  The magnitudes grow with the code: the
 * candidate is the largest code whose magnitude is <= t, then the midpoint
 * to the next code decides. */
static int e4m3_nearest(double a, double d) {
  int lo = 0, hi = 126;
  while (lo < hi) { /* largest c with magnitude(c) * d <= a */
    const int mid = (lo + hi + 1) / 2;
    if (e4m3_magnitude(mid) * d <= a) lo = mid; else hi = mid - 1;
  }
  if (lo == 126) return 126;
  const double m = 0.5 * (e4m3_magnitude(lo) + e4m3_magnitude(lo + 1)) * d;
  if (a > m) return lo + 1;
  if (a == m) return (lo & 1) ? lo + 1 : lo;
  return lo;
}

/* the E2M1 magnitude code (0..7) nearest to a / s (a >= 0, s > 0), ties to
 * the even mantissa, by the same exact midpoint comparisons */
static int e2m1_nearest_scaled(double a, double s) {
  int c = 0;
  while (c < 7 && e2m1_magnitude(c + 1) * s <= a) ++c;
  if (c == 7) return 7;
  const double m = 0.5 * (e2m1_magnitude(c) + e2m1_magnitude(c + 1)) * s;
  if (a > m) return c + 1;
  if (a == m) return (c & 1) ? c + 1 : c;
  return c;
}

/* ---------------------------------------------------------------------
 * mxfp8 (reading R17).  codes [N, K/4] words (bytes in row order), scales
 * [N, K/32] bytes holding X + 127; K a multiple of 32.
 * ------------------------------------------------------------------- */
int oracle_quantize_mxfp8(const float *w, int64_t N, int64_t K, uint32_t *codes,
                          uint8_t *scales) {
  if (N < 0 || K < 0 || K % 32) return OR_ERR_ARG;
  for (int64_t i = 0; i < N * K; ++i)
    if (!isfinite(w[i])) return OR_ERR_RANGE;
  const int64_t wpr = K / 4, ng = K / 32;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    uint32_t *row = codes + n * wpr;
    memset(row, 0, (size_t)wpr * sizeof(uint32_t));
    for (int64_t g = 0; g < ng; ++g) {
      const float *grp = w + n * K + g * 32;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs((double)grp[i]));
      int X = -127;
      if (amax > 0.0) {
        int ex;
        frexp(amax, &ex); /* floor(log2(amax)) = ex - 1 */
        X = ex - 1 - 8;
        X = X < -127 ? -127 : (X > 127 ? 127 : X);
      }
      scales[n * ng + g] = (uint8_t)(X + 127);
      const double d = ldexp(1.0, X);
      for (int i = 0; i < 32; ++i) {
        const int code = (signbit(grp[i]) ? 0x80 : 0) | e4m3_nearest(fabs((double)grp[i]), d);
        const int64_t k = g * 32 + i;
        row[k / 4] |= (uint32_t)code << (8 * (k % 4));
      }
    }
  }
  return OR_OK;
}

int oracle_dequantize_mxfp8_exact(const uint32_t *codes, const uint8_t *scales, int64_t N,
                                  int64_t K, double *out) {
  if (N < 0 || K < 0 || K % 32) return OR_ERR_ARG;
  const int64_t wpr = K / 4, ng = K / 32;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      const int code = (int)((codes[n * wpr + k / 4] >> (8 * (k % 4))) & 0xFFu);
      out[n * K + k] = ldexp(oracle_e4m3_to_double(code), (int)scales[n * ng + k / 32] - 127);
    }
  return OR_OK;
}

/* ---------------------------------------------------------------------
 * nvfp4 (reading R18).  codes [N, K/8] words (as mxfp4), scales [N, K/16]
 * E4M3 bytes, tensor scale 2^T; K a multiple of 16.
 * ------------------------------------------------------------------- */
int oracle_quantize_nvfp4(const float *w, int64_t N, int64_t K, int T, uint32_t *codes,
                          uint8_t *scales) {
  if (N < 0 || K < 0 || K % 16 || T < -100 || T > 100) return OR_ERR_ARG;
  for (int64_t i = 0; i < N * K; ++i)
    if (!isfinite(w[i])) return OR_ERR_RANGE;
  const int64_t wpr = K / 8, ng = K / 16;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    uint32_t *row = codes + n * wpr;
    memset(row, 0, (size_t)wpr * sizeof(uint32_t));
    for (int64_t g = 0; g < ng; ++g) {
      const float *grp = w + n * K + g * 16;
      double amax = 0.0;
      for (int i = 0; i < 16; ++i) amax = fmax(amax, fabs((double)grp[i]));
      const int sc = e4m3_nearest(amax, ldexp(6.0, T)); /* nearest to amax / (6 * 2^T) */
      scales[n * ng + g] = (uint8_t)sc;
      const double s = ldexp(e4m3_magnitude(sc), T);    /* the group's step, s * 2^T */
      for (int i = 0; i < 16; ++i) {
        const int mag = s > 0.0 ? e2m1_nearest_scaled(fabs((double)grp[i]), s) : 0;
        const int code = (signbit(grp[i]) ? 8 : 0) | mag;
        const int64_t k = g * 16 + i;
        row[k / 8] |= (uint32_t)code << (4 * (k % 8));
      }
    }
  }
  return OR_OK;
}

int oracle_dequantize_nvfp4_exact(const uint32_t *codes, const uint8_t *scales, int64_t N,
                                  int64_t K, int T, double *out) {
  if (N < 0 || K < 0 || K % 16 || T < -100 || T > 100) return OR_ERR_ARG;
  const int64_t wpr = K / 8, ng = K / 16;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      const int code = (int)((codes[n * wpr + k / 8] >> (4 * (k % 8))) & 15u);
      out[n * K + k] =
          ldexp(oracle_e2m1_to_double(code) * oracle_e4m3_to_double(scales[n * ng + k / 16]), T);
    }
  return OR_OK;
}
