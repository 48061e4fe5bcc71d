// aq_fp.hip -- the block-scaled float modes mxfp4, nvfp4 and mxfp8, for
// gfx950: quantize, dequantize, the M = 1 matrix-vector product, the
// product for 2 and more rows of x and the mixture-of-experts gather.
//
// The modes (MLX "Quantization", the paragraph on the newer modes;
// "Quantizing a Model for MLX", "Modes, bits and mixed recipes": groups of
// 32 / 16 / 32 weights with 4 / 4 / 8-bit float codes and a per-group scale
// in place of an affine scale and bias; ExecuTorch "Quantization": nvfp4 is
// NVIDIA's FP4 weight-only format at group size 16).  The pages give no bit
// layout; the definitions of those names are taken:
//   E2M1 code (4 bits): bit 3 sign, bits 2..1 exponent e (bias 1), bit 0
//     mantissa m; (1 + m/2) 2^(e-1), or m/2 for e = 0: 0, 0.5, 1, 1.5, 2, 3,
//     4, 6.  Eight to a uint32 word, least significant nibble first.
//   E4M3 code (8 bits): bit 7 sign, bits 6..3 exponent e (bias 7), bits 2..0
//     mantissa m; (1 + m/8) 2^(e-7), or (m/8) 2^-6 for e = 0; magnitude
//     pattern 0x7F is not a number; largest 448.  Four to a word, in order.
//   mxfp4: E2M1 codes, scale 2^X per 32 (byte X + 127),
//     X = floor(log2 max|w|) - 2 clamped to [-127, 127] (-127 for zeros).
//   mxfp8: E4M3 codes, scale 2^X per 32, X = floor(log2 max|w|) - 8.
//   nvfp4: E2M1 codes, an E4M3 scale s per 16 (its byte), under a tensor
//     scale 2^T: s = the E4M3 value nearest to max|w| / (6 * 2^T), value =
//     code * s * 2^T.
//   Codes are the nearest grid values of w / scale, ties to the even code,
//   saturating at the largest finite magnitude; an nvfp4 group whose s is 0
//   keeps only signs.
//
// Quantize decisions are exact: the E2M1 midpoints times 2^X or times
// s * 2^T, and the E4M3 midpoints times 6 * 2^T, have at most 8 significant
// bits, so they are exact binary32 values, and non-negative binary32 numbers
// (subnormals included) order as their bit patterns, which is how they are
// compared; mxfp8 rounds w / 2^X (a power-of-two scaling, exact) to E4M3 by
// integer rounding of the binary32 pattern.
//
// Dequantize and the product decode codes with the gfx950 scaled converts
// (v_cvt_scalef32_pk_{f16,bf16}_{fp4,fp8}); with scale 1.0 every E2M1 and
// E4M3 value is exact in fp16 and bf16.  The product (M = 1) has the layout
// of the affine decode kernel: x resident in registers, a ring of chunk
// loads per wave across row boundaries, rows parked in LDS; a chunk (32
// codes) is dotted with x by v_dot2 in binary32 and scaled once per group.
// From two rows of x on (and for the gather) the products run on the
// matrix cores, each group's MFMA result scaled once (see mm_fp_rows_kernel).
#include "aq_device.hpp"
#include "aq_internal.hpp"

namespace aq {
namespace {

typedef _Float16 fp_h2 __attribute__((ext_vector_type(2)));
typedef __bf16 fp_b2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const uint8_t gbyte;
typedef uint32_t fp_u4 __attribute__((ext_vector_type(4)));

constexpr int kFpRound = 32;  // rows per wave between output flushes
constexpr int kFpUnroll = 4;  // 8-weight units per thread and pass (quantize, dequantize)

// ---- number formats on binary32 bit patterns ------------------------------------------

// (1 + mant / 2^23) * 2^e as a binary32 pattern; exact for -129 <= e <= 127
// with mant holding at most two leading bits (the subnormal shift drops
// only zeros)
__device__ __forceinline__ uint32_t pow2_bits(uint32_t mant, int e) {
  const int E = e + 127;
  if (E >= 1) return ((uint32_t)E << 23) | mant;
  return (0x800000u | mant) >> (1 - E);
}

// E2M1 midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 as (mantissa field, exponent)
__device__ constexpr uint32_t kMidMant[7] = {0u, 0x400000u, 0x200000u, 0x600000u,
                                             0x200000u, 0x600000u, 0x200000u};
__device__ constexpr int kMidExp[7] = {-2, -1, 0, 0, 1, 1, 2};

// the magnitude code (0..7) of a weight whose |w| has pattern a, given the
// patterns of the seven midpoints times the scale: a tie goes to the even
// mantissa, i.e. up across the midpoints into codes 2, 4, 6 and down across
// the others
__device__ __forceinline__ uint32_t e2m1_code(uint32_t a, const uint32_t (&t)[7]) {
  return (uint32_t)(a > t[0]) + (uint32_t)(a >= t[1]) + (uint32_t)(a > t[2]) +
         (uint32_t)(a >= t[3]) + (uint32_t)(a > t[4]) + (uint32_t)(a >= t[5]) +
         (uint32_t)(a > t[6]);
}

// binary32 pattern of E2M1 code c (sign in bit 3) times 2^X, X in [-127, 128];
// +-inf past the binary32 range.  Selects only: every lane takes one path.
__device__ __forceinline__ uint32_t e2m1_value_bits(uint32_t c, int X) {
  const uint32_t sign = (c & 8u) << 28, m = c & 7u;
  // m >= 1: (1 + mb/2) 2^e with e = (m >> 1) - 1, mb = m & 1 from m = 2 on
  const uint32_t mb = m >= 2u ? (m & 1u) << 22 : 0u;
  const int E = (int)(m >> 1) - 1 + X + 127;  // biased exponent, in [-1, 257]
  const uint32_t normal = ((uint32_t)E << 23) | mb;
  const uint32_t sub = (0x800000u | mb) >> ((uint32_t)(1 - E) & 31u);  // for E in {-1, 0}
  uint32_t r = E >= 255 ? 0x7F800000u : (E >= 1 ? normal : sub);
  r = m == 0u ? 0u : r;
  return sign | r;
}

// value of an E4M3 magnitude code c (0..127) as a binary32 (exact; NaN for 0x7F)
__device__ __forceinline__ float e4m3_mag(uint32_t c) {
  const int e = (int)(c >> 3), m = (int)(c & 7u);
  const float v = e ? __builtin_ldexpf((float)(8 + m), e - 10) : __builtin_ldexpf((float)m, -9);
  return c == 0x7Fu ? __builtin_nanf("") : v;
}

// the finite E4M3 magnitude code nearest to t (t >= 0 exact, t < 2^10),
// ties to the even code, saturating at 448 (code 126)
__device__ __forceinline__ uint32_t e4m3_round(float t) {
  const uint32_t b = __builtin_bit_cast(uint32_t, t);
  if (b >= 0x3C800000u) {  // t >= 2^-6: normal; round the mantissa to 3 bits
    const uint32_t r = (b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20;
    const int c = (int)r - (120 << 3);  // exponent bias 127 -> 7
    return c > 126 ? 126u : (uint32_t)c;
  }
  return (uint32_t)__builtin_rintf(t * 512.0f);  // steps of 2^-9: 0..8
}

// maximum over the lanes of a DPP quad / of a lane pair
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t pair_max(uint32_t a) {
  return umax(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t quad_max(uint32_t a) {
  a = pair_max(a);
  return umax(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x4E, 0xF, 0xF, false));
}

// ---- quantize: one thread per 8 weights ------------------------------------------------
// A workgroup takes kFpUnroll * 256 consecutive units per pass, unit
// base + u * 256 + thread, so every load and store instruction of a wave
// covers one contiguous span.  A group is the 4 (mxfp4, mxfp8) or 2 (nvfp4)
// lanes of a DPP quad or pair; the unit count is a multiple of that, so a
// group's lanes leave the loop together.
template <int MODE, int WDT>
__global__ __launch_bounds__(256) void quantize_fp_kernel(const void *__restrict__ w,
                                                          int64_t units, int T,
                                                          uint32_t *__restrict__ codes,
                                                          uint8_t *__restrict__ scales) {
  const int64_t pass = (int64_t)gridDim.x * (256 * kFpUnroll);
  for (int64_t base = (int64_t)blockIdx.x * (256 * kFpUnroll); base < units; base += pass) {
    float v[kFpUnroll][8];
#pragma unroll
    for (int u = 0; u < kFpUnroll; ++u) {
      const int64_t t = base + u * 256 + threadIdx.x;
      if (t < units) load8<WDT>(w, t * 8, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kFpUnroll; ++u) {
      const int64_t t = base + u * 256 + threadIdx.x;
      if (t >= units) break;
      uint32_t a[8], amax = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        a[i] = __builtin_bit_cast(uint32_t, v[u][i]) & 0x7FFFFFFFu;
        amax = umax(amax, a[i]);
      }
      if constexpr (MODE == FP_NVFP4) {
        amax = pair_max(amax);
        // s: the E4M3 code nearest to amax / (6 * 2^T).  The binary32
        // quotient is within a few ulps, so its rounding is at most one code
        // off; the exact tests against the midpoints between neighbouring
        // codes, times 6 * 2^T, settle it (a tie keeps the even code).
        const float amaxf = __builtin_bit_cast(float, amax);
        uint32_t sc = e4m3_round(__builtin_ldexpf(amaxf * (1.0f / 6.0f), -T));
        auto bound = [&](uint32_t c) {  // pattern of 6 * 2^T * (v(c) + v(c + 1)) / 2
          return __builtin_bit_cast(
              uint32_t, __builtin_ldexpf(3.0f * (e4m3_mag(c) + e4m3_mag(c + 1)), T));
        };
        if (sc > 0) {
          const uint32_t lo = bound(sc - 1);
          if (amax < lo || (amax == lo && (sc & 1u))) --sc;
        }
        if (sc < 126) {
          const uint32_t hi = bound(sc);
          if (amax > hi || (amax == hi && (sc & 1u))) ++sc;
        }
        const float step = __builtin_ldexpf(e4m3_mag(sc), T);  // s * 2^T, exact
        uint32_t th[7];
#pragma unroll
        for (int k = 0; k < 7; ++k)
          th[k] = __builtin_bit_cast(
              uint32_t, __builtin_bit_cast(float, pow2_bits(kMidMant[k], kMidExp[k])) * step);
        uint32_t q = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t mag = sc == 0 ? 0u : e2m1_code(a[i], th);
          q |= (mag | ((__builtin_bit_cast(uint32_t, v[u][i]) >> 31) << 3)) << (4 * i);
        }
        codes[t] = q;
        if ((threadIdx.x & 1) == 0) scales[t >> 1] = (uint8_t)sc;
      } else {
        amax = quad_max(amax);
        // floor(log2 max) = biased exponent - 127 for a normal maximum; a
        // zero or subnormal maximum has biased exponent 0 and clamps
        constexpr int EMAX = MODE == FP_MXFP4 ? 2 : 8;  // exponent of the largest code value
        const int eb = (int)(amax >> 23);
        int X = eb - 127 - EMAX;
        X = X < -127 ? -127 : X;
        if constexpr (MODE == FP_MXFP4) {
          uint32_t th[7];
#pragma unroll
          for (int k = 0; k < 7; ++k) th[k] = pow2_bits(kMidMant[k], kMidExp[k] + X);
          uint32_t q = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            q |= (e2m1_code(a[i], th) | ((__builtin_bit_cast(uint32_t, v[u][i]) >> 31) << 3))
                 << (4 * i);
          codes[t] = q;
        } else {
          // |w| / 2^X < 512 exactly (a power-of-two scaling of a normal |w|;
          // a subnormal |w| is its integer mantissa times 2^-149), then
          // rounded to E4M3; a result below 2^-126 rounds to code 0 anyway
          uint32_t q[2] = {0u, 0u};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float tq = (a[i] >> 23) ? __builtin_ldexpf(__builtin_bit_cast(float, a[i]), -X)
                                          : __builtin_ldexpf((float)a[i], -149 - X);
            const uint32_t c = e4m3_round(tq) | ((__builtin_bit_cast(uint32_t, v[u][i]) >> 31) << 7);
            q[i >> 2] |= c << (8 * (i & 3));
          }
          reinterpret_cast<uint2 *>(codes)[t] = make_uint2(q[0], q[1]);
        }
        if ((threadIdx.x & 3) == 0) scales[t >> 2] = (uint8_t)(X + 127);
      }
    }
  }
}

// ---- dequantize: one thread per 8 weights ----------------------------------------------

// eight binary32 patterns -> out[8 t .. 8 t + 7] in OUT
template <int OUT>
__device__ __forceinline__ void store8(void *out, int64_t t, const uint32_t (&f)[8]) {
  if constexpr (OUT == X_F32) {
    uint4 *o = reinterpret_cast<uint4 *>(out) + 2 * t;
    o[0] = make_uint4(f[0], f[1], f[2], f[3]);
    o[1] = make_uint4(f[4], f[5], f[6], f[7]);
  } else {
    uint32_t h[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = __builtin_bit_cast(float, f[2 * j]);
      const float b = __builtin_bit_cast(float, f[2 * j + 1]);
      if constexpr (OUT == X_F16)
        h[j] = (uint32_t)f32_to_f16_rne(a) | ((uint32_t)f32_to_f16_rne(b) << 16);
      else
        h[j] = (uint32_t)f32_to_bf16_rne(a) | ((uint32_t)f32_to_bf16_rne(b) << 16);
    }
    reinterpret_cast<uint4 *>(out)[t] = make_uint4(h[0], h[1], h[2], h[3]);
  }
}

// the two fp16 values of a convert's result as binary32 patterns
__device__ __forceinline__ void h2_to_f32(fp_h2 h, uint32_t &lo, uint32_t &hi) {
  lo = __builtin_bit_cast(uint32_t, (float)h[0]);
  hi = __builtin_bit_cast(uint32_t, (float)h[1]);
}

template <int MODE, int OUT>
__global__ __launch_bounds__(256) void dequantize_fp_kernel(const uint32_t *__restrict__ codes,
                                                            const uint8_t *__restrict__ scales,
                                                            int64_t units, int T,
                                                            void *__restrict__ out) {
  constexpr int WPU = MODE == FP_MXFP8 ? 2 : 1;  // code words per unit of 8 weights
  const int64_t pass = (int64_t)gridDim.x * (256 * kFpUnroll);
  for (int64_t base = (int64_t)blockIdx.x * (256 * kFpUnroll); base < units; base += pass) {
    uint32_t wd[kFpUnroll][WPU], sc[kFpUnroll];
#pragma unroll
    for (int u = 0; u < kFpUnroll; ++u) {
      const int64_t t = base + u * 256 + threadIdx.x;
      if (t < units) {
        if constexpr (WPU == 2) {
          const uint2 p = reinterpret_cast<const uint2 *>(codes)[t];
          wd[u][0] = p.x;
          wd[u][1] = p.y;
        } else {
          wd[u][0] = codes[t];
        }
        sc[u] = scales[MODE == FP_NVFP4 ? t >> 1 : t >> 2];
      }
    }
#pragma unroll
    for (int u = 0; u < kFpUnroll; ++u) {
      const int64_t t = base + u * 256 + threadIdx.x;
      if (t >= units) break;
      uint32_t f[8];
      if constexpr (MODE == FP_MXFP4) {
        const int X = (int)sc[u] - 127;
        // A code value times 2^X has at most two significant bits: exact in
        // bf16 (subnormals down to 2^-128 included), and binary32 is its
        // upper half.  The scaled convert (code pair * 2^X, the scale given
        // as a binary32) returns exactly that pair, +-inf past the range,
        // for X up to 127 (checked on the MI355X for every code pair and
        // exponent); X = 128 (byte 255) has no binary32 scale and takes the
        // bit construction.
        const float scale = __builtin_bit_cast(float, (uint32_t)(X + 127) << 23);
        uint32_t pr[4];
        pr[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[u][0], scale, 0));
        pr[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[u][0], scale, 1));
        pr[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[u][0], scale, 2));
        pr[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[u][0], scale, 3));
        const bool edge = X > 127;
        if constexpr (OUT == X_BF16) {
          if (!edge) {
            reinterpret_cast<uint4 *>(out)[t] = make_uint4(pr[0], pr[1], pr[2], pr[3]);
            continue;
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f[2 * j] = pr[j] << 16;
          f[2 * j + 1] = pr[j] & 0xFFFF0000u;
        }
        if (edge) {
#pragma unroll
          for (int j = 0; j < 8; ++j) f[j] = e2m1_value_bits((wd[u][0] >> (4 * j)) & 15u, X);
        }
      } else if constexpr (MODE == FP_NVFP4) {
        // |code value| (exact in fp16) times |s| * 2^T: at most six
        // significant bits and a normal binary32 (|T| <= 100), so the
        // product is exact; the signs of code and scale are applied to the
        // bits afterwards.  (Multiplying signed values, the compiler fuses
        // product and fp16 conversion into one mixed-precision FMA with a +0
        // addend, which turns a -0 product into +0.)
        const float step = __builtin_ldexpf(e4m3_mag(sc[u] & 0x7Fu), T);
        const uint32_t ssign = (sc[u] & 0x80u) << 24;
        const uint32_t mags = wd[u][0] & 0x77777777u;
        const fp_h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(mags, 1.0f, 0);
        const fp_h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(mags, 1.0f, 1);
        const fp_h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(mags, 1.0f, 2);
        const fp_h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(mags, 1.0f, 3);
        const fp_h2 ps[4] = {p0, p1, p2, p3};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f[2 * j] = __builtin_bit_cast(uint32_t, (float)ps[j][0] * step) ^ ssign ^
                     (((wd[u][0] >> (8 * j + 3)) & 1u) << 31);
          f[2 * j + 1] = __builtin_bit_cast(uint32_t, (float)ps[j][1] * step) ^ ssign ^
                         (((wd[u][0] >> (8 * j + 7)) & 1u) << 31);
        }
      } else {
        // E4M3 value (exact in fp16) times 2^X: ldexp rounds only where the
        // result leaves the binary32 range (to +-inf); binary32 subnormals
        // down to 2^-136 hold every such value exactly
        const int X = (int)sc[u] - 127;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const fp_h2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wd[u][h], 1.0f, false);
          const fp_h2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wd[u][h], 1.0f, true);
          f[4 * h] = __builtin_bit_cast(uint32_t, __builtin_ldexpf((float)lo[0], X));
          f[4 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_ldexpf((float)lo[1], X));
          f[4 * h + 2] = __builtin_bit_cast(uint32_t, __builtin_ldexpf((float)hi[0], X));
          f[4 * h + 3] = __builtin_bit_cast(uint32_t, __builtin_ldexpf((float)hi[1], X));
        }
      }
      store8<OUT>(out, t, f);
    }
  }
}

// ---- the M = 1 product -------------------------------------------------------------

// sum over the 8 E2M1 codes of word w of x * code value, x as 4 packed pairs
// in natural order (byte select b yields codes 2b and 2b + 1)
__device__ __forceinline__ float fp4_word_dot(f16_t, uint32_t w, const uint32_t *xp, float acc) {
  acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0),
                               __builtin_bit_cast(fp_h2, xp[0]), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1),
                               __builtin_bit_cast(fp_h2, xp[1]), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2),
                               __builtin_bit_cast(fp_h2, xp[2]), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3),
                               __builtin_bit_cast(fp_h2, xp[3]), acc, false);
  return acc;
}
__device__ __forceinline__ float fp4_word_dot(bf16_t, uint32_t w, const uint32_t *xp, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0),
                                        __builtin_bit_cast(fp_b2, xp[0]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1),
                                        __builtin_bit_cast(fp_b2, xp[1]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2),
                                        __builtin_bit_cast(fp_b2, xp[2]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3),
                                        __builtin_bit_cast(fp_b2, xp[3]), acc, false);
  return acc;
}
// the same for the 4 E4M3 codes of word w (x as 2 packed pairs)
__device__ __forceinline__ float fp8_word_dot(f16_t, uint32_t w, const uint32_t *xp, float acc) {
  acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false),
                               __builtin_bit_cast(fp_h2, xp[0]), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true),
                               __builtin_bit_cast(fp_h2, xp[1]), acc, false);
  return acc;
}
__device__ __forceinline__ float fp8_word_dot(bf16_t, uint32_t w, const uint32_t *xp, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false),
                                        __builtin_bit_cast(fp_b2, xp[0]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true),
                                        __builtin_bit_cast(fp_b2, xp[1]), acc, false);
  return acc;
}

// per-mode chunk layout: a chunk is 32 codes (VW 16-byte vectors) and its
// scale bytes (one exponent, or two E4M3 scales for nvfp4's two groups)
template <int MODE> struct chunk_fmt {
  static constexpr int VW = MODE == FP_MXFP8 ? 2 : 1;
  static constexpr int SB = MODE == FP_NVFP4 ? 2 : 1;
};

// x * w^ over one chunk, the chunk's scale applied
template <int MODE, typename XT>
__device__ __forceinline__ float chunk_sum(const fp_u4 (&cw)[chunk_fmt<MODE>::VW], uint32_t sb,
                                           const uint32_t *xv) {
  if constexpr (MODE == FP_MXFP4) {
    float s = 0.f;
    s = fp4_word_dot(XT{}, cw[0][0], xv, s);
    s = fp4_word_dot(XT{}, cw[0][1], xv + 4, s);
    s = fp4_word_dot(XT{}, cw[0][2], xv + 8, s);
    s = fp4_word_dot(XT{}, cw[0][3], xv + 12, s);
    return __builtin_ldexpf(s, (int)sb - 127);
  } else if constexpr (MODE == FP_NVFP4) {
    float s0 = 0.f, s1 = 0.f;
    s0 = fp4_word_dot(XT{}, cw[0][0], xv, s0);
    s0 = fp4_word_dot(XT{}, cw[0][1], xv + 4, s0);
    s1 = fp4_word_dot(XT{}, cw[0][2], xv + 8, s1);
    s1 = fp4_word_dot(XT{}, cw[0][3], xv + 12, s1);
    // the two E4M3 scales through one convert (exact in fp16)
    const fp_h2 sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb, 1.0f, false);
    return s0 * (float)sc[0] + s1 * (float)sc[1];
  } else {
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int j = 0; j < 4; ++j) s = fp8_word_dot(XT{}, cw[v][j], xv + 8 * v + 2 * j, s);
    return __builtin_ldexpf(s, (int)sb - 127);
  }
}

// a wave-uniform global pointer (its address goes to scalar registers)
__device__ __forceinline__ gbyte *wave_ptr(const void *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<gbyte *>(((uint64_t)hi << 32) | lo);
}

// code bytes and scale bytes per row
template <int MODE>
__device__ __forceinline__ void row_bytes(int64_t K, int64_t &cb, int64_t &sbb) {
  cb = MODE == FP_MXFP8 ? K : K / 2;
  sbb = MODE == FP_NVFP4 ? K / 16 : K / 32;
}

// The decode kernel for K <= 64 * 32 * CPL.  Lane l owns chunks l, l + 64,
// ... of every row (each load instruction of a wave reads 64 consecutive
// 16-byte pieces of one row) and keeps the matching x chunks in registers.
// Rows are dealt to waves round-robin (row gw, gw + TW, ...); the ring holds
// the D = CPL * UD chunk loads of UD rows and each slot is reloaded with the
// next rows' chunk as soon as it is consumed.
template <int MODE, typename XT, int CPL, int UD, int W>
__global__ __launch_bounds__(64 * W) void qmv1_fp_kernel(const uint16_t *__restrict__ x,
                                                         const uint32_t *__restrict__ codes,
                                                         const uint8_t *__restrict__ scales,
                                                         int64_t N, int64_t K, int T,
                                                         uint16_t *__restrict__ y) {
  using CF = chunk_fmt<MODE>;
  constexpr int D = CPL * UD, CP = 64 * CPL;
  constexpr int XS = (4 * CP + 64 * W - 1) / (64 * W);  // x loads per thread
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nch = (int)(K >> 5);
  int64_t rcb, rsb;
  row_bytes<MODE>(K, rcb, rsb);
  const int64_t TW = (int64_t)gridDim.x * W, gw = (int64_t)blockIdx.x * W + wave;
  const int nunits = gw < N ? (int)((N - 1 - gw) / TW + 1) : 0;
  // x as 16-byte quarters of chunks, quarter-major (quarter j of chunk c at
  // j * CP + c: 64 lanes reading one quarter hit consecutive addresses);
  // chunks past the row are zero
  uint4 *xl = reinterpret_cast<uint4 *>(smem);
  uint16_t *obuf = reinterpret_cast<uint16_t *>(smem + (size_t)CP * 64) + (size_t)wave * kFpRound;

  fp_u4 cb[D][CF::VW];
  uint32_t sb[D];
  auto load = [&](int d, int64_t row) {
    const int c0 = (d % CPL) * 64 + lane;
    const uint32_t c = (uint32_t)(c0 < nch ? c0 : nch - 1);  // padding lanes re-read the last
    gbyte *rc = wave_ptr(reinterpret_cast<const uint8_t *>(codes) + row * rcb);
    gbyte *rs = wave_ptr(scales + row * rsb);
#pragma unroll
    for (int v = 0; v < CF::VW; ++v)
      cb[d][v] = *reinterpret_cast<__attribute__((address_space(1))) const fp_u4 *>(
          rc + (c * CF::VW + v) * 16u);
    if constexpr (CF::SB == 2)
      sb[d] = *reinterpret_cast<__attribute__((address_space(1))) const uint16_t *>(rs + c * 2u);
    else
      sb[d] = rs[c];
  };

  // x loads, then the first ring fill, then x into LDS: the weight loads
  // stay in flight across the wait for x.  The first fill is unconditional
  // (a wave without rows re-reads row N - 1 and stores nothing).
  uint4 xst[XS];
  const uint4 *xg = reinterpret_cast<const uint4 *>(x);
#pragma unroll
  for (int i = 0; i < XS; ++i) {
    const int e = (int)threadIdx.x + i * 64 * W;  // quarter e & 3 of chunk e >> 2
    xst[i] = e < 4 * nch ? xg[e] : make_uint4(0u, 0u, 0u, 0u);
  }
  __builtin_amdgcn_sched_barrier(0);
  {
    const int nu = nunits < kFpRound ? nunits : kFpRound;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int i = d / CPL < nu ? d / CPL : (nu > 0 ? nu - 1 : 0);
      const int64_t row = gw + (int64_t)i * TW;
      load(d, row < N ? row : N - 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int i = 0; i < XS; ++i) {
    const int e = (int)threadIdx.x + i * 64 * W;
    if (e < 4 * CP) xl[(e & 3) * CP + (e >> 2)] = xst[i];
  }
  __syncthreads();
  if (nunits == 0) return;
  uint32_t xv[CPL][16];
#pragma unroll
  for (int p = 0; p < CPL; ++p)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 v = xl[j * CP + p * 64 + lane];
      xv[p][4 * j] = v.x; xv[p][4 * j + 1] = v.y; xv[p][4 * j + 2] = v.z; xv[p][4 * j + 3] = v.w;
    }

  for (int u0 = 0; u0 < nunits; u0 += kFpRound) {
    const int nu = nunits - u0 < kFpRound ? nunits - u0 : kFpRound;
    auto row_of = [&](int i) -> int64_t {
      i = i < nu ? i : nu - 1;  // past the end: harmless re-read of the last row
      return gw + (int64_t)(u0 + i) * TW;
    };
    if (u0 > 0) {  // the first round was filled above
#pragma unroll
      for (int d = 0; d < D; ++d) {
        load(d, row_of(d / CPL));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    float acc = 0.f;
    auto consume = [&](int d, int unit) {
      const int p = d % CPL;
      acc += chunk_sum<MODE, XT>(cb[d], sb[d], xv[p]);
      if (p == CPL - 1) {
        float v = wave_sum(acc);
        if constexpr (MODE == FP_NVFP4) v = __builtin_ldexpf(v, T);
        if (lane == 0) obuf[unit] = xtraits<XT>::from_f32(v);
        acc = 0.f;
      }
    };
    int i = 0;
    for (; i + UD <= nu; i += UD) {  // whole rings of UD rows
#pragma unroll
      for (int d = 0; d < D; ++d) {
        consume(d, i + d / CPL);
        load(d, row_of(i + UD + d / CPL));
        __builtin_amdgcn_sched_barrier(0);  // keep each reload right behind its use
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d)  // the last < UD rows: already loaded
      if (i + d / CPL < nu) consume(d, i + d / CPL);
    __builtin_amdgcn_wave_barrier();
    for (int e = lane; e < nu; e += 64) y[gw + (int64_t)(u0 + e) * TW] = obuf[e];
    __builtin_amdgcn_wave_barrier();
  }
}

// The decode kernel for longer rows: x stays in LDS (K * 2 bytes) and every
// lane walks its chunks l, l + 64, ... reading x from there.
template <int MODE, typename XT, int W>
__global__ __launch_bounds__(64 * W) void qmv1_fp_lds_kernel(const uint16_t *__restrict__ x,
                                                             const uint32_t *__restrict__ codes,
                                                             const uint8_t *__restrict__ scales,
                                                             int64_t N, int64_t K, int T,
                                                             uint16_t *__restrict__ y) {
  using CF = chunk_fmt<MODE>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nch = (int)(K >> 5);
  int64_t rcb, rsb;
  row_bytes<MODE>(K, rcb, rsb);
  uint4 *xl = reinterpret_cast<uint4 *>(smem);  // chunk c at xl[4 c .. 4 c + 3]
  const uint4 *xg = reinterpret_cast<const uint4 *>(x);
  for (int e = (int)threadIdx.x; e < 4 * nch; e += 64 * W) xl[e] = xg[e];
  __syncthreads();
  const int64_t TW = (int64_t)gridDim.x * W;
  for (int64_t row = (int64_t)blockIdx.x * W + wave; row < N; row += TW) {
    gbyte *rc = wave_ptr(reinterpret_cast<const uint8_t *>(codes) + row * rcb);
    gbyte *rs = wave_ptr(scales + row * rsb);
    float acc = 0.f;
#pragma unroll 4
    for (int c = lane; c < nch; c += 64) {
      fp_u4 cw[CF::VW];
#pragma unroll
      for (int v = 0; v < CF::VW; ++v)
        cw[v] = *reinterpret_cast<__attribute__((address_space(1))) const fp_u4 *>(
            rc + ((uint32_t)c * CF::VW + v) * 16u);
      uint32_t sbv;
      if constexpr (CF::SB == 2)
        sbv = *reinterpret_cast<__attribute__((address_space(1))) const uint16_t *>(
            rs + (uint32_t)c * 2u);
      else
        sbv = rs[c];
      uint32_t xp[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 v = xl[4 * c + j];
        xp[4 * j] = v.x; xp[4 * j + 1] = v.y; xp[4 * j + 2] = v.z; xp[4 * j + 3] = v.w;
      }
      acc += chunk_sum<MODE, XT>(cw, sbv, xp);
    }
    float v = wave_sum(acc);
    if constexpr (MODE == FP_NVFP4) v = __builtin_ldexpf(v, T);
    if (lane == 0) y[row] = xtraits<XT>::from_f32(v);
  }
}

// ---- products for 2 and more rows of x, on the matrix cores ---------------------------
//
// y[m, n] = sum_k x[m, k] * w^[n, k] for slices of up to 16 rows of x (the
// QMV of "Quantization", metalworking MLX notes, at the widths of its
// dispatch section: several rows of x per pass over W, as in speculative
// decoding).  v_mfma_f32_16x16x32_{f16,bf16}: A = 16 rows of x (rows past M
// read as zero), B = 16 rows of W over one 32-code chunk, its codes
// converted with scale 1 (E2M1 and E4M3 values are exact in fp16 and
// bf16).  An mx group is one chunk, so each MFMA's result is the group's
// sum, scaled once by its 2^X into the binary32 accumulators; nvfp4's chunk
// holds two 16-code groups, so it takes two MFMAs against x masked to each
// group's half of the chunk, and the matrix's 2^T is applied to the sums.
//  * Loads: lane (n16 = l % 16, quarter h = l / 16) of block b reads chunk
//    c0 + h of W row 16 b + n16 (16 bytes; fp8 32), and a 4x4 transpose of
//    (quarter, word) gives quarter h word h of every chunk of the step (fp8:
//    words 2h and 2h + 1): codes 8h .. 8h + 7 of chunk c0 + j, the B operand
//    of MFMA j.  x comes straight from global memory (it stays in L2), one
//    16-byte load per lane and chunk (codes 8h .. 8h + 7 of x row n16, the A
//    operand), shared by the R blocks; scales, two dword loads (nvfp4:
//    three) per row and step from the dword boundary below the step's first
//    scale byte.
//  * Workgroup: R blocks of 16 rows of W, K split over W waves in steps of
//    4 chunks, D steps of loads in flight per wave; chunks past K read as
//    zero through out-of-range buffer offsets; the waves' partial sums meet
//    in LDS.
constexpr uint32_t kFpOutside = 0x80000000u;  // a buffer offset past every resource

__device__ __forceinline__ __amdgpu_buffer_rsrc_t fp_rsrc(const void *base, int64_t bytes) {
  const int n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (bytes < 0 ? 0 : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, n, 0x00020000);
}

typedef float fp_f4 __attribute__((ext_vector_type(4)));
typedef _Float16 fp_h8 __attribute__((ext_vector_type(8)));
typedef __bf16 fp_b8 __attribute__((ext_vector_type(8)));

template <typename XT>
__device__ __forceinline__ fp_f4 mfma_x16(fp_u4 a, fp_u4 b) {
  const fp_f4 z = {0.f, 0.f, 0.f, 0.f};
  if constexpr (std::is_same<XT, bf16_t>::value)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(fp_b8, a),
                                                   __builtin_bit_cast(fp_b8, b), z, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(fp_h8, a),
                                                  __builtin_bit_cast(fp_h8, b), z, 0, 0, 0);
}

// 4x4 transpose of (lane quarter, word): afterwards quarter h holds in r[j]
// what quarter j held in r[h]
__device__ __forceinline__ void quarter_transpose(uint32_t (&r)[4]) {
  auto a = __builtin_amdgcn_permlane32_swap(r[0], r[2], false, false);
  r[0] = a[0]; r[2] = a[1];
  auto b = __builtin_amdgcn_permlane32_swap(r[1], r[3], false, false);
  r[1] = b[0]; r[3] = b[1];
  auto c = __builtin_amdgcn_permlane16_swap(r[0], r[1], false, false);
  r[0] = c[0]; r[1] = c[1];
  auto d = __builtin_amdgcn_permlane16_swap(r[2], r[3], false, false);
  r[2] = d[0]; r[3] = d[1];
}

// 8 consecutive codes (fp4: one word; fp8: two) -> their exact values as 4
// packed pairs in the activation type, natural order
template <int MODE, typename XT>
__device__ __forceinline__ fp_u4 codes_to_b(uint32_t w0, uint32_t w1) {
  fp_u4 b;
  if constexpr (MODE == FP_MXFP8) {
    if constexpr (std::is_same<XT, bf16_t>::value) {
      b[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
      b[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
      b[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
      b[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
    } else {
      b[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false));
      b[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true));
      b[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false));
      b[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true));
    }
  } else {
    (void)w1;
    if constexpr (std::is_same<XT, bf16_t>::value) {
      b[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w0, 1.0f, 0));
      b[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w0, 1.0f, 1));
      b[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w0, 1.0f, 2));
      b[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w0, 1.0f, 3));
    } else {
      b[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 0));
      b[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 1));
      b[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 2));
      b[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 3));
    }
  }
  return b;
}

// DPP row_ror: lane l of each row of 16 lanes receives the value of lane
// (l + 16 - K16) % 16 of the same row
template <int K16>
__device__ __forceinline__ fp_u4 fp_row_ror(fp_u4 v) {
  if constexpr (K16 == 0) {
    return v;
  } else {
    constexpr int ctl = 0x120 + K16;
    fp_u4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = (uint32_t)__builtin_amdgcn_mov_dpp((int)v[i], ctl, 0xF, 0xF, false);
    return r;
  }
}

// One pass of a workgroup over its R blocks of 16 rows of W against up to
// XR rows of x: lane (n16, h) gets the byte offset xro of x row n16 % XR in
// rx (kFpOutside for a missing row: it reads as zero); srow0 is the block's
// first row in the scale array rs.  XR = 8 or 4 (at most that many rows of
// x): the A-operand rows XR..15 only feed discarded output rows, so one
// 16-byte x load carries 16 / XR chunks (lanes XR s .. XR s + XR - 1 of each
// row of 16 hold chunk slot s) and a row rotation moves a slot into lanes
// 0 .. XR - 1: a half or a quarter of the x loads.
// Leaves the x rows x W rows sums of the wave's K range in part[wave] (entry
// [b][n][m] for W row 16 b + n, x row m; rows m >= XR hold no result) and
// meets the other waves at a barrier; the caller adds the W partial sums.
template <int MODE, typename XT, int W, int R, int D, int XR>
__device__ __forceinline__ void fp_rows_pass(__amdgpu_buffer_rsrc_t rx, uint32_t xro,
                                             __amdgpu_buffer_rsrc_t rc,
                                             __amdgpu_buffer_rsrc_t rs, int64_t srow0,
                                             int64_t K, float (*part)[R][16][16]) {
  using CF = chunk_fmt<MODE>;
  constexpr int CB = 16 * CF::VW;      // code bytes per chunk and row
  constexpr int NSW = CF::SB + 1;      // scale dwords loaded per row and step
  constexpr int NXL = 16 / XR;         // chunks per x load
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15, h = lane >> 4;
  const int nch = (int)(K >> 5);
  const int nsteps = (nch + 3) >> 2;
  const int spw = (nsteps + W - 1) / W;
  const int s0 = wave * spw, s1 = s0 + spw < nsteps ? s0 + spw : nsteps;
  int64_t rcb, rsb;
  row_bytes<MODE>(K, rcb, rsb);

  struct Step {
    uint32_t cw[R][4 * CF::VW];  // chunk c0 + h of row 16 b + n16, as loaded
    uint32_t sc[R][NSW];         // dwords holding the row's scale bytes of the step
    fp_u4 xl[4 / NXL];           // codes 8h .. 8h + 7 of chunk c0 + NXL q + n16 / XR of x row n16 % XR
  };
  auto load = [&](Step &st, int s) {
    const bool in = s < s1;  // uniform; past the range every offset lies outside
    const int c0 = 4 * s;
#pragma unroll
    for (int b = 0; b < R; ++b) {
      const int r = 16 * b + n16, c = c0 + h;
      const uint32_t off = in && c < nch ? (uint32_t)(r * rcb + (int64_t)c * CB) : kFpOutside;
#pragma unroll
      for (int v = 0; v < CF::VW; ++v) {
        const fp_u4 t = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)(off + 16u * v), 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) st.cw[b][4 * v + i] = t[i];
      }
      const uint32_t so = (uint32_t)((srow0 + r) * rsb + (int64_t)c0 * CF::SB);
      const uint32_t sa = in ? (so & ~3u) : kFpOutside;
#pragma unroll
      for (int i = 0; i < NSW; ++i)
        st.sc[b][i] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(sa + 4u * i), 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 4 / NXL; ++q) {
      const int c = c0 + NXL * q + n16 / XR;
      const uint32_t off =
          in && c < nch ? (uint32_t)(xro + ((int64_t)c * 32 + 8 * h) * 2) : kFpOutside;
      st.xl[q] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0);
    }
  };

  fp_f4 acc[R];
#pragma unroll
  for (int b = 0; b < R; ++b) acc[b] = fp_f4{0.f, 0.f, 0.f, 0.f};
  const fp_u4 zero4 = {0u, 0u, 0u, 0u};
  auto compute = [&](const Step &st, int s) {
    const int c0 = 4 * s;
    fp_u4 xa[4];  // the A operand of chunk c0 + j: x rows in lanes 0 .. XR - 1
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (NXL == 1) {
        xa[j] = st.xl[j];
      } else if constexpr (NXL == 2) {
        xa[j] = (j & 1) ? fp_row_ror<8>(st.xl[j >> 1]) : st.xl[j >> 1];
      } else {  // chunk j in lanes 4j .. 4j + 3
        xa[j] = j == 0 ? st.xl[0]
              : j == 1 ? fp_row_ror<12>(st.xl[0])
              : j == 2 ? fp_row_ror<8>(st.xl[0]) : fp_row_ror<4>(st.xl[0]);
      }
    }
#pragma unroll
    for (int b = 0; b < R; ++b) {
      uint32_t e[4], o[4];  // fp4: word h of each chunk; fp8: words 2h and 2h + 1
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[i] = st.cw[b][CF::VW * i];
        o[i] = CF::VW == 2 ? st.cw[b][2 * i + 1] : 0u;
      }
      quarter_transpose(e);
      if constexpr (CF::VW == 2) quarter_transpose(o);
      // the row's scale bytes of chunks c0 .. c0 + 3 (SB each), from the
      // dwords loaded at the dword boundary below them
      const uint32_t sh = (uint32_t)((srow0 + 16 * b + n16) * rsb) & 3u;
      const uint32_t sl = __builtin_amdgcn_alignbyte(st.sc[b][1], st.sc[b][0], sh);
      const uint32_t sh2 = CF::SB == 2 ? __builtin_amdgcn_alignbyte(st.sc[b][NSW - 1], st.sc[b][1], sh)
                                       : 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool live = c0 + j < nch;  // uniform: chunks past K contribute nothing
        const fp_u4 bw = codes_to_b<MODE, XT>(e[j], o[j]);
        if constexpr (MODE == FP_NVFP4) {
          // the two E4M3 scales of the chunk (its groups 0 and 1) through one
          // convert (exact in fp16); x masked to each group's 16 codes
          const uint32_t sw = j < 2 ? sl : sh2;
          const fp_h2 g = (j & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, true)
                                  : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
          const fp_u4 x0 = h < 2 ? xa[j] : zero4, x1 = h < 2 ? zero4 : xa[j];
          const fp_f4 t0 = mfma_x16<XT>(x0, bw), t1 = mfma_x16<XT>(x1, bw);
          const float g0 = live ? (float)g[0] : 0.f, g1 = live ? (float)g[1] : 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[b][i] = __builtin_fmaf(t1[i], g1, __builtin_fmaf(t0[i], g0, acc[b][i]));
        } else {
          const float g = live ? __builtin_ldexpf(1.0f, (int)((sl >> (8 * j)) & 0xFFu) - 127) : 0.f;
          const fp_f4 t = mfma_x16<XT>(xa[j], bw);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[b][i] = __builtin_fmaf(t[i], g, acc[b][i]);
        }
      }
    }
  };

  Step st[D];
#pragma unroll
  for (int d = 0; d < D; ++d) load(st[d], s0 + d);
  for (int s = s0; s < s1; s += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (s + d < s1) compute(st[d], s + d);
      load(st[d], s + d + D);
    }
  }
  // lane (n16, h) holds x rows 4h .. 4h + 3 of W row 16 b + n16
#pragma unroll
  for (int b = 0; b < R; ++b)
    *reinterpret_cast<fp_f4 *>(&part[wave][b][n16][4 * h]) = acc[b];
  __syncthreads();
}

template <int MODE, typename XT, int W, int R, int D, int XR>
__global__ __launch_bounds__(64 * W) void mm_fp_rows_kernel(const uint16_t *__restrict__ x,
                                                            int64_t M,
                                                            const uint32_t *__restrict__ codes,
                                                            const uint8_t *__restrict__ scales,
                                                            int64_t N, int64_t K, int T,
                                                            uint16_t *__restrict__ y) {
  __shared__ __attribute__((aligned(16))) float part[W][R][16][16];
  const int n16 = threadIdx.x & 15;
  const int64_t row0 = (int64_t)blockIdx.x * 16 * R;
  const int64_t rows = N - row0 < 16 * R ? N - row0 : 16 * R;
  const int64_t m0 = (int64_t)blockIdx.y * 16;
  const int64_t mrows = M - m0 < 16 ? M - m0 : 16;
  int64_t rcb, rsb;
  row_bytes<MODE>(K, rcb, rsb);
  const __amdgpu_buffer_rsrc_t rc =
      fp_rsrc(reinterpret_cast<const uint8_t *>(codes) + row0 * rcb, rows * rcb);
  // scales: the whole array, in whole dwords (it starts 16-byte aligned, so
  // the dword holding its last byte lies inside its allocation)
  const __amdgpu_buffer_rsrc_t rs = fp_rsrc(scales, (N * rsb + 3) & ~(int64_t)3);
  const __amdgpu_buffer_rsrc_t rx = fp_rsrc(x + m0 * K, mrows * K * 2);
  const int xm = n16 % XR;
  fp_rows_pass<MODE, XT, W, R, D, XR>(rx, xm < mrows ? (uint32_t)(xm * K * 2) : kFpOutside, rc,
                                      rs, row0, K, part);
  for (int t = threadIdx.x; t < R * 256; t += 64 * W) {
    const int b = t >> 8, m = (t >> 4) & 15, nn = t & 15;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) v += part[w][b][nn][m];
    if constexpr (MODE == FP_NVFP4) v = __builtin_ldexpf(v, T);
    const int64_t n = row0 + 16 * b + nn;
    if (m < mrows && n < N) y[(m0 + m) * N + n] = xtraits<XT>::from_f32(v);
  }
}

// Mixture-of-experts gather of the block-scaled product ("Quantization",
// metalworking: gather variants of the kernels for MoE experts):
// y[t, j, :] = x[t] @ W_{ids[t, j]}^T.  One workgroup per (32 rows, expert
// e) lists the (token, slot) pairs routed to e, 256 ids at a time, and runs
// them through fp_rows_pass in batches of 16 (x rows by token, y rows by
// pair), so each expert's rows are read once per batch of 16 pairs that
// chose it and experts no pair chose are never read.  Pairs whose id lies
// outside [0, E) get zero rows, written by the workgroups of expert 0.
template <int MODE, typename XT, int W, int R, int D>
__global__ __launch_bounds__(64 * W) void gather_fp_rows_kernel(
    const uint16_t *__restrict__ x, int64_t Tk, const uint32_t *__restrict__ codes,
    const uint8_t *__restrict__ scales, int64_t E, int64_t N, int64_t K,
    const int32_t *__restrict__ ids, int topk, int T, uint16_t *__restrict__ y) {
  __shared__ __attribute__((aligned(16))) float part[W][R][16][16];
  __shared__ int list[256];
  __shared__ int count;
  const int n16 = threadIdx.x & 15;
  const int64_t e = blockIdx.y;
  const int64_t row0 = (int64_t)blockIdx.x * 16 * R;
  const int64_t rows = N - row0 < 16 * R ? N - row0 : 16 * R;
  const int64_t total = Tk * topk;
  int64_t rcb, rsb;
  row_bytes<MODE>(K, rcb, rsb);
  if (e == 0)
    for (int64_t p = threadIdx.x; p < total; p += 64 * W) {
      const int32_t id = ids[p];
      if (id < 0 || id >= E)
        for (int nn = 0; nn < rows; ++nn) y[p * N + row0 + nn] = 0;
    }
  const __amdgpu_buffer_rsrc_t rc = fp_rsrc(
      reinterpret_cast<const uint8_t *>(codes) + (e * N + row0) * rcb, rows * rcb);
  const __amdgpu_buffer_rsrc_t rs = fp_rsrc(scales, (E * N * rsb + 3) & ~(int64_t)3);
  const __amdgpu_buffer_rsrc_t rx = fp_rsrc(x, Tk * K * 2);
  for (int64_t t0 = 0; t0 < total; t0 += 256) {
    __syncthreads();  // every thread has read the last round's count
    if (threadIdx.x == 0) count = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < 256; i += 64 * W) {
      const int64_t p = t0 + i;
      if (p < total && ids[p] == e) list[atomicAdd(&count, 1)] = i;
    }
    __syncthreads();
    const int n = count;
    for (int b0 = 0; b0 < n; b0 += 16) {  // uniform
      const int nb = n - b0 < 16 ? n - b0 : 16;
      const uint32_t xro = n16 < nb ? (uint32_t)(((t0 + list[b0 + n16]) / topk) * K * 2)
                                    : kFpOutside;
      fp_rows_pass<MODE, XT, W, R, D, 16>(rx, xro, rc, rs, e * N + row0, K, part);
      for (int t = threadIdx.x; t < R * 256; t += 64 * W) {
        const int b = t >> 8, m = (t >> 4) & 15, nn = t & 15;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) v += part[w][b][nn][m];
        if constexpr (MODE == FP_NVFP4) v = __builtin_ldexpf(v, T);
        const int64_t nr = row0 + 16 * b + nn;
        if (m < nb && nr < N) y[(t0 + list[b0 + m]) * N + nr] = xtraits<XT>::from_f32(v);
      }
      __syncthreads();  // part and list reused
    }
  }
}

template <typename KernelT>
int resident_blocks(KernelT kern, int threads, size_t lds) {
  int v = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, reinterpret_cast<const void *>(kern),
                                                   threads, lds) != hipSuccess ||
      v <= 0)
    v = 1;
  return v;
}

template <int MODE, typename XT, int CPL, int UD, int W>
hipError_t qmv1_fp_launch(const void *x, const uint32_t *codes, const uint8_t *scales, int64_t N,
                          int64_t K, int T, void *y, int wpc, hipStream_t s) {
  auto kern = qmv1_fp_kernel<MODE, XT, CPL, UD, W>;
  const size_t lds = (size_t)64 * CPL * 64 + (size_t)W * kFpRound * 2;
  static int per_cu = 0;  // resident workgroups per CU for this instantiation
  if (per_cu == 0) per_cu = resident_blocks(kern, 64 * W, lds);
  const int64_t want = (N + W - 1) / W;
  const int64_t cap = (int64_t)device_cus() * (wpc > 0 && wpc < per_cu ? wpc : per_cu);
  const dim3 grid((unsigned)(want < cap ? want : cap));
  hipLaunchKernelGGL(kern, grid, dim3(64 * W), lds, s, (const uint16_t *)x, codes, scales, N, K, T,
                     (uint16_t *)y);
  return hipGetLastError();
}

template <int MODE, typename XT>
hipError_t qmv1_fp_lds_launch(const void *x, const uint32_t *codes, const uint8_t *scales,
                              int64_t N, int64_t K, int T, void *y, hipStream_t s) {
  constexpr int W = 8;
  auto kern = qmv1_fp_lds_kernel<MODE, XT, W>;
  const size_t lds = (size_t)K * 2;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)lds);
    if (e != hipSuccess) return e;
  }
  const int per_cu = resident_blocks(kern, 64 * W, lds);
  const int64_t want = (N + W - 1) / W;
  const int64_t cap = (int64_t)device_cus() * per_cu;
  const dim3 grid((unsigned)(want < cap ? want : cap));
  hipLaunchKernelGGL(kern, grid, dim3(64 * W), lds, s, (const uint16_t *)x, codes, scales, N, K, T,
                     (uint16_t *)y);
  return hipGetLastError();
}

template <int MODE, typename XT>
hipError_t qmv_fp_dispatch(const void *x, const uint32_t *codes, const uint8_t *scales, int64_t N,
                           int64_t K, int T, void *y, hipStream_t s) {
  int cpl, ud, w, wpc;
  qmv1_fp_shape(N, K, MODE, cpl, ud, w, wpc);
#define AQ_FP1(C, U, WW) \
  return qmv1_fp_launch<MODE, XT, C, U, WW>(x, codes, scales, N, K, T, y, wpc, s)
  switch (cpl) {
    case 0: return qmv1_fp_lds_launch<MODE, XT>(x, codes, scales, N, K, T, y, s);
    case 1: AQ_FP1(1, 4, 4);
    case 2:
      if (w == 16) AQ_FP1(2, 1, 16);
      if (ud == 1) AQ_FP1(2, 1, 4);
      AQ_FP1(2, 2, 4);
    case 3: AQ_FP1(3, 1, 4);
    case 4: AQ_FP1(4, 1, 4);
    case 5: AQ_FP1(5, 1, 8);
    case 6: AQ_FP1(6, 1, 8);
    case 7: AQ_FP1(7, 1, 8);
    case 8: AQ_FP1(8, 1, 8);
  }
#undef AQ_FP1
  return hipErrorInvalidValue;
}

template <int MODE>
hipError_t qmv_fp_mode(const void *x, int x_dtype, const uint32_t *codes, const uint8_t *scales,
                       int64_t N, int64_t K, int T, void *y, hipStream_t s) {
  if (x_dtype == X_F16) return qmv_fp_dispatch<MODE, f16_t>(x, codes, scales, N, K, T, y, s);
  if (x_dtype == X_BF16) return qmv_fp_dispatch<MODE, bf16_t>(x, codes, scales, N, K, T, y, s);
  return hipErrorInvalidValue;
}

// 2+ rows of x: workgroups of R blocks of 16 rows of W per slice of 16 x
// rows (R = 2, or 1 when that leaves compute units without a workgroup),
// and the steps of 4 chunks split over 2, 4 or 8 waves so that the launch
// holds about four waves per SIMD, each wave with at least 4 steps (16-wave
// workgroups would cap a wave at 128 registers: nvfp4 then spills); D steps
// of loads in flight per wave
template <int MODE> constexpr int kFewDepth = 2;

template <int MODE, typename XT, int R, int XR>
hipError_t mm_fp_rows_r(const void *x, int64_t M, const uint32_t *codes, const uint8_t *scales,
                        int64_t N, int64_t K, int T, void *y, hipStream_t s) {
  constexpr int D = kFewDepth<MODE>;
  const int64_t blocks = (N + 16 * R - 1) / (16 * R), slices = (M + 15) / 16;
  if (blocks > 0x7FFFFFFF || slices > 65535) return hipErrorInvalidValue;
  const int64_t steps = (K / 32 + 3) / 4, wgs = blocks * slices;
  const int64_t target = 4 * 4 * (int64_t)device_cus();
  int w = wgs * 2 >= target ? 2 : wgs * 4 >= target ? 4 : 8;
  while (w > 2 && steps < 4 * w) w /= 2;
  const dim3 grid((unsigned)blocks, (unsigned)slices);
#define AQ_MMFP(WW)                                                                           \
  hipLaunchKernelGGL((mm_fp_rows_kernel<MODE, XT, WW, R, D, XR>), grid, dim3(64 * WW), 0, s,  \
                     (const uint16_t *)x, M, codes, scales, N, K, T, (uint16_t *)y);          \
  break;
  switch (w) {
    case 2: AQ_MMFP(2)
    case 4: AQ_MMFP(4)
    default: AQ_MMFP(8)
  }
#undef AQ_MMFP
  return hipGetLastError();
}

template <int MODE, typename XT>
hipError_t mm_fp_rows_mode(const void *x, int64_t M, const uint32_t *codes, const uint8_t *scales,
                           int64_t N, int64_t K, int T, void *y, hipStream_t s) {
  const bool two = (N + 31) / 32 * ((M + 15) / 16) >= device_cus();
  if (M <= 4)  // up to 4 rows of x: four chunks per x load
    return two ? mm_fp_rows_r<MODE, XT, 2, 4>(x, M, codes, scales, N, K, T, y, s)
               : mm_fp_rows_r<MODE, XT, 1, 4>(x, M, codes, scales, N, K, T, y, s);
  if (M <= 8)  // up to 8 rows of x: two chunks per x load
    return two ? mm_fp_rows_r<MODE, XT, 2, 8>(x, M, codes, scales, N, K, T, y, s)
               : mm_fp_rows_r<MODE, XT, 1, 8>(x, M, codes, scales, N, K, T, y, s);
  return two ? mm_fp_rows_r<MODE, XT, 2, 16>(x, M, codes, scales, N, K, T, y, s)
             : mm_fp_rows_r<MODE, XT, 1, 16>(x, M, codes, scales, N, K, T, y, s);
}

// gather: workgroups of 32 rows of one expert (16 when that leaves compute
// units idle), steps split over 2, 4 or 8 waves as above
template <int MODE, typename XT, int R>
hipError_t gather_fp_rows_r(const void *x, int64_t Tk, const uint32_t *codes,
                            const uint8_t *scales, int64_t E, int64_t N, int64_t K,
                            const int32_t *ids, int topk, int T, void *y, hipStream_t s) {
  constexpr int D = kFewDepth<MODE>;
  const int64_t blocks = (N + 16 * R - 1) / (16 * R);
  if (blocks > 0x7FFFFFFF || E > 65535) return hipErrorInvalidValue;
  const int64_t steps = (K / 32 + 3) / 4, wgs = blocks * E;
  const int64_t target = 4 * 4 * (int64_t)device_cus();
  int w = wgs * 2 >= target ? 2 : wgs * 4 >= target ? 4 : 8;
  while (w > 2 && steps < 4 * w) w /= 2;
  const dim3 grid((unsigned)blocks, (unsigned)E);
#define AQ_GFP(WW)                                                                              \
  hipLaunchKernelGGL((gather_fp_rows_kernel<MODE, XT, WW, R, D>), grid, dim3(64 * WW), 0, s,    \
                     (const uint16_t *)x, Tk, codes, scales, E, N, K, ids, topk, T,             \
                     (uint16_t *)y);                                                            \
  break;
  switch (w) {
    case 2: AQ_GFP(2)
    case 4: AQ_GFP(4)
    default: AQ_GFP(8)
  }
#undef AQ_GFP
  return hipGetLastError();
}

template <int MODE>
hipError_t gather_fp_rows_dtype(const void *x, int x_dtype, int64_t Tk, const uint32_t *codes,
                                const uint8_t *scales, int64_t E, int64_t N, int64_t K,
                                const int32_t *ids, int topk, int T, void *y, hipStream_t s) {
  const bool two = (N + 31) / 32 * E >= device_cus();
  if (x_dtype == X_F16)
    return two ? gather_fp_rows_r<MODE, f16_t, 2>(x, Tk, codes, scales, E, N, K, ids, topk, T, y, s)
               : gather_fp_rows_r<MODE, f16_t, 1>(x, Tk, codes, scales, E, N, K, ids, topk, T, y, s);
  if (x_dtype == X_BF16)
    return two ? gather_fp_rows_r<MODE, bf16_t, 2>(x, Tk, codes, scales, E, N, K, ids, topk, T, y, s)
               : gather_fp_rows_r<MODE, bf16_t, 1>(x, Tk, codes, scales, E, N, K, ids, topk, T, y, s);
  return hipErrorInvalidValue;
}

template <int MODE>
hipError_t mm_fp_rows_dtype(const void *x, int x_dtype, int64_t M, const uint32_t *codes,
                            const uint8_t *scales, int64_t N, int64_t K, int T, void *y,
                            hipStream_t s) {
  if (x_dtype == X_F16) return mm_fp_rows_mode<MODE, f16_t>(x, M, codes, scales, N, K, T, y, s);
  if (x_dtype == X_BF16) return mm_fp_rows_mode<MODE, bf16_t>(x, M, codes, scales, N, K, T, y, s);
  return hipErrorInvalidValue;
}

// grid for the quantize / dequantize loops: kFpUnroll units per thread and
// pass, at most 2^22 workgroups (then several passes)
dim3 unit_grid(int64_t units) {
  const int64_t b = (units + 256 * kFpUnroll - 1) / (256 * kFpUnroll);
  return dim3((unsigned)(b < (1 << 22) ? b : (1 << 22)));
}

template <int MODE>
hipError_t quantize_fp_mode(const void *w, int w_dtype, int64_t units, int T, uint32_t *codes,
                            uint8_t *scales, hipStream_t s) {
  const dim3 grid = unit_grid(units);
  switch (w_dtype) {
    case X_F32:
      hipLaunchKernelGGL((quantize_fp_kernel<MODE, X_F32>), grid, dim3(256), 0, s, w, units, T,
                         codes, scales);
      break;
    case X_F16:
      hipLaunchKernelGGL((quantize_fp_kernel<MODE, X_F16>), grid, dim3(256), 0, s, w, units, T,
                         codes, scales);
      break;
    case X_BF16:
      hipLaunchKernelGGL((quantize_fp_kernel<MODE, X_BF16>), grid, dim3(256), 0, s, w, units, T,
                         codes, scales);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int MODE>
hipError_t dequantize_fp_mode(const uint32_t *codes, const uint8_t *scales, int64_t units, int T,
                              void *out, int out_dtype, hipStream_t s) {
  const dim3 grid = unit_grid(units);
  switch (out_dtype) {
    case X_F32:
      hipLaunchKernelGGL((dequantize_fp_kernel<MODE, X_F32>), grid, dim3(256), 0, s, codes, scales,
                         units, T, out);
      break;
    case X_F16:
      hipLaunchKernelGGL((dequantize_fp_kernel<MODE, X_F16>), grid, dim3(256), 0, s, codes, scales,
                         units, T, out);
      break;
    case X_BF16:
      hipLaunchKernelGGL((dequantize_fp_kernel<MODE, X_BF16>), grid, dim3(256), 0, s, codes,
                         scales, units, T, out);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// M = 1 launch shape: the affine decode kernel's (x chunks per lane, rows in
// flight, waves per workgroup, workgroups per CU); cpl = 0 selects the LDS
// kernel: for K > 16384, and for nvfp4 at 8 chunks per lane (its two scales
// per chunk would push the register kernel past 256 registers).
void qmv1_fp_shape(int64_t N, int64_t K, int mode, int &cpl, int &ud, int &w, int &wpc) {
  int sl;
  if (K > 8 * 2048 || (mode == FP_NVFP4 && K > 7 * 2048)) {
    cpl = 0;
    ud = 1;
    w = 8;
    wpc = 0;
    return;
  }
  qmv1_shape(N, K, 32, cpl, ud, w, sl, wpc);
}

hipError_t launch_quantize_fp(const void *w, int w_dtype, int64_t N, int64_t K, int mode, int T,
                              uint32_t *codes, uint8_t *scales, hipStream_t s) {
  const int64_t units = N * (K / 8);
  switch (mode) {
    case FP_MXFP4: return quantize_fp_mode<FP_MXFP4>(w, w_dtype, units, T, codes, scales, s);
    case FP_NVFP4: return quantize_fp_mode<FP_NVFP4>(w, w_dtype, units, T, codes, scales, s);
    case FP_MXFP8: return quantize_fp_mode<FP_MXFP8>(w, w_dtype, units, T, codes, scales, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_dequantize_fp(const uint32_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                                int mode, int T, void *out, int out_dtype, hipStream_t s) {
  const int64_t units = N * (K / 8);
  switch (mode) {
    case FP_MXFP4: return dequantize_fp_mode<FP_MXFP4>(codes, scales, units, T, out, out_dtype, s);
    case FP_NVFP4: return dequantize_fp_mode<FP_NVFP4>(codes, scales, units, T, out, out_dtype, s);
    case FP_MXFP8: return dequantize_fp_mode<FP_MXFP8>(codes, scales, units, T, out, out_dtype, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_qmv_fp(const void *x, int x_dtype, const uint32_t *codes, const uint8_t *scales,
                         int64_t N, int64_t K, int mode, int T, void *y, hipStream_t s) {
  switch (mode) {
    case FP_MXFP4: return qmv_fp_mode<FP_MXFP4>(x, x_dtype, codes, scales, N, K, T, y, s);
    case FP_NVFP4: return qmv_fp_mode<FP_NVFP4>(x, x_dtype, codes, scales, N, K, T, y, s);
    case FP_MXFP8: return qmv_fp_mode<FP_MXFP8>(x, x_dtype, codes, scales, N, K, T, y, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_mm_fp_rows(const void *x, int x_dtype, int64_t M, const uint32_t *codes,
                             const uint8_t *scales, int64_t N, int64_t K, int mode, int T, void *y,
                             hipStream_t s) {
  switch (mode) {
    case FP_MXFP4: return mm_fp_rows_dtype<FP_MXFP4>(x, x_dtype, M, codes, scales, N, K, T, y, s);
    case FP_NVFP4: return mm_fp_rows_dtype<FP_NVFP4>(x, x_dtype, M, codes, scales, N, K, T, y, s);
    case FP_MXFP8: return mm_fp_rows_dtype<FP_MXFP8>(x, x_dtype, M, codes, scales, N, K, T, y, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gather_mm_fp(const void *x, int x_dtype, int64_t Tk, const uint32_t *codes,
                               const uint8_t *scales, int64_t E, int64_t N, int64_t K,
                               const int32_t *ids, int topk, int mode, int T, void *y,
                               hipStream_t s) {
  switch (mode) {
    case FP_MXFP4:
      return gather_fp_rows_dtype<FP_MXFP4>(x, x_dtype, Tk, codes, scales, E, N, K, ids, topk, T, y, s);
    case FP_NVFP4:
      return gather_fp_rows_dtype<FP_NVFP4>(x, x_dtype, Tk, codes, scales, E, N, K, ids, topk, T, y, s);
    case FP_MXFP8:
      return gather_fp_rows_dtype<FP_MXFP8>(x, x_dtype, Tk, codes, scales, E, N, K, ids, topk, T, y, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace aq
