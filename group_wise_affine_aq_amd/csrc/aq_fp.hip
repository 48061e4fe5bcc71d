// aq_mx.hip -- mxfp4: block-scaled 4-bit float codes, for gfx950.  Quantize,
// dequantize and the M = 1 matrix-vector product.
//
// Format (MLX "Quantization", the paragraph on the newer modes; "Quantizing a
// Model for MLX", "Modes, bits and mixed recipes": groups of 32 weights with
// 4-bit codes and one exponent per group in place of a scale and a bias; the
// pages give no bit layout, so the microscaling (MX) definition of that name
// is taken):
//   a code is an E2M1 float: bit 3 the sign, bits 2..1 an exponent e with
//   bias 1, bit 0 a mantissa m; its value is (1 + m/2) 2^(e-1) for e > 0 and
//   m/2 for e = 0, so codes 0..7 are 0, 0.5, 1, 1.5, 2, 3, 4, 6;
//   codes sit eight to a uint32 word, least significant nibble first (the
//   bitstream of the affine format with 4-bit codes): a group is 4 words;
//   the group's scale is 2^X, stored as the byte X + 127.
// Quantize: X = floor(log2 max|w|) - 2 (2 being the exponent of 6, the
// largest code value), clamped to [-127, 127], and -127 for a group of
// zeros; each weight takes its own sign bit and the magnitude code nearest
// to |w| / 2^X, ties to the even mantissa, saturating at 6.
//
// Every decision is taken on binary32 bit patterns: non-negative floats
// (subnormals included) order as their patterns do, and the thresholds
// between neighbouring code values, times 2^X, are exact binary32 values
// built from their exponent and mantissa fields, so no rounding mode or
// denormal setting enters.  A dequantized value (a code value times 2^X:
// at most two significant bits, exact in bf16 and binary32 down to 2^-128)
// comes from the gfx950 scaled convert, or for the one exponent binary32
// cannot scale by (X = 128) from the same bit construction, then is rounded
// to nearest even into the output type.
//
// The product (decode, M = 1): the E2M1 pairs go through the gfx950
// scaled-convert instruction (v_cvt_scalef32_pk_f16_fp4 / _bf16_fp4, scale
// 1.0: every code value is exact in fp16 and bf16) straight into v_dot2
// against x; each 32-weight chunk's binary32 sum is scaled once by 2^X
// (v_ldexp_f32).  Structure as in the affine decode kernel: x resident in
// registers, a ring of CPL chunk loads per wave that crosses row
// boundaries, finished rows parked in LDS and written in batches.
#include "aq_device.hpp"
#include "aq_internal.hpp"

namespace aq {
namespace {

typedef _Float16 fp4h2v __attribute__((ext_vector_type(2)));
typedef __bf16 fp4b2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const uint8_t gbyte;
typedef uint32_t mxu4 __attribute__((ext_vector_type(4)));

constexpr int kMxRound = 32;  // rows per wave between output flushes

// ---- E2M1 arithmetic on binary32 bit patterns ----------------------------------------

// (1 + mant / 2^23) * 2^e as a binary32 pattern; exact for -129 <= e <= 127
// with mant holding at most two leading bits (the subnormal shift drops
// only zeros)
__device__ __forceinline__ uint32_t pow2_bits(uint32_t mant, int e) {
  const int E = e + 127;
  if (E >= 1) return ((uint32_t)E << 23) | mant;
  return (0x800000u | mant) >> (1 - E);
}

// the magnitude code (0..7) of a weight whose |w| has pattern a, given the
// patterns of the seven midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 times
// 2^X: a tie goes to the even mantissa, i.e. up across the midpoints into
// codes 2, 4, 6 and down across the others
__device__ __forceinline__ uint32_t e2m1_code(uint32_t a, const uint32_t (&t)[7]) {
  return (uint32_t)(a > t[0]) + (uint32_t)(a >= t[1]) + (uint32_t)(a > t[2]) +
         (uint32_t)(a >= t[3]) + (uint32_t)(a > t[4]) + (uint32_t)(a >= t[5]) +
         (uint32_t)(a > t[6]);
}

// binary32 pattern of code c (sign in bit 3) times 2^X, X in [-127, 128];
// +-inf where that exceeds the binary32 range (X = 128, or 127 with |c| > 1.5).
// Written with selects only: every lane takes the same path.
__device__ __forceinline__ uint32_t e2m1_value_bits(uint32_t c, int X) {
  const uint32_t sign = (c & 8u) << 28, m = c & 7u;
  // m >= 1: value (1 + mb/2) 2^e with e = (m >> 1) - 1 and mb = m & 1 from
  // m = 2 on (code 1 is 0.5 = 2^-1)
  const uint32_t mb = m >= 2u ? (m & 1u) << 22 : 0u;
  const int E = (int)(m >> 1) - 1 + X + 127;  // biased exponent, in [-1, 257]
  const uint32_t normal = ((uint32_t)E << 23) | mb;
  const uint32_t sub = (0x800000u | mb) >> ((uint32_t)(1 - E) & 31u);  // used for E in {-1, 0}
  uint32_t r = E >= 255 ? 0x7F800000u : (E >= 1 ? normal : sub);
  r = m == 0u ? 0u : r;
  return sign | r;
}

// ---- quantize and dequantize: one thread per word (8 codes) ----------------------------
// A workgroup takes kMxUnroll * 256 consecutive words per pass, word
// base + u * 256 + thread, so every load and store instruction of a wave
// covers one contiguous span and each thread has kMxUnroll words in flight.
// Four consecutive words are one group: the four lanes of a DPP quad.
constexpr int kMxUnroll = 4;

__device__ __forceinline__ uint32_t quad_max(uint32_t a) {
  uint32_t b = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
  a = a > b ? a : b;
  b = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x4E, 0xF, 0xF, false);           // [2,3,0,1]
  return a > b ? a : b;
}

template <int WDT>
__global__ __launch_bounds__(256) void quantize_mx_kernel(const void *__restrict__ w,
                                                          int64_t words,
                                                          uint32_t *__restrict__ codes,
                                                          uint8_t *__restrict__ scales) {
  // midpoints as (mantissa field, exponent)
  constexpr uint32_t kMant[7] = {0u, 0x400000u, 0x200000u, 0x600000u, 0x200000u, 0x600000u,
                                 0x200000u};
  constexpr int kExp[7] = {-2, -1, 0, 0, 1, 1, 2};
  const int64_t pass = (int64_t)gridDim.x * (256 * kMxUnroll);
  for (int64_t base = (int64_t)blockIdx.x * (256 * kMxUnroll); base < words; base += pass) {
    float v[kMxUnroll][8];
#pragma unroll
    for (int u = 0; u < kMxUnroll; ++u) {
      const int64_t t = base + u * 256 + threadIdx.x;
      if (t < words) load8<WDT>(w, t * 8, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kMxUnroll; ++u) {
      const int64_t t = base + u * 256 + threadIdx.x;
      if (t >= words) break;  // words is a multiple of 4: quads leave together
      uint32_t amax = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t a = __builtin_bit_cast(uint32_t, v[u][i]) & 0x7FFFFFFFu;
        amax = a > amax ? a : amax;
      }
      amax = quad_max(amax);
      // floor(log2 max) = biased exponent - 127 for a normal maximum; a zero
      // or subnormal maximum (biased exponent 0) and the exponent 1 both clamp
      const int eb = (int)(amax >> 23);
      const int X = (eb < 2 ? 2 : eb) - 129;
      uint32_t th[7];
#pragma unroll
      for (int k = 0; k < 7; ++k) th[k] = pow2_bits(kMant[k], kExp[k] + X);
      uint32_t q = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t b = __builtin_bit_cast(uint32_t, v[u][i]);
        q |= (e2m1_code(b & 0x7FFFFFFFu, th) | ((b >> 31) << 3)) << (4 * i);
      }
      codes[t] = q;
      if ((threadIdx.x & 3) == 0) scales[t >> 2] = (uint8_t)(X + 127);
    }
  }
}

template <int OUT>
__global__ __launch_bounds__(256) void dequantize_mx_kernel(const uint32_t *__restrict__ codes,
                                                            const uint8_t *__restrict__ scales,
                                                            int64_t words, void *__restrict__ out) {
  const int64_t pass = (int64_t)gridDim.x * (256 * kMxUnroll);
  for (int64_t base = (int64_t)blockIdx.x * (256 * kMxUnroll); base < words; base += pass) {
    uint32_t wd[kMxUnroll], sc[kMxUnroll];
#pragma unroll
    for (int u = 0; u < kMxUnroll; ++u) {
      const int64_t t = base + u * 256 + threadIdx.x;
      if (t < words) {
        wd[u] = codes[t];
        sc[u] = scales[t >> 2];
      }
    }
#pragma unroll
    for (int u = 0; u < kMxUnroll; ++u) {
      const int64_t t = base + u * 256 + threadIdx.x;
      if (t >= words) break;
      const int X = (int)sc[u] - 127;
      // Every code value times 2^X has at most two significant bits, so it
      // is exact in bf16 (subnormals down to 2^-128 included) and binary32
      // is its upper half.  The scaled convert (code pair * 2^X, the scale
      // 2^X given as a binary32) returns exactly that pair, +-inf past the
      // range, for X up to 127, checked on the MI355X for every code pair
      // and exponent.  X = 128 (scale byte 255) has no binary32 scale: those
      // groups take the bit construction.
      const float scale = __builtin_bit_cast(float, (uint32_t)(X + 127) << 23);
      uint32_t pr[4];
      pr[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[u], scale, 0));
      pr[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[u], scale, 1));
      pr[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[u], scale, 2));
      pr[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[u], scale, 3));
      uint32_t f[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[2 * j] = pr[j] << 16;
        f[2 * j + 1] = pr[j] & 0xFFFF0000u;
      }
      const bool edge = X > 127;
      if (edge) {
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = e2m1_value_bits((wd[u] >> (4 * j)) & 15u, X);
      }
      if constexpr (OUT == X_F32) {
        uint4 *o = reinterpret_cast<uint4 *>(out) + 2 * t;
        o[0] = make_uint4(f[0], f[1], f[2], f[3]);
        o[1] = make_uint4(f[4], f[5], f[6], f[7]);
      } else if constexpr (OUT == X_F16) {
        uint32_t h[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          h[j] = (uint32_t)f32_to_f16_rne(__builtin_bit_cast(float, f[2 * j])) |
                 ((uint32_t)f32_to_f16_rne(__builtin_bit_cast(float, f[2 * j + 1])) << 16);
        reinterpret_cast<uint4 *>(out)[t] = make_uint4(h[0], h[1], h[2], h[3]);
      } else {
        if (edge) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            pr[j] = (uint32_t)f32_to_bf16_rne(__builtin_bit_cast(float, f[2 * j])) |
                    ((uint32_t)f32_to_bf16_rne(__builtin_bit_cast(float, f[2 * j + 1])) << 16);
        }
        reinterpret_cast<uint4 *>(out)[t] = make_uint4(pr[0], pr[1], pr[2], pr[3]);
      }
    }
  }
}

// ---- the M = 1 product -------------------------------------------------------------

// sum over the 8 codes of word w of x * code value, x given as 4 packed pairs
// in natural order (the convert's byte select b yields codes 2b and 2b + 1)
__device__ __forceinline__ float fp4_word_dot(f16_t, uint32_t w, const uint32_t *xp, float acc) {
  acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0),
                               __builtin_bit_cast(fp4h2v, xp[0]), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1),
                               __builtin_bit_cast(fp4h2v, xp[1]), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2),
                               __builtin_bit_cast(fp4h2v, xp[2]), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3),
                               __builtin_bit_cast(fp4h2v, xp[3]), acc, false);
  return acc;
}
__device__ __forceinline__ float fp4_word_dot(bf16_t, uint32_t w, const uint32_t *xp, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0),
                                        __builtin_bit_cast(fp4b2v, xp[0]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1),
                                        __builtin_bit_cast(fp4b2v, xp[1]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2),
                                        __builtin_bit_cast(fp4b2v, xp[2]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3),
                                        __builtin_bit_cast(fp4b2v, xp[3]), acc, false);
  return acc;
}

// a wave-uniform global pointer (its address goes to scalar registers)
__device__ __forceinline__ gbyte *wave_ptr(const void *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<gbyte *>(((uint64_t)hi << 32) | lo);
}

// The decode kernel for K <= 64 * 32 * CPL.  Lane l owns chunks l, l + 64,
// ... of every row (a chunk = 32 codes = 16 bytes, so each load instruction
// of a wave reads 1 KB of one row) and keeps the matching x chunks in
// registers.  Rows are dealt to waves round-robin (row gw, gw + TW, ...);
// the ring holds the D = CPL * UD chunk loads of UD rows and each slot is
// reloaded with the next rows' chunk as soon as it is consumed.
template <typename XT, int CPL, int UD, int W>
__global__ __launch_bounds__(64 * W) void qmv1_mx_kernel(const uint16_t *__restrict__ x,
                                                         const uint32_t *__restrict__ codes,
                                                         const uint8_t *__restrict__ scales,
                                                         int64_t N, int64_t K,
                                                         uint16_t *__restrict__ y) {
  constexpr int D = CPL * UD, CP = 64 * CPL;
  constexpr int XS = (4 * CP + 64 * W - 1) / (64 * W);  // x loads per thread
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nch = (int)(K >> 5);
  const int64_t TW = (int64_t)gridDim.x * W, gw = (int64_t)blockIdx.x * W + wave;
  const int nunits = gw < N ? (int)((N - 1 - gw) / TW + 1) : 0;
  // x as 16-byte quarters of chunks, quarter-major (quarter j of chunk c at
  // j * CP + c: 64 lanes reading one quarter hit consecutive addresses);
  // chunks past the row are zero
  uint4 *xl = reinterpret_cast<uint4 *>(smem);
  uint16_t *obuf = reinterpret_cast<uint16_t *>(smem + (size_t)CP * 64) + (size_t)wave * kMxRound;

  mxu4 cb[D];
  uint32_t sb[D];
  auto load = [&](int d, int64_t row) {
    const int c0 = (d % CPL) * 64 + lane;
    const uint32_t c = (uint32_t)(c0 < nch ? c0 : nch - 1);  // padding lanes re-read the last
    gbyte *rc = wave_ptr(codes + row * (K >> 3));
    gbyte *rs = wave_ptr(scales + row * (int64_t)nch);
    cb[d] = *reinterpret_cast<__attribute__((address_space(1))) const mxu4 *>(rc + c * 16u);
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
    const int nu = nunits < kMxRound ? nunits : kMxRound;
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

  for (int u0 = 0; u0 < nunits; u0 += kMxRound) {
    const int nu = nunits - u0 < kMxRound ? nunits - u0 : kMxRound;
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
      float s = 0.f;
      s = fp4_word_dot(XT{}, cb[d][0], &xv[p][0], s);
      s = fp4_word_dot(XT{}, cb[d][1], &xv[p][4], s);
      s = fp4_word_dot(XT{}, cb[d][2], &xv[p][8], s);
      s = fp4_word_dot(XT{}, cb[d][3], &xv[p][12], s);
      acc += __builtin_ldexpf(s, (int)sb[d] - 127);
      if (p == CPL - 1) {
        const float v = wave_sum(acc);
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
template <typename XT, int W>
__global__ __launch_bounds__(64 * W) void qmv1_mx_lds_kernel(const uint16_t *__restrict__ x,
                                                             const uint32_t *__restrict__ codes,
                                                             const uint8_t *__restrict__ scales,
                                                             int64_t N, int64_t K,
                                                             uint16_t *__restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nch = (int)(K >> 5);
  uint4 *xl = reinterpret_cast<uint4 *>(smem);  // chunk c at xl[4 c .. 4 c + 3]
  const uint4 *xg = reinterpret_cast<const uint4 *>(x);
  for (int e = (int)threadIdx.x; e < 4 * nch; e += 64 * W) xl[e] = xg[e];
  __syncthreads();
  const int64_t TW = (int64_t)gridDim.x * W;
  for (int64_t row = (int64_t)blockIdx.x * W + wave; row < N; row += TW) {
    gbyte *rc = wave_ptr(codes + row * (K >> 3));
    gbyte *rs = wave_ptr(scales + row * (int64_t)nch);
    float acc = 0.f;
#pragma unroll 4
    for (int c = lane; c < nch; c += 64) {
      const mxu4 w = *reinterpret_cast<__attribute__((address_space(1))) const mxu4 *>(
          rc + (uint32_t)c * 16u);
      const int X = (int)rs[c] - 127;
      uint32_t xp[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 v = xl[4 * c + j];
        xp[4 * j] = v.x; xp[4 * j + 1] = v.y; xp[4 * j + 2] = v.z; xp[4 * j + 3] = v.w;
      }
      float s = 0.f;
      s = fp4_word_dot(XT{}, w[0], &xp[0], s);
      s = fp4_word_dot(XT{}, w[1], &xp[4], s);
      s = fp4_word_dot(XT{}, w[2], &xp[8], s);
      s = fp4_word_dot(XT{}, w[3], &xp[12], s);
      acc += __builtin_ldexpf(s, X);
    }
    const float v = wave_sum(acc);
    if (lane == 0) y[row] = xtraits<XT>::from_f32(v);
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

template <typename XT, int CPL, int UD, int W>
hipError_t qmv1_mx_launch(const void *x, const uint32_t *codes, const uint8_t *scales, int64_t N,
                          int64_t K, void *y, int wpc, hipStream_t s) {
  auto kern = qmv1_mx_kernel<XT, CPL, UD, W>;
  const size_t lds = (size_t)64 * CPL * 64 + (size_t)W * kMxRound * 2;
  static int per_cu = 0;  // resident workgroups per CU for this instantiation
  if (per_cu == 0) per_cu = resident_blocks(kern, 64 * W, lds);
  const int64_t want = (N + W - 1) / W;
  const int64_t cap = (int64_t)device_cus() * (wpc > 0 && wpc < per_cu ? wpc : per_cu);
  const dim3 grid((unsigned)(want < cap ? want : cap));
  hipLaunchKernelGGL(kern, grid, dim3(64 * W), lds, s, (const uint16_t *)x, codes, scales, N, K,
                     (uint16_t *)y);
  return hipGetLastError();
}

template <typename XT>
hipError_t qmv1_mx_lds_launch(const void *x, const uint32_t *codes, const uint8_t *scales,
                              int64_t N, int64_t K, void *y, hipStream_t s) {
  constexpr int W = 8;
  auto kern = qmv1_mx_lds_kernel<XT, W>;
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
  hipLaunchKernelGGL(kern, grid, dim3(64 * W), lds, s, (const uint16_t *)x, codes, scales, N, K,
                     (uint16_t *)y);
  return hipGetLastError();
}

template <typename XT>
hipError_t qmv_mx_dispatch(const void *x, const uint32_t *codes, const uint8_t *scales, int64_t N,
                           int64_t K, void *y, hipStream_t s) {
  int cpl, ud, w, wpc;
  qmv1_mx_shape(N, K, cpl, ud, w, wpc);
#define AQ_MX1(C, U, WW) return qmv1_mx_launch<XT, C, U, WW>(x, codes, scales, N, K, y, wpc, s)
  switch (cpl) {
    case 0: return qmv1_mx_lds_launch<XT>(x, codes, scales, N, K, y, s);
    case 1: AQ_MX1(1, 4, 4);
    case 2:
      if (w == 16) AQ_MX1(2, 1, 16);
      if (ud == 1) AQ_MX1(2, 1, 4);
      AQ_MX1(2, 2, 4);
    case 3: AQ_MX1(3, 1, 4);
    case 4: AQ_MX1(4, 1, 4);
    case 5: AQ_MX1(5, 1, 8);
    case 6: AQ_MX1(6, 1, 8);
    case 7: AQ_MX1(7, 1, 8);
    case 8: AQ_MX1(8, 1, 8);
  }
#undef AQ_MX1
  return hipErrorInvalidValue;
}

// grid for the quantize / dequantize loops over words: kMxUnroll words per
// thread and pass, at most 2^22 workgroups (then several passes)
dim3 word_grid(int64_t words) {
  const int64_t b = (words + 256 * kMxUnroll - 1) / (256 * kMxUnroll);
  return dim3((unsigned)(b < (1 << 22) ? b : (1 << 22)));
}

}  // namespace

// M = 1 launch shape: the affine decode kernel's (x chunks per lane, rows in
// flight, waves per workgroup, workgroups per CU), the mxfp4 rows being
// slightly shorter than affine 4-bit rows at G = 64 (4.25 against 4.5 bits
// per weight); cpl = 0 selects the LDS kernel for K > 16384.
void qmv1_mx_shape(int64_t N, int64_t K, int &cpl, int &ud, int &w, int &wpc) {
  int sl;
  if (K > 8 * 2048) {
    cpl = 0;
    ud = 1;
    w = 8;
    wpc = 0;
    return;
  }
  qmv1_shape(N, K, 32, cpl, ud, w, sl, wpc);
}

hipError_t launch_quantize_mx(const void *w, int w_dtype, int64_t N, int64_t K, uint32_t *codes,
                              uint8_t *scales, hipStream_t s) {
  const int64_t words = N * (K / 8);
  const dim3 grid = word_grid(words);
  switch (w_dtype) {
    case X_F32:
      hipLaunchKernelGGL(quantize_mx_kernel<X_F32>, grid, dim3(256), 0, s, w, words, codes, scales);
      break;
    case X_F16:
      hipLaunchKernelGGL(quantize_mx_kernel<X_F16>, grid, dim3(256), 0, s, w, words, codes, scales);
      break;
    case X_BF16:
      hipLaunchKernelGGL(quantize_mx_kernel<X_BF16>, grid, dim3(256), 0, s, w, words, codes,
                         scales);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dequantize_mx(const uint32_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                                void *out, int out_dtype, hipStream_t s) {
  const int64_t words = N * (K / 8);
  const dim3 grid = word_grid(words);
  switch (out_dtype) {
    case X_F32:
      hipLaunchKernelGGL(dequantize_mx_kernel<X_F32>, grid, dim3(256), 0, s, codes, scales, words,
                         out);
      break;
    case X_F16:
      hipLaunchKernelGGL(dequantize_mx_kernel<X_F16>, grid, dim3(256), 0, s, codes, scales, words,
                         out);
      break;
    case X_BF16:
      hipLaunchKernelGGL(dequantize_mx_kernel<X_BF16>, grid, dim3(256), 0, s, codes, scales, words,
                         out);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_qmv_mx(const void *x, int x_dtype, const uint32_t *codes, const uint8_t *scales,
                         int64_t N, int64_t K, void *y, hipStream_t s) {
  if (x_dtype == X_F16) return qmv_mx_dispatch<f16_t>(x, codes, scales, N, K, y, s);
  if (x_dtype == X_BF16) return qmv_mx_dispatch<bf16_t>(x, codes, scales, N, K, y, s);
  return hipErrorInvalidValue;
}

}  // namespace aq
