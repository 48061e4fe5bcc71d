// aq_quant.hip -- quantize and dequantize kernels for gfx950.
//
// Quantize ("Quantizing a Model for MLX", "What MLX quantization stores":
// per-group scale and offset; "mlx-gptq", "How it works": the grid spans the
// group's min-max range; round-to-nearest): per group of G weights along a
// row,
//   b = largest fp16 <= min(w)            (bias never exceeds a member)
//   s = smallest fp16 >= 0 with b + L*s >= max(w),   L = 2^bits - 1
//   q = argmin_q |w - (b + q*s)|, ties to even q (q = 0 if s == 0)
// Every decision is an exact comparison: b + L*s and the midpoints
// b + (j+1/2)*s are multiples of 2^-25 below 2^26, exact in binary64, and the
// binary32 weights are exact in binary64.  Approximate binary32 arithmetic
// only proposes candidates that the exact tests then correct by one step.
//
// Range search ("mlx-gptq", "How it works", the --mse option: a group may be
// quantized over a range narrower than its min-max span, trading error on its
// outermost members for a finer step on the others): candidate i < steps
// moves both ends of [min, max] inwards by d = (max - min) * (i / 200)
// (binary64, no contraction), keeping the centred fraction (100 - i) / 100
// of the width, so every candidate lies inside [min, max]; each is quantized
// by the rules above and the least binary64 sum of squared errors wins, an
// equal one keeping the wider candidate.
//
// Integer zero point ("mlx-gptq", "On NVIDIA: the same recipe in AWQ format",
// --zero-point int: every group's offset is a whole number of steps, for a
// lossless conversion to a layout that stores integer zero points): the zero
// point z is an integer in [0, 2^bits - 1], so every grid -z*s + q*s holds 0;
// s is the smallest fp16 for which some such z has -z*s <= min,
// (2^bits - 1 - z)*s >= max and -z*s exactly an fp16 value, z the smallest
// one for that s, bias = -z*s, codes as above.  Every test is exact: z*s has
// at most 19 significant bits.
//
// Dequantize ("Tutorial 10: Quantization", s.3/s.7): q*s + b in binary32
// (one rounding, the product is exact), then round-to-nearest-even to the
// output type.
//
// Thread mapping.  Quantize: one thread per 8 consecutive weights; their 8
// codes fill exactly `bits` bytes at byte offset 8k/8*bits of the row, so
// every thread stores whole bytes and no two threads share a byte.  A group
// is G/8 adjacent lanes, reduced with lane shuffles.  Dequantize: one thread
// per 32-code chunk (`bits` words); a wave's 64 output chunks are one
// contiguous span, stored through LDS in lane-contiguous 16-byte units.
#include "aq_device.hpp"
#include "aq_internal.hpp"

namespace aq {
namespace {

__device__ __forceinline__ double h2d(uint16_t h) { return (double)f16_to_f32(h); }

// next binary16 pattern towards -infinity
__device__ __forceinline__ uint16_t f16_next_down(uint16_t h) {
  if (h == 0) return 0x8001u;
  return (h & 0x8000u) ? (uint16_t)(h + 1) : (uint16_t)(h - 1);
}

// largest binary16 value <= f; -0 is returned as +0
__device__ __forceinline__ uint16_t f16_round_down(float f) {
  uint16_t h = f32_to_f16_rne(f);  // nearest; at most one step above f
  if (f16_to_f32(h) > f) h = f16_next_down(h);
  return h == 0x8000u ? (uint16_t)0 : h;
}

// the same for a binary64 value: rounding to binary32 and then to binary16
// preserves the order against every binary16 value, so the result is again
// the answer or one step above it
__device__ __forceinline__ uint16_t f16_round_down_d(double x) {
  uint16_t h = f32_to_f16_rne((float)x);
  if (h2d(h) > x) h = f16_next_down(h);
  return h == 0x8000u ? (uint16_t)0 : h;
}

// smallest binary16 s >= 0 with b + L*s >= top (exact test in binary64)
__device__ __forceinline__ uint16_t f16_scale_up(double b, double top, int L) {
  if (b >= top) return 0;
  const float t = (float)(top - b) / (float)L;  // candidate, within a step of the answer
  uint16_t s = f32_to_f16_rne(t);
  if (s > 0x7BFFu) s = 0x7BFFu;
#pragma unroll
  for (int it = 0; it < 3; ++it)
    if (s < 0x7BFFu && b + L * h2d(s) < top) ++s;
#pragma unroll
  for (int it = 0; it < 3; ++it)
    if (s > 0 && b + L * h2d((uint16_t)(s - 1)) >= top) --s;
  return s;
}

// nearest grid index, ties to even.  mid(j) = b + (j + 1/2) s separates j, j+1.
// The binary32 estimate t = (w - b) * rcp(s) of the real (w - b) / s has a
// relative error below 2^-22 (one rounding in the subtraction, at most one
// unit in the last place in v_rcp_f32, one in the product), so below 2^-14
// absolutely for t <= 255: when t is farther than 2^-10 from every
// half-integer, rint(t) clamped to [0, L] is already the answer; only the
// rest take the exact binary64 tests.
__device__ __forceinline__ uint32_t nearest_code(float w, double b, double s, float bf, float rs,
                                                 int L) {
  if (s == 0.0) return 0;
  const float t = (w - bf) * rs;
  const float r = __builtin_rintf(t);
  int q = (int)r;  // candidate, within one of the answer (saturating conversion)
  q = q < 0 ? 0 : (q > L ? L : q);
  if (__builtin_fabsf(t - r) <= 0.5f - 0x1p-10f) return (uint32_t)q;
  const double wd = (double)w;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    if (q > 0) {
      const double mid = b + ((double)q - 0.5) * s;
      if (wd < mid || (wd == mid && (q & 1))) --q;
    }
  }
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    if (q < L) {
      const double mid = b + ((double)q + 0.5) * s;
      if (wd > mid || (wd == mid && (q & 1))) ++q;
    }
  }
  return (uint32_t)q;
}

// One thread per 32-weight chunk: a group is G/32 adjacent lanes (1, 2 or
// 4), reduced by lane shuffles; the thread writes its chunk's BITS words of
// codes whole.  (With 8 weights per thread, the group search and the
// shuffles ran once per 8 weights instead of once per 32: 277-307 us
// against 208 us on a 28672 x 8192 fp32 matrix at 4/64, bit-identical.)
template <int WDT, int BITS>
__global__ __launch_bounds__(256) void quantize_kernel(const void *__restrict__ w, int64_t N,
                                                       int64_t K, int G,
                                                       uint32_t *__restrict__ codes,
                                                       uint16_t *__restrict__ scales,
                                                       uint16_t *__restrict__ biases) {
  const int64_t cpr = K >> 5;  // chunks per row
  const int64_t total = N * cpr;
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool active = idx < total;
  if (!active) idx = total - 1;  // whole groups are inactive together; keep loads in bounds
  const int64_t n = idx / cpr, o = idx - n * cpr;

  float v[32];
  load32<WDT>(w, n * K + o * 32, v);
  float lo = v[0], hi = v[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) { lo = fminf(lo, v[i]); hi = fmaxf(hi, v[i]); }
  const int lanes = G >> 5;
  for (int d = 1; d < lanes; d <<= 1) {
    lo = fminf(lo, __shfl_xor(lo, d));
    hi = fmaxf(hi, __shfl_xor(hi, d));
  }
  constexpr int L = (1 << BITS) - 1;
  const uint16_t b16 = f16_round_down(lo);
  const double b = h2d(b16);
  const uint16_t s16 = f16_scale_up(b, (double)hi, L);
  const double s = h2d(s16);
  const float bf = (float)b;
  const float rs = s16 ? __builtin_amdgcn_rcpf((float)s) : 0.f;

  // code i at bit i * BITS of the chunk's LSB-first bitstream
  uint32_t words[BITS];
#pragma unroll
  for (int j = 0; j < BITS; ++j) words[j] = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t q = nearest_code(v[i], b, s, bf, rs, L);
    const int bit = i * BITS, wi = bit >> 5, sh = bit & 31;
    words[wi] |= q << sh;
    if (sh + BITS > 32) words[wi + 1] |= q >> (32 - sh);
  }

  if (!active) return;
  if ((o & (lanes - 1)) == 0) {
    const int64_t gi = n * (K / G) + (o * 32) / G;
    scales[gi] = s16;
    biases[gi] = b16;
  }
  uint32_t *dst = codes + n * (K * BITS / 32) + o * BITS;  // 4 BITS bytes, 4-byte aligned
  if constexpr (BITS % 4 == 0) {
#pragma unroll
    for (int j = 0; j < BITS; j += 4)
      *reinterpret_cast<uint4 *>(dst + j) = make_uint4(words[j], words[j + 1], words[j + 2], words[j + 3]);
  } else if constexpr (BITS % 2 == 0) {
#pragma unroll
    for (int j = 0; j < BITS; j += 2) *reinterpret_cast<uint2 *>(dst + j) = make_uint2(words[j], words[j + 1]);
  } else {
#pragma unroll
    for (int j = 0; j < BITS; ++j) dst[j] = words[j];
  }
}

// The range search: the thread mapping of quantize_kernel; every lane of a
// group evaluates every candidate (its 8 codes and their squared errors, the
// group sum by a butterfly, whose result is the same bits on every lane) and
// keeps the best.
template <int WDT, int BITS>
__global__ __launch_bounds__(256) void quantize_mse_kernel(const void *__restrict__ w, int64_t N,
                                                           int64_t K, int G, int steps,
                                                           uint32_t *__restrict__ codes,
                                                           uint16_t *__restrict__ scales,
                                                           uint16_t *__restrict__ biases) {
  // the thread mapping of quantize_kernel: one 32-weight chunk per thread
  const int64_t cpr = K >> 5;
  const int64_t total = N * cpr;
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool active = idx < total;
  if (!active) idx = total - 1;
  const int64_t n = idx / cpr, o = idx - n * cpr;

  float v[32];
  load32<WDT>(w, n * K + o * 32, v);
  float lo = v[0], hi = v[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) { lo = fminf(lo, v[i]); hi = fmaxf(hi, v[i]); }
  const int lanes = G >> 5;
  for (int d = 1; d < lanes; d <<= 1) {
    lo = fminf(lo, __shfl_xor(lo, d));
    hi = fmaxf(hi, __shfl_xor(hi, d));
  }
  constexpr int L = (1 << BITS) - 1;
  double best = __builtin_inf();
  uint16_t best_b = 0, best_s = 0;
  uint32_t best_w[BITS];
#pragma unroll
  for (int j = 0; j < BITS; ++j) best_w[j] = 0;
  const double width = (double)hi - (double)lo;
  for (int i = 0; i < steps; ++i) {
    double clo, chi;
    {
#pragma clang fp contract(off)
      const double d = width * ((double)i / 200.0);
      clo = (double)lo + d;
      chi = (double)hi - d;
    }
    const uint16_t b16 = f16_round_down_d(clo);
    const double b = h2d(b16);
    const uint16_t s16 = f16_scale_up(b, chi, L);
    const double s = h2d(s16);
    const float bf = (float)b;
    const float rs = s16 ? __builtin_amdgcn_rcpf((float)s) : 0.f;
    uint32_t words[BITS];
#pragma unroll
    for (int j = 0; j < BITS; ++j) words[j] = 0;
    double e = 0.0;
    {
#pragma clang fp contract(off)
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const uint32_t q = nearest_code(v[k], b, s, bf, rs, L);
        const int bit = k * BITS, wi = bit >> 5, sh = bit & 31;
        words[wi] |= q << sh;
        if (sh + BITS > 32) words[wi + 1] |= q >> (32 - sh);
        const double dv = (double)v[k] - (b + (double)q * s);
        e = e + dv * dv;
      }
      for (int d = 1; d < lanes; d <<= 1) e = e + __shfl_xor(e, d);
    }
    if (e < best) {
      best = e;
      best_b = b16;
      best_s = s16;
#pragma unroll
      for (int j = 0; j < BITS; ++j) best_w[j] = words[j];
    }
  }

  if (!active) return;
  if ((o & (lanes - 1)) == 0) {
    const int64_t gi = n * (K / G) + (o * 32) / G;
    scales[gi] = best_s;
    biases[gi] = best_b;
  }
  uint32_t *dst = codes + n * (K * BITS / 32) + o * BITS;
#pragma unroll
  for (int j = 0; j < BITS; ++j) dst[j] = best_w[j];
}

// Smallest u in [0, cap] with u s >= t (t >= 0, s > 0), or cap + 1 when
// cap s < t.  u <= 255 and s an fp16 value make every product u s exact in
// binary32, so each comparison is exact; the reciprocal only seeds the walk.
__device__ __forceinline__ int ceil_steps(float t, float s, int cap) {
  if ((float)cap * s < t) return cap + 1;
  int u = (int)__builtin_ceilf(t * __builtin_amdgcn_rcpf(s));
  u = u < 0 ? 0 : (u > cap ? cap : u);
  while (u > 0 && (float)(u - 1) * s >= t) --u;
  while ((float)u * s < t) ++u;
  return u;
}

// The smallest zero point admitted by the nonzero scale pattern p for a group
// in [-nlo, hi0] (nlo, hi0 >= 0): the least integer z with z s >= nlo,
// (L - z) s >= hi0 and z s an fp16 value (exact in binary32: z <= 255), or -1.
__device__ __forceinline__ int zero_point_at(uint16_t p, float nlo, float hi0, int L) {
  const float sv = f16_to_f32(p);
  const int zmin = ceil_steps(nlo, sv, L);
  const int zmax = L - ceil_steps(hi0, sv, L);
  for (int zz = zmin; zz <= zmax; ++zz) {
    const float bottom = (float)zz * sv;
    if (f16_to_f32(f32_to_f16_rne(bottom)) == bottom) return zz;
  }
  return -1;
}

// The zero-point search for one group with members in [lo, hi]: the smallest
// scale pattern admitting a zero point, and that zero point.  Scales start at
// the smallest one whose L steps span [min(lo, 0), max(hi, 0)] (a grid holding
// 0 cannot be narrower) and go up one pattern at a time; the `lanes` lanes of
// the group test consecutive patterns side by side (lane li tests base + li)
// and the least lane offset with an answer wins.
__device__ __forceinline__ uint16_t zero_point_scale(float lo, float hi, int L, int lanes, int li,
                                                     int &z) {
  const float nlo = lo < 0.f ? -lo : 0.f, hi0 = hi > 0.f ? hi : 0.f;
  const uint16_t p0 = f16_scale_up(lo < 0.f ? (double)lo : 0.0, (double)hi0, L);
  z = 0;
  if (p0 == 0) return 0;  // only an all-zero group: z = 0, s = 0
  for (uint32_t base = p0; base <= 0x7BFFu; base += (uint32_t)lanes) {
    const uint32_t p = base + (uint32_t)li;
    const int zz = p <= 0x7BFFu ? zero_point_at((uint16_t)p, nlo, hi0, L) : -1;
    uint32_t key = zz >= 0 ? ((uint32_t)li << 8) | (uint32_t)zz : 0xFFFFFFFFu;
    for (int d = 1; d < lanes; d <<= 1) {
      const uint32_t other = (uint32_t)__shfl_xor((int)key, d);
      key = other < key ? other : key;
    }
    if (key != 0xFFFFFFFFu) {
      z = (int)(key & 0xFFu);
      return (uint16_t)(base + (key >> 8));
    }
  }
  return 0x7BFFu;  // outside the documented precondition
}

// Integer-zero-point quantize: the thread mapping of quantize_kernel; the
// lanes of a group share its scale search.
template <int WDT, int BITS>
__global__ __launch_bounds__(256) void quantize_zp_kernel(const void *__restrict__ w, int64_t N,
                                                          int64_t K, int G,
                                                          uint32_t *__restrict__ codes,
                                                          uint16_t *__restrict__ scales,
                                                          uint16_t *__restrict__ biases,
                                                          uint8_t *__restrict__ zeros) {
  const int64_t opr = K >> 3;
  const int64_t total = N * opr;
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool active = idx < total;
  if (!active) idx = total - 1;
  const int64_t n = idx / opr, o = idx - n * opr;

  float v[8];
  load8<WDT>(w, n * K + o * 8, v);
  float lo = v[0], hi = v[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) { lo = fminf(lo, v[i]); hi = fmaxf(hi, v[i]); }
  const int lanes = G >> 3;
  for (int d = 1; d < lanes; d <<= 1) {
    lo = fminf(lo, __shfl_xor(lo, d));
    hi = fmaxf(hi, __shfl_xor(hi, d));
  }
  constexpr int L = (1 << BITS) - 1;
  int z = 0;
  const uint16_t s16 = zero_point_scale(lo, hi, L, lanes, (int)threadIdx.x & (lanes - 1), z);
  const double s = h2d(s16);
  const uint16_t b16 = z == 0 ? (uint16_t)0 : f32_to_f16_rne(-((float)z * (float)s));
  const double b = h2d(b16);
  const float bf = (float)b;
  const float rs = s16 ? __builtin_amdgcn_rcpf((float)s) : 0.f;
  uint64_t packed = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    packed |= (uint64_t)nearest_code(v[i], b, s, bf, rs, L) << (BITS * i);

  if (!active) return;
  if ((o & (lanes - 1)) == 0) {
    const int64_t gi = n * (K / G) + (o * 8) / G;
    scales[gi] = s16;
    biases[gi] = b16;
    if (zeros) zeros[gi] = (uint8_t)z;
  }
  uint8_t *dst = reinterpret_cast<uint8_t *>(codes + n * (K * BITS / 32)) + o * BITS;
#pragma unroll
  for (int j = 0; j < BITS; ++j) dst[j] = (uint8_t)(packed >> (8 * j));
}

// two binary32 values rounded to nearest even into fp16 or bf16 and packed
// (v_cvt_pk_bf16_f32 for bf16; the values here are finite, where it agrees
// bit for bit with the integer rounding used elsewhere)
template <int ODT>
__device__ __forceinline__ uint32_t pack_rne(float lo, float hi) {
  if constexpr (ODT == X_BF16) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const b2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
}

// One thread per 32-code chunk of an output row.  With GATHER (quantized
// embedding, "Tutorial 10: Quantization", s.6) output row t is table row
// ids[t] (N table rows, T output rows); an id outside [0, N) gives a zero row.
template <int BITS, int ODT, bool GATHER>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint32_t *__restrict__ codes,
                                                         const uint16_t *__restrict__ scales,
                                                         const uint16_t *__restrict__ biases,
                                                         int64_t N, int64_t K, int G,
                                                         const int32_t *__restrict__ ids, int64_t T,
                                                         void *__restrict__ out) {
  // Output chunk idx is elements [32 idx, 32 idx + 32) (row t of the output
  // is row t of the table, or the t-th looked-up row), so a wave's output is
  // one contiguous span: each lane's chunk goes through LDS, and the wave
  // stores the span with consecutive 16-byte units per lane (8 cache lines
  // per store instruction instead of 32 at one chunk per lane).
  constexpr int NQ = ODT == X_F32 ? 8 : 4;  // 16-byte units per chunk
  __shared__ __attribute__((aligned(16))) uint4 stage[256 * NQ];
  const int64_t cpr = K >> 5;  // chunks per row
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (GATHER ? T : N) * cpr;
  const bool live = idx < total;
  int64_t t = 0, c = 0;
  if (total <= 0xFFFFFFFFll) {  // uniform: 32-bit division when the index fits
    const uint32_t t32 = (uint32_t)idx / (uint32_t)cpr;
    t = t32;
    c = (int64_t)((uint32_t)idx - t32 * (uint32_t)cpr);
  } else {
    t = idx / cpr;
    c = idx - t * cpr;
  }
  int64_t n = t;
  bool zero = !live;
  if constexpr (GATHER) {
    if (live) {
      const int32_t id = ids[t];
      zero = id < 0 || (int64_t)id >= N;
      n = zero ? 0 : id;
    }
  }
  float r[32];
  if (zero) {
#pragma unroll
    for (int i = 0; i < 32; ++i) r[i] = 0.f;
  } else {
    uint32_t wv[BITS];
    load_chunk<BITS>(codes + n * (K * BITS / 32) + c * BITS, wv);
    const int64_t gi = n * (K / G) + (c * 32) / G;
    // a null bias array means every bias is +0: q*s + 0 is q*s exactly
    const float s = f16_to_f32(scales[gi]), b = biases ? f16_to_f32(biases[gi]) : 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) r[i] = __builtin_fmaf((float)chunk_code<BITS>(wv, i), s, b);
  }
  uint4 q[NQ];
  if constexpr (ODT == X_F32) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      q[j] = make_uint4(__float_as_uint(r[4 * j]), __float_as_uint(r[4 * j + 1]),
                        __float_as_uint(r[4 * j + 2]), __float_as_uint(r[4 * j + 3]));
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      q[j] = make_uint4(pack_rne<ODT>(r[8 * j], r[8 * j + 1]), pack_rne<ODT>(r[8 * j + 2], r[8 * j + 3]),
                        pack_rne<ODT>(r[8 * j + 4], r[8 * j + 5]), pack_rne<ODT>(r[8 * j + 6], r[8 * j + 7]));
  }
  const int lane = threadIdx.x & 63;
  uint4 *ws = stage + (threadIdx.x >> 6) * 64 * NQ;  // this wave's span
#pragma unroll
  for (int j = 0; j < NQ; ++j) ws[lane * NQ + j] = q[j];
  __syncthreads();
  const int64_t w0 = idx - lane;  // the wave's first chunk
  uint4 *o = reinterpret_cast<uint4 *>(out) + w0 * NQ;
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int u = j * 64 + lane;  // unit u of the span: chunk w0 + u / NQ
    if (w0 + u / NQ < total) o[u] = ws[u];
  }
}

template <int WDT>
hipError_t quantize_w(const void *w, int64_t N, int64_t K, int G, int bits, uint32_t *codes,
                      uint16_t *scales, uint16_t *biases, hipStream_t s) {
  const int64_t total = N * (K / 32);
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
#define AQ_Q(B) case B: hipLaunchKernelGGL((quantize_kernel<WDT, B>), grid, block, 0, s, w, N, K, G, codes, scales, biases); break;
  switch (bits) {
    AQ_Q(2) AQ_Q(3) AQ_Q(4) AQ_Q(5) AQ_Q(6) AQ_Q(7) AQ_Q(8)
    default: return hipErrorInvalidValue;
  }
#undef AQ_Q
  return hipGetLastError();
}

template <int WDT>
hipError_t quantize_mse_w(const void *w, int64_t N, int64_t K, int G, int bits, int steps,
                          uint32_t *codes, uint16_t *scales, uint16_t *biases, hipStream_t s) {
  const int64_t total = N * (K / 32);
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
#define AQ_Q(B) case B: hipLaunchKernelGGL((quantize_mse_kernel<WDT, B>), grid, block, 0, s, w, N, K, G, steps, codes, scales, biases); break;
  switch (bits) {
    AQ_Q(2) AQ_Q(3) AQ_Q(4) AQ_Q(5) AQ_Q(6) AQ_Q(7) AQ_Q(8)
    default: return hipErrorInvalidValue;
  }
#undef AQ_Q
  return hipGetLastError();
}

template <int WDT>
hipError_t quantize_zp_w(const void *w, int64_t N, int64_t K, int G, int bits, uint32_t *codes,
                         uint16_t *scales, uint16_t *biases, uint8_t *zeros, hipStream_t s) {
  const int64_t total = N * (K / 8);
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
#define AQ_Q(B) case B: hipLaunchKernelGGL((quantize_zp_kernel<WDT, B>), grid, block, 0, s, w, N, K, G, codes, scales, biases, zeros); break;
  switch (bits) {
    AQ_Q(2) AQ_Q(3) AQ_Q(4) AQ_Q(5) AQ_Q(6) AQ_Q(7) AQ_Q(8)
    default: return hipErrorInvalidValue;
  }
#undef AQ_Q
  return hipGetLastError();
}

template <int ODT, bool GATHER>
hipError_t dequantize_o(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                        int64_t N, int64_t K, int G, int bits, const int32_t *ids, int64_t T,
                        void *out, hipStream_t s) {
  const int64_t total = (GATHER ? T : N) * (K / 32);
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
#define AQ_D(B) case B: hipLaunchKernelGGL((dequantize_kernel<B, ODT, GATHER>), grid, block, 0, s, codes, scales, biases, N, K, G, ids, T, out); break;
  switch (bits) {
    AQ_D(2) AQ_D(3) AQ_D(4) AQ_D(5) AQ_D(6) AQ_D(7) AQ_D(8)
    default: return hipErrorInvalidValue;
  }
#undef AQ_D
  return hipGetLastError();
}

template <bool GATHER>
hipError_t dequantize_dt(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                         int64_t N, int64_t K, int G, int bits, const int32_t *ids, int64_t T,
                         void *out, int out_dtype, hipStream_t s) {
  switch (out_dtype) {
    case X_F32: return dequantize_o<X_F32, GATHER>(codes, scales, biases, N, K, G, bits, ids, T, out, s);
    case X_F16: return dequantize_o<X_F16, GATHER>(codes, scales, biases, N, K, G, bits, ids, T, out, s);
    case X_BF16: return dequantize_o<X_BF16, GATHER>(codes, scales, biases, N, K, G, bits, ids, T, out, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_quantize(const void *w, int w_dtype, int64_t N, int64_t K, int G, int bits,
                           uint32_t *codes, uint16_t *scales, uint16_t *biases, hipStream_t s) {
  switch (w_dtype) {
    case X_F32: return quantize_w<X_F32>(w, N, K, G, bits, codes, scales, biases, s);
    case X_F16: return quantize_w<X_F16>(w, N, K, G, bits, codes, scales, biases, s);
    case X_BF16: return quantize_w<X_BF16>(w, N, K, G, bits, codes, scales, biases, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_quantize_mse(const void *w, int w_dtype, int64_t N, int64_t K, int G, int bits,
                               int steps, uint32_t *codes, uint16_t *scales, uint16_t *biases,
                               hipStream_t s) {
  switch (w_dtype) {
    case X_F32: return quantize_mse_w<X_F32>(w, N, K, G, bits, steps, codes, scales, biases, s);
    case X_F16: return quantize_mse_w<X_F16>(w, N, K, G, bits, steps, codes, scales, biases, s);
    case X_BF16: return quantize_mse_w<X_BF16>(w, N, K, G, bits, steps, codes, scales, biases, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_quantize_zp(const void *w, int w_dtype, int64_t N, int64_t K, int G, int bits,
                              uint32_t *codes, uint16_t *scales, uint16_t *biases, uint8_t *zeros,
                              hipStream_t s) {
  switch (w_dtype) {
    case X_F32: return quantize_zp_w<X_F32>(w, N, K, G, bits, codes, scales, biases, zeros, s);
    case X_F16: return quantize_zp_w<X_F16>(w, N, K, G, bits, codes, scales, biases, zeros, s);
    case X_BF16: return quantize_zp_w<X_BF16>(w, N, K, G, bits, codes, scales, biases, zeros, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_dequantize(const uint32_t *codes, const uint16_t *scales,
                             const uint16_t *biases, int64_t N, int64_t K, int G, int bits,
                             void *out, int out_dtype, hipStream_t s) {
  return dequantize_dt<false>(codes, scales, biases, N, K, G, bits, nullptr, 0, out, out_dtype, s);
}

hipError_t launch_embedding(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                            int64_t V, int64_t K, int G, int bits, const int32_t *ids, int64_t T,
                            void *out, int out_dtype, hipStream_t s) {
  return dequantize_dt<true>(codes, scales, biases, V, K, G, bits, ids, T, out, out_dtype, s);
}

}  // namespace aq
