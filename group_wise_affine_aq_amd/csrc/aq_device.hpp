// aq_device.hpp -- device helpers shared by the libaq kernels (gfx950).
//
// Number formats: fp16 = IEEE binary16, bf16 = upper half of binary32.
// Packed codes: one least-significant-bit-first bitstream per row ("Tutorial
// 10: Quantization", s.3, shift-and-mask extraction); a "chunk" is 32
// consecutive codes of a row, i.e. exactly `BITS` uint32 words, and always
// lies inside one group because group sizes are multiples of 32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "aq_internal.hpp"

namespace aq {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

struct f16_t { uint16_t bits; };
struct bf16_t { uint16_t bits; };

// ---- scalar conversions --------------------------------------------------------

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}
// round-to-nearest-even binary32 -> binary16 (hardware convert, default mode)
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
// round-to-nearest-even binary32 -> bfloat16 for finite inputs; NaN stays NaN
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename XT> struct xtraits;
template <> struct xtraits<f16_t> {
  static __device__ __forceinline__ float to_f32(uint16_t h) { return f16_to_f32(h); }
  static __device__ __forceinline__ uint16_t from_f32(float f) { return f32_to_f16_rne(f); }
};
template <> struct xtraits<bf16_t> {
  static __device__ __forceinline__ float to_f32(uint16_t h) { return bf16_to_f32(h); }
  static __device__ __forceinline__ uint16_t from_f32(float f) { return f32_to_bf16_rne(f); }
};

// ---- packed dot products (v_dot2c_f32_f16 / v_dot2c_f32_bf16) ---------------------

__device__ __forceinline__ float dot2(f16_t, uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a), __builtin_bit_cast(half2v, b), c,
                                false);
}
__device__ __forceinline__ float dot2(bf16_t, uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, a),
                                         __builtin_bit_cast(bf16x2v, b), c, false);
}

// ---- code extraction ---------------------------------------------------------------

// code i (0..31) of a chunk held in w[0..BITS-1]
template <int BITS>
__device__ __forceinline__ uint32_t chunk_code(const uint32_t *w, int i) {
  const int pos = i * BITS, word = pos >> 5, sh = pos & 31;
  const uint32_t mask = (1u << BITS) - 1u;
  if (sh + BITS <= 32) return (w[word] >> sh) & mask;
  return __builtin_amdgcn_alignbit(w[word + 1], w[word], sh) & mask;
}

// ---- wavefront reduction (64 lanes, DPP) ----------------------------------------------

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xF, false));
}
// sum over the 64 lanes; the result is returned in every lane
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);        // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);        // quad_perm [2,3,0,1]
  v += dpp_f<0x124>(v);       // row_ror:4
  v += dpp_f<0x128>(v);       // row_ror:8   -> every lane holds its 16-lane row sum
  v += dpp_f<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_f<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3 -> lane 63 holds the total
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

}  // namespace aq

namespace aq {

// ---- chunk loads: the BITS words of one 32-code chunk ---------------------------------
// A chunk starts at word c*BITS of its row, so its byte address is a multiple
// of 4*BITS: 16-byte vector loads for BITS in {4, 8}, 8-byte for {2, 6}.
template <int BITS>
__device__ __forceinline__ void load_chunk(const uint32_t *__restrict__ p, uint32_t *w) {
  if constexpr (BITS % 4 == 0) {
#pragma unroll
    for (int j = 0; j < BITS / 4; ++j) {
      uint4 v = reinterpret_cast<const uint4 *>(p)[j];
      w[4 * j] = v.x; w[4 * j + 1] = v.y; w[4 * j + 2] = v.z; w[4 * j + 3] = v.w;
    }
  } else if constexpr (BITS % 2 == 0) {
#pragma unroll
    for (int j = 0; j < BITS / 2; ++j) {
      uint2 v = reinterpret_cast<const uint2 *>(p)[j];
      w[2 * j] = v.x; w[2 * j + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int j = 0; j < BITS; ++j) w[j] = p[j];
  }
}

// ---- weight loads for the quantizers ------------------------------------------------

template <int WDT>
__device__ __forceinline__ void load8(const void *__restrict__ base, int64_t e, float *v) {
  if constexpr (WDT == X_F32) {
    const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) + e);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    uint4 a = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(base) + e);
    uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (WDT == X_F16) {
        v[2 * i] = f16_to_f32((uint16_t)(u[i] & 0xFFFFu));
        v[2 * i + 1] = f16_to_f32((uint16_t)(u[i] >> 16));
      } else {
        v[2 * i] = bf16_to_f32((uint16_t)(u[i] & 0xFFFFu));
        v[2 * i + 1] = bf16_to_f32((uint16_t)(u[i] >> 16));
      }
    }
  }
}

// 32 weights (one 32-code chunk, BITS whole words of codes) of the row
// starting at element e, widened exactly to binary32
template <int WDT>
__device__ __forceinline__ void load32(const void *__restrict__ base, int64_t e, float *v) {
#pragma unroll
  for (int j = 0; j < 4; ++j) load8<WDT>(base, e + 8 * j, v + 8 * j);
}

}  // namespace aq
