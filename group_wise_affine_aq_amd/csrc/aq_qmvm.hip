// aq_qmvm.hip -- quantized matrix-vector product for a few rows (2 <= M <= 8)
// on the gfx950 matrix cores, 4-bit and 8-bit codes.
//
// The operation is the QMV of "Quantization" (metalworking, MLX notes, QMV
// bullet), y = x @ W^T with W packed, for the speculative-decoding widths
// the same page discusses (its dispatch section: a wider QMV for M around
// 3-6).  The vector-ALU kernels spend about 0.5 VALU lane-ops per weight per
// row of x on the dot products, which makes M >= 4 VALU-bound on MI355X
// (about 2.8 lane-ops per weight are available at full HBM bandwidth).
// Here the dot products run on the matrix cores instead, with the integer
// codes as one operand:
//
//  * v_mfma_f32_16x16x32_{bf16,f16}: A = x (16 rows, rows >= M read as
//    zero), B = 16 rows of W, each code q entering as the exact value
//    OFF + q, so one MFMA over 32 codes gives P = sum x * (OFF + q).
//    4-bit: one v_and_or_b32 per pair (OFF = 128 in bf16, 1024 in fp16).
//    8-bit, fp16: one v_perm_b32 per pair puts the byte under an 0x64 high
//    byte (OFF = 1024).  8-bit, bf16: bf16 has too few mantissa bits for
//    that, so the byte goes through binary32 (v_cvt_f32_ubyte*, exact) and
//    a packed round to bf16, also exact (OFF = 0);
//  * a second MFMA against a register of ones gives X = sum x over the same
//    chunk, already in the output lane layout;
//  * per group, y += s * (P - OFF * X) + b * X = s * P + (b - OFF * s) * X,
//    the same identity the vector kernels apply (sum_k x (q s + b) over a
//    group), in binary32;
//  * codes arrive as 16-byte loads.  4-bit: lane quarter h reads chunk h of
//    a 4-chunk step of its row, and a 4x4 transpose across the lane quarters
//    (v_permlane32_swap, v_permlane16_swap) gives each quarter code word h of
//    every chunk, which is the MFMA B-operand layout.  8-bit: each of two
//    loads covers two chunks; quarter h holds codes 16h .. 16h+15 of them,
//    which already is the B layout of two MFMAs when a group spans both
//    chunks (G >= 64); for G = 32 one v_permlane32_swap per register pair
//    brings each MFMA back inside one chunk (quarter h then holds 8-code
//    unit sigma(h) = (0, 2, 1, 3)[h] of it).  The MFMA's k order is free as
//    long as x follows it, and x is loaded to match;
//  * x is read straight from global memory (it stays in L2), one 16-byte load
//    per lane carrying two chunks (M <= 8) or four (M <= 4) in the lanes of
//    A-operand rows that only feed discarded output rows, moved into place by
//    a DPP row rotation; its pairs are permuted to the order the unpack
//    produces (code e with code e+4);
//  * the workgroup's scales and biases (16 R whole rows, one contiguous range
//    each) are staged in LDS once with 16-byte loads: per-group 2-byte
//    loads from every lane cost more than all the rest of the kernel;
//  * a workgroup of W waves covers 16 R rows; its waves split K and add their
//    partial sums through LDS at the end (W chosen per shape so that the
//    grid fills the chip with waves that each keep loads in flight).
#include "aq_device.hpp"
#include "aq_internal.hpp"

namespace aq {
namespace {

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8v __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

constexpr int kStepK = 128;  // k per step: 4 chunks

// per (activation type, code width): the register constant of the unpack
// and the offset OFF that every code value carries into the products
template <typename XT, int BITS>
struct mm_traits;
template <>
struct mm_traits<bf16_t, 4> {
  static constexpr uint32_t magic = 0x43004300u;  // bf16 128.0 in both halves
  static constexpr uint32_t ones = 0x3F803F80u;   // bf16 1.0
  static constexpr float off = 128.f;
};
template <>
struct mm_traits<f16_t, 4> {
  static constexpr uint32_t magic = 0x64006400u;  // fp16 1024.0
  static constexpr uint32_t ones = 0x3C003C00u;   // fp16 1.0
  static constexpr float off = 1024.f;
};
template <>
struct mm_traits<bf16_t, 8> {
  static constexpr uint32_t magic = 0u;  // unused: codes are converted exactly
  static constexpr uint32_t ones = 0x3F803F80u;
  static constexpr float off = 0.f;
};
template <>
struct mm_traits<f16_t, 8> {
  static constexpr uint32_t magic = 0x64646464u;  // high bytes of fp16 1024 + q
  static constexpr uint32_t ones = 0x3C003C00u;
  static constexpr float off = 1024.f;
};

template <typename XT>
__device__ __forceinline__ f32x4v mfma16(uint4 a, uint4 b, f32x4v c) {
  if constexpr (std::is_same<XT, bf16_t>::value)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, a),
                                                   __builtin_bit_cast(bf16x8v, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8v, a),
                                                  __builtin_bit_cast(f16x8v, b), c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mk_rsrc(const void *base, int64_t bytes) {
  const int n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (bytes < 0 ? 0 : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, n, 0x00020000);
}

__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xE4, 0xF, 0xF, false);
}

// 4x4 transpose of (lane quarter, register): afterwards quarter h holds in
// r[j] what quarter j held in r[h]
__device__ __forceinline__ void transpose4(uint32_t (&r)[4]) {
  auto a = __builtin_amdgcn_permlane32_swap(r[0], r[2], false, false);
  r[0] = a[0]; r[2] = a[1];
  auto b = __builtin_amdgcn_permlane32_swap(r[1], r[3], false, false);
  r[1] = b[0]; r[3] = b[1];
  auto c = __builtin_amdgcn_permlane16_swap(r[0], r[1], false, false);
  r[0] = c[0]; r[1] = c[1];
  auto d = __builtin_amdgcn_permlane16_swap(r[2], r[3], false, false);
  r[2] = d[0]; r[3] = d[1];
}

// 8 codes of a word -> 4 registers of (OFF + q_e, OFF + q_{e+4}) pairs.
// Plain C on register-held constants: the compiler emits v_and_or_b32 and
// tracks the MFMA operand hazards of the registers it writes (an inline-asm
// write would be invisible to that check).
__device__ __forceinline__ uint4 unpack_word(uint32_t w, uint32_t mask, uint32_t magic) {
  uint32_t p[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) p[e] = ((w >> (4 * e)) & mask) | magic;
  return make_uint4(p[0], p[1], p[2], p[3]);
}

// 8 codes of two words (8-bit) -> 4 registers of (OFF + q_2e, OFF + q_2e+1)
// pairs, in code order.  fp16: v_perm_b32 places bytes e, e+1 under the
// 0x64 bytes of the magic register (fp16 0x64qq = 1024 + q exactly).  bf16:
// unsigned byte to binary32 and a packed round to bf16, exact for q < 256.
template <typename XT>
__device__ __forceinline__ uint4 unpack_bytes(uint32_t w0, uint32_t w1, uint32_t magic) {
  if constexpr (std::is_same<XT, f16_t>::value) {
    return make_uint4(__builtin_amdgcn_perm(magic, w0, 0x04010400u),
                      __builtin_amdgcn_perm(magic, w0, 0x04030402u),
                      __builtin_amdgcn_perm(magic, w1, 0x04010400u),
                      __builtin_amdgcn_perm(magic, w1, 0x04030402u));
  } else {
    uint32_t p[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t w = i == 0 ? w0 : w1;
      const bf16x2v lo = {(__bf16)(float)(w & 0xFFu), (__bf16)(float)((w >> 8) & 0xFFu)};
      const bf16x2v hi = {(__bf16)(float)((w >> 16) & 0xFFu), (__bf16)(float)(w >> 24)};
      p[2 * i] = __builtin_bit_cast(uint32_t, lo);
      p[2 * i + 1] = __builtin_bit_cast(uint32_t, hi);
    }
    return make_uint4(p[0], p[1], p[2], p[3]);
  }
}

// natural pairs (x0 x1)(x2 x3)(x4 x5)(x6 x7) -> (x0 x4)(x1 x5)(x2 x6)(x3 x7)
__device__ __forceinline__ uint4 permute_x(uint4 v) {
  return make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u),  // lo16(x) | lo16(z) << 16
                    __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),  // hi16(x) | hi16(z) << 16
                    __builtin_amdgcn_perm(v.w, v.y, 0x05040100u),
                    __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
}

// one step (4 chunks) of one wave's K range, as loaded
template <int NXL, int BITS>
struct MStep {
  // 4-bit: quarter h holds chunk c0 + h of row n16.  8-bit: words 4r .. 4r+3
  // hold words 4 (h & 1) .. +3 of chunk c0 + 2r + (h >> 1)
  uint32_t cw[BITS];
  uint4 xl[4 / NXL];   // x loads of the step, NXL MFMA slots each (natural pair order)
};

// lane l of a row of 16 receives the value of lane (l + 16 - k) % 16 ... i.e. a
// rotation of each 16-lane row by k (DPP row_ror)
template <int K16>
__device__ __forceinline__ uint4 row_ror(uint4 v) {
  if constexpr (K16 == 0) return v;
  constexpr int ctl = 0x120 + K16;
  return make_uint4((uint32_t)__builtin_amdgcn_mov_dpp((int)v.x, ctl, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_mov_dpp((int)v.y, ctl, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_mov_dpp((int)v.z, ctl, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_mov_dpp((int)v.w, ctl, 0xF, 0xF, false));
}

// One workgroup's share: 16 rows of W (rows past the matrix read as zero)
// against up to XR rows of x, K split over its W waves.  GS: log2 of the
// chunks per group.  XR: rows of x carried per chunk slot of an x load --
// output rows >= XR are discarded, so A-operand rows XR.. may hold
// anything, and one 16-byte load per lane carries NXL = 16 / XR chunks
// (lanes XR s .. XR s + XR - 1 of a row of 16 hold chunk slot s); a row
// rotation moves a slot to lanes 0.. .
template <typename XT, int BITS, int W, int GS, int XR>
struct MBlock {
  static constexpr int CPG = 1 << GS;  // chunks per group (G = 32 CPG)
  static constexpr int NG = 4 / CPG;   // groups per step
  static constexpr int NXL = 16 / XR;
  // 8-bit with a group inside each 32-code chunk: a lane-half swap per
  // register pair keeps every MFMA inside one chunk (one group)
  static constexpr bool kSwap = BITS == 8 && GS == 0;

  // first chunk of the codes behind MFMA slot j of the step at chunk c0 (the
  // slot is past K iff this chunk is), and quarter h's offset into its x row
  // in elements, so that x follows the k order of the B operand
  static __device__ __forceinline__ int slot_chunk(int c0, int j) {
    return BITS == 8 && !kSwap ? c0 + 2 * (j >> 1) : c0 + j;
  }
  static __device__ __forceinline__ int slot_xoff(int cb, int j, int h) {
    if constexpr (BITS == 4) return cb * 32 + 8 * h;
    else if constexpr (kSwap) return cb * 32 + 8 * ((h >> 1) | ((h & 1) << 1));
    else return cb * 32 + 16 * h + 8 * (j & 1);
  }

  __amdgpu_buffer_rsrc_t rw, rx;
  const uint16_t *sbl;  // LDS: [2][16][gpr] scales, biases of the 16 rows
  int64_t K, wpr, gpr;
  int nch, n16, h, c_beg, c_end;

  __device__ void setup(const uint32_t *codes16, int64_t nrows, int64_t K_, int kw, int wave,
                        int lane, const uint16_t *sbl_, __amdgpu_buffer_rsrc_t rx_) {
    K = K_;
    nch = (int)(K >> 5);
    wpr = (int64_t)nch * BITS;  // a 32-code chunk is BITS words
    gpr = nch >> GS;
    n16 = lane & 15;
    h = lane >> 4;
    rw = mk_rsrc(codes16, nrows * wpr * 4);
    rx = rx_;
    sbl = sbl_;
    // this wave's K range, whole steps of 4 chunks (each a whole number of groups)
    c_beg = wave * (kw >> 5);
    c_end = c_beg + (kw >> 5) < nch ? c_beg + (kw >> 5) : nch;
  }

  // scales and biases of the 16 rows (one contiguous, 16-byte aligned range
  // each) to LDS with 16-byte loads; a load that crosses the end of the valid
  // rows reads as zero as a whole, so whole units inside them first, then
  // 2-byte loads, zeros past them.  The caller synchronizes.
  static __device__ void stage_sb(const uint16_t *scales16, const uint16_t *biases16,
                                  int64_t nrows, int64_t gpr_, uint16_t *sb) {
    const __amdgpu_buffer_rsrc_t rs = mk_rsrc(scales16, nrows * gpr_ * 2);
    const __amdgpu_buffer_rsrc_t rb = mk_rsrc(biases16, nrows * gpr_ * 2);
    const int valid = (int)(nrows * gpr_), total = 16 * (int)gpr_;
    const int full = valid >> 3;
    for (int i = threadIdx.x; i < full; i += 64 * W) {
      const u32x4v vs = __builtin_amdgcn_raw_buffer_load_b128(rs, i * 16, 0, 0);
      const u32x4v vb = __builtin_amdgcn_raw_buffer_load_b128(rb, i * 16, 0, 0);
      *reinterpret_cast<u32x4v *>(sb + i * 8) = vs;
      *reinterpret_cast<u32x4v *>(sb + total + i * 8) = vb;
    }
    for (int e = full * 8 + threadIdx.x; e < total; e += 64 * W) {
      const bool in = e < valid;
      sb[e] = in ? (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs, e * 2, 0, 0) : (uint16_t)0;
      sb[total + e] = in ? (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rb, e * 2, 0, 0) : (uint16_t)0;
    }
  }

  __device__ void load(int c0, uint32_t xro, MStep<NXL, BITS> &st) const {
#pragma unroll
    for (int r = 0; r < BITS / 4; ++r) {
      // 4-bit: chunk c0 + h.  8-bit: words 4 (h & 1) .. of chunk c0 + 2r + (h >> 1)
      const int ch = BITS == 4 ? c0 + h : c0 + 2 * r + (h >> 1);
      const bool inside = ch < nch;  // chunks past K read as zero
      const int64_t wo = BITS == 4 ? (int64_t)ch * 4 : (int64_t)ch * 8 + 4 * (h & 1);
      const uint32_t o = (uint32_t)(((int64_t)n16 * wpr + (inside ? wo : 0)) * 4);
      const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)o, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) st.cw[4 * r + i] = inside ? v[i] : 0u;
    }
#pragma unroll
    for (int t = 0; t < 4 / NXL; ++t) {
      const int j = t * NXL + n16 / XR;  // MFMA slot this lane's load carries
      const int cb = slot_chunk(c0, j);
      const int xo = cb < nch ? slot_xoff(cb, j, h) : 0;
      const u32x4v u = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(xro + (uint32_t)xo * 2u), 0, 0);
      st.xl[t] = make_uint4(u[0], u[1], u[2], u[3]);
    }
  }

  __device__ void compute(int c0, MStep<NXL, BITS> &st, f32x4v &acc, uint32_t vmask,
                          uint32_t vmagic, uint4 ones) const {
    const float off = mm_traits<XT, BITS>::off;
    if constexpr (BITS == 4) {
      transpose4(st.cw);  // quarter h: word h of chunks c0 .. c0+3
    } else if constexpr (kSwap) {
      // quarters (0 1 | 2 3) of pair 0 and pair 1 -> pair 0 of chunk 2r, pair 1 of 2r+1
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          auto v = __builtin_amdgcn_permlane32_swap(st.cw[4 * r + i], st.cw[4 * r + 2 + i], false, false);
          st.cw[4 * r + i] = v[0];
          st.cw[4 * r + 2 + i] = v[1];
        }
    }
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      if (c0 + q * CPG >= c_end) break;  // past K (uniform)
      f32x4v xg = (f32x4v){0.f, 0.f, 0.f, 0.f}, pg = (f32x4v){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < CPG; ++jj) {
        const int j = q * CPG + jj;
        uint4 xr = st.xl[j / NXL];
        if constexpr (NXL == 2) {
          if (j % 2 == 1) xr = row_ror<8>(xr);
        } else if constexpr (NXL == 4) {
          if (j % 4 == 1) xr = row_ror<12>(xr);
          if (j % 4 == 2) xr = row_ror<8>(xr);
          if (j % 4 == 3) xr = row_ror<4>(xr);
        }
        uint4 xa, wb;
        if constexpr (BITS == 4) {
          xa = permute_x(xr);
          wb = unpack_word(st.cw[j], vmask, vmagic);
        } else {
          xa = xr;
          wb = unpack_bytes<XT>(st.cw[2 * j], st.cw[2 * j + 1], vmagic);
        }
        if (slot_chunk(c0, j) >= nch) xa = make_uint4(0, 0, 0, 0);
        xg = mfma16<XT>(xa, ones, xg);
        pg = mfma16<XT>(xa, wb, pg);
      }
      const int li = n16 * (int)gpr + (c0 >> GS) + q;
      const float sc = f16_to_f32(sbl[li]), bi = f16_to_f32(sbl[16 * (int)gpr + li]);
      const float bo = __builtin_fmaf(-off, sc, bi);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(bo, xg[e], __builtin_fmaf(sc, pg[e], acc[e]));
    }
  }

  // partial sums of this wave's K range; lane (n16, h) gets output rows
  // m = 4 h + e of x against W row n16.  xro: byte offset of the x row that
  // chunk slot row (n16 % XR) carries (past the x resource: zeros).
  __device__ f32x4v run(uint32_t xro) const {
    const uint32_t vmask = opaque(0x000F000Fu), vmagic = opaque(mm_traits<XT, BITS>::magic);
    const uint32_t vones = opaque(mm_traits<XT, BITS>::ones);
    const uint4 ones = make_uint4(vones, vones, vones, vones);
    f32x4v acc = (f32x4v){0.f, 0.f, 0.f, 0.f};
    if (c_beg >= c_end) return acc;
    // double-buffered: the next step's loads are in flight while this one
    // computes.  The prefetch is unconditional (past the range it re-reads
    // memory inside the matrix, or zeros past K): a load issued on only some
    // paths would make the in-order load counter wait for everything in flight.
    MStep<NXL, BITS> sa, sb;
    load(c_beg, xro, sa);
    int c0 = c_beg;
    for (; c0 + 8 <= c_end; c0 += 8) {
      load(c0 + 4, xro, sb);
      compute(c0, sa, acc, vmask, vmagic, ones);
      load(c0 + 8, xro, sa);
      compute(c0 + 4, sb, acc, vmask, vmagic, ones);
    }
    if (c0 < c_end) {
      load(c0 + 4, xro, sb);
      compute(c0, sa, acc, vmask, vmagic, ones);
      if (c0 + 4 < c_end) compute(c0 + 4, sb, acc, vmask, vmagic, ones);
    }
    return acc;
  }
};

// sum the W waves' partial sums (lanes h < 2 hold output rows 0..7) through
// LDS; out(n, m, v) receives row n of the 16, x row m < 8, value v
template <int W, typename F>
__device__ __forceinline__ void reduce_out(float (&part)[W][16][8], int wave, int lane,
                                           const f32x4v &acc, F out) {
  const int n16 = lane & 15, h = lane >> 4;
  if (h < 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) part[wave][n16][4 * h + e] = acc[e];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * 8; i += 64 * W) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) v += part[w][i >> 3][i & 7];
    out(i >> 3, i & 7, v);
  }
}

template <typename XT, int BITS, int W, int GS, int XR>
__global__ __launch_bounds__(64 * W) void qmvm_kernel(const uint16_t *__restrict__ x, int M,
                                                      const uint32_t *__restrict__ codes,
                                                      const uint16_t *__restrict__ scales,
                                                      const uint16_t *__restrict__ biases,
                                                      int64_t N, int64_t K, int kw,
                                                      uint16_t *__restrict__ y) {
  __shared__ float part[W][16][8];
  extern __shared__ __attribute__((aligned(16))) uint16_t sbl[];  // [2][16][gpr]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int64_t nrows = N - row0 < 16 ? N - row0 : 16;
  const int64_t gpr = (K >> 5) >> GS;
  MBlock<XT, BITS, W, GS, XR> blk;
  blk.setup(codes + row0 * (K >> 5) * BITS, nrows, K, kw, wave, lane, sbl,
            mk_rsrc(x, (int64_t)M * K * 2));  // rows of x past M read as zero
  MBlock<XT, BITS, W, GS, XR>::stage_sb(scales + row0 * gpr, biases + row0 * gpr, nrows, gpr, sbl);
  __syncthreads();
  const f32x4v acc = blk.run((uint32_t)((int64_t)((lane & 15) % XR) * K * 2));
  reduce_out<W>(part, wave, lane, acc, [&](int nn, int m, float v) {
    if (m < M && row0 + nn < N) y[(int64_t)m * N + row0 + nn] = xtraits<XT>::from_f32(v);
  });
}

// Mixture-of-experts gather ("Quantization", metalworking, gather variants
// for MoE experts): y[t, j, :] = x[t] @ W_{ids[t, j]}^T.  One workgroup per
// (16 rows, expert e) collects the (token, slot) pairs routed to e and runs
// them in batches of up to 8 x rows through the matrix cores, so each
// expert's rows are read once per batch of tokens that chose it (experts no
// token chose are never read).  Pairs whose id is outside [0, E) get zero
// rows, written by the workgroups of expert 0.
constexpr int kGTile = 256;  // ids scanned per round

template <typename XT, int BITS, int W, int GS>
__global__ __launch_bounds__(64 * W) void gather_qmvm_kernel(
    const uint16_t *__restrict__ x, int64_t T, const uint32_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ biases, int64_t E, int64_t N,
    int64_t K, const int32_t *__restrict__ ids, int topk, int kw, uint16_t *__restrict__ y) {
  __shared__ float part[W][16][8];
  __shared__ int list[kGTile];
  __shared__ int count;
  extern __shared__ __attribute__((aligned(16))) uint16_t sbl[];  // [2][16][gpr]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int e = blockIdx.y;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int64_t nrows = N - row0 < 16 ? N - row0 : 16;
  const int64_t gpr = (K >> 5) >> GS, wpe = N * (K >> 5) * BITS;
  const int64_t total = T * topk;

  // pairs with an id outside the table: zero rows (expert-0 workgroups)
  if (e == 0)
    for (int64_t p = threadIdx.x; p < total; p += 64 * W) {
      const int32_t id = ids[p];
      if (id < 0 || id >= E)
        for (int nn = 0; nn < nrows; ++nn) y[p * N + row0 + nn] = 0;
    }
  // does any pair choose this expert?  (if not, nothing of it is read)
  if (threadIdx.x == 0) count = 0;
  __syncthreads();
  for (int64_t p = threadIdx.x; p < total; p += 64 * W)
    if (ids[p] == e) atomicAdd(&count, 1);
  __syncthreads();
  if (count == 0) return;

  MBlock<XT, BITS, W, GS, 8> blk;
  blk.setup(codes + e * wpe + row0 * (K >> 5) * BITS, nrows, K, kw, wave, lane, sbl,
            mk_rsrc(x, T * K * 2));
  MBlock<XT, BITS, W, GS, 8>::stage_sb(scales + (e * N + row0) * gpr, biases + (e * N + row0) * gpr,
                                 nrows, gpr, sbl);
  for (int64_t t0 = 0; t0 < total; t0 += kGTile) {
    __syncthreads();  // also publishes the staged scales before the first batch
    if (threadIdx.x == 0) count = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < kGTile; i += 64 * W) {
      const int64_t p = t0 + i;
      if (p < total && ids[p] == e) list[atomicAdd(&count, 1)] = (int)i;
    }
    __syncthreads();
    const int n = count;
    for (int b0 = 0; b0 < n; b0 += 8) {
      // slot row m = n16 % 8 carries pair list[b0 + m]; missing pairs read
      // past the x resource (zeros)
      const int m = lane & 7;
      const uint32_t xro = b0 + m < n ? (uint32_t)(((t0 + list[b0 + m]) / topk) * K * 2)
                                      : (uint32_t)(T * K * 2);
      const f32x4v acc = blk.run(xro);
      reduce_out<W>(part, wave, lane, acc, [&](int nn, int mm, float v) {
        if (b0 + mm < n && row0 + nn < N)
          y[(t0 + list[b0 + mm]) * N + row0 + nn] = xtraits<XT>::from_f32(v);
      });
      __syncthreads();  // part and list reused
    }
  }
}

template <typename XT, int BITS, int W, int XR>
hipError_t qmvm_go(const void *x, int M, const uint32_t *codes, const uint16_t *scales,
                   const uint16_t *biases, int64_t N, int64_t K, int G, void *y, hipStream_t s) {
  const int64_t steps = (K + kStepK - 1) / kStepK;
  const int kw = (int)((steps + W - 1) / W) * kStepK;  // k per wave, whole steps
  const int64_t blocks = (N + 15) / 16;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(64 * W);
  const size_t lds = (size_t)2 * 16 * (K / G) * 2;  // scales + biases of the rows
  switch (G) {
    case 32: hipLaunchKernelGGL((qmvm_kernel<XT, BITS, W, 0, XR>), grid, block, lds, s, (const uint16_t *)x, M, codes, scales, biases, N, K, kw, (uint16_t *)y); break;
    case 64: hipLaunchKernelGGL((qmvm_kernel<XT, BITS, W, 1, XR>), grid, block, lds, s, (const uint16_t *)x, M, codes, scales, biases, N, K, kw, (uint16_t *)y); break;
    case 128: hipLaunchKernelGGL((qmvm_kernel<XT, BITS, W, 2, XR>), grid, block, lds, s, (const uint16_t *)x, M, codes, scales, biases, N, K, kw, (uint16_t *)y); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename XT, int BITS>
hipError_t gather_go(const void *x, int64_t T, const uint32_t *codes, const uint16_t *scales,
                     const uint16_t *biases, int64_t E, int64_t N, int64_t K,
                     const int32_t *ids, int topk, int G, void *y, hipStream_t s) {
  constexpr int W = 2;  // the grid has (rows / 16) x E workgroups: split K in two
  const int64_t steps = (K + kStepK - 1) / kStepK;
  const int kw = (int)((steps + W - 1) / W) * kStepK;
  const int64_t blocks = (N + 15) / 16;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks, (unsigned)E), block(64 * W);
  const size_t lds = (size_t)2 * 16 * (K / G) * 2;
  switch (G) {
    case 32: hipLaunchKernelGGL((gather_qmvm_kernel<XT, BITS, W, 0>), grid, block, lds, s, (const uint16_t *)x, T, codes, scales, biases, E, N, K, ids, topk, kw, (uint16_t *)y); break;
    case 64: hipLaunchKernelGGL((gather_qmvm_kernel<XT, BITS, W, 1>), grid, block, lds, s, (const uint16_t *)x, T, codes, scales, biases, E, N, K, ids, topk, kw, (uint16_t *)y); break;
    case 128: hipLaunchKernelGGL((gather_qmvm_kernel<XT, BITS, W, 2>), grid, block, lds, s, (const uint16_t *)x, T, codes, scales, biases, E, N, K, ids, topk, kw, (uint16_t *)y); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool qmvm_supported(int M, int bits, int64_t N, int64_t K, int G) {
  // scales and biases of 16 rows staged in LDS: at most 48 KB
  return M >= 2 && M <= 8 && (bits == 4 || bits == 8) && N >= 1 && K >= 32 && 16 * K * 2 <= 0x7FFFFFFF &&
         (int64_t)2 * 16 * (K / G) * 2 <= 48 * 1024;
}

hipError_t launch_qmvm(const void *x, int x_dtype, int M, const uint32_t *codes,
                       const uint16_t *scales, const uint16_t *biases, int64_t N, int64_t K, int G,
                       int bits, void *y, hipStream_t s) {
  // 16 rows per workgroup (<= 128 VGPRs, so 4 waves per SIMD), and K split
  // over W waves so that the grid has about four waves per SIMD: each wave
  // keeps two steps of loads in flight, and the chip needs tens of KB in
  // flight per CU to stream from HBM
  const int64_t rowblocks = (N + 15) / 16;
  const int64_t target = 4 * 4 * (int64_t)device_cus();
  const int W = rowblocks * 2 >= target ? 2 : rowblocks * 4 >= target ? 4 : rowblocks * 8 >= target ? 8 : 16;
#define AQ_QMVM_W(T, B, XR) \
  switch (W) { \
    case 2: return qmvm_go<T, B, 2, XR>(x, M, codes, scales, biases, N, K, G, y, s); \
    case 4: return qmvm_go<T, B, 4, XR>(x, M, codes, scales, biases, N, K, G, y, s); \
    case 8: return qmvm_go<T, B, 8, XR>(x, M, codes, scales, biases, N, K, G, y, s); \
    default: return qmvm_go<T, B, 16, XR>(x, M, codes, scales, biases, N, K, G, y, s); \
  }
#define AQ_QMVM_B(T, B) \
  if (M <= 4) { AQ_QMVM_W(T, B, 4) } else { AQ_QMVM_W(T, B, 8) }
#define AQ_QMVM(T) \
  if (bits == 4) { AQ_QMVM_B(T, 4) } else { AQ_QMVM_B(T, 8) }
  if (x_dtype == X_BF16) { AQ_QMVM(bf16_t) }
  if (x_dtype == X_F16) { AQ_QMVM(f16_t) }
#undef AQ_QMVM
#undef AQ_QMVM_B
#undef AQ_QMVM_W
  return hipErrorInvalidValue;
}

bool gather_qmvm_supported(int bits, int64_t K, int G) {
  return (bits == 4 || bits == 8) && K >= 32 && (int64_t)2 * 16 * (K / G) * 2 <= 48 * 1024;
}

hipError_t launch_gather_qmvm(const void *x, int x_dtype, int64_t T, const uint32_t *codes,
                              const uint16_t *scales, const uint16_t *biases, int64_t E, int64_t N,
                              int64_t K, const int32_t *ids, int topk, int G, int bits,
                              void *y, hipStream_t s) {
#define AQ_GATHER(XT) \
  return bits == 4 ? gather_go<XT, 4>(x, T, codes, scales, biases, E, N, K, ids, topk, G, y, s) \
                   : gather_go<XT, 8>(x, T, codes, scales, biases, E, N, K, ids, topk, G, y, s);
  if (x_dtype == X_BF16) { AQ_GATHER(bf16_t) }
  if (x_dtype == X_F16) { AQ_GATHER(f16_t) }
#undef AQ_GATHER
  return hipErrorInvalidValue;
}

}  // namespace aq

