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
//    a DPP row rotation; for 4-bit codes its pairs are permuted once per load
//    to the order the unpack produces (code e with code e+4);
//  * the workgroup's scales and biases (16 R whole rows, one contiguous range
//    each) are staged in LDS once, by loads that write LDS directly, issued
//    ahead of the first steps' loads: per-group 2-byte loads from every lane
//    cost more than all the rest of the kernel;
//  * a workgroup of W waves covers R blocks of 16 rows, every wave all R of
//    them (each x load and Sum-x MFMA serves R blocks); its waves split K and
//    add their partial sums through LDS at the end (R and W chosen per shape,
//    see qmvm_shape);
//  * step offsets are scalar, steps past a wave's range read outside every
//    buffer resource (zeros, no memory access) so every load is issued
//    unconditionally, and the steady-state loop is branch-free with its
//    refills pinned in place (the in-order load counter then waits only for
//    the step being computed).
#include "aq_device.hpp"
#include "aq_internal.hpp"

namespace aq {
namespace {

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8v __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate: at most n vector-memory operations outstanding (gfx9
// encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima)
constexpr int vmcnt_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }

// LDS entries of one staged array (scales or biases) of `rows` rows: whole
// 512-entry blocks, the unit one wave's 16-byte-per-lane copy fills
__host__ __device__ constexpr int sb_entries(int rows, int64_t gpr) {
  return (int)(((rows * gpr + 511) >> 9) << 9);
}

constexpr int kStepK = 128;  // k per step: 4 chunks
// steps of loads in flight per wave (measured: a third step helps 8-bit
// codes, whose steps are twice as long, and slows 4-bit ones)
template <int BITS>
constexpr int kDepth = BITS == 8 ? 3 : 2;
// a buffer offset past every resource (sizes are clamped to 2^31 - 1): the
// load returns zeros without a memory access
constexpr uint32_t kOutside = 0x80000000u;

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

// biases of a range of rows; without a bias array (null) a resource of size 0,
// whose loads return 0 (+0.0) without touching memory
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bias_rsrc(const uint16_t *scales_rows,
                                                          const uint16_t *biases_rows,
                                                          int64_t bytes) {
  return biases_rows ? mk_rsrc(biases_rows, bytes) : mk_rsrc(scales_rows, 0);
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
template <int NXL, int BITS, int R, int XS>
struct MStep {
  // per block of 16 rows.  4-bit: quarter h holds chunk c0 + h of row n16.
  // 8-bit: words 4r .. 4r+3 hold words 4 (h & 1) .. +3 of chunk c0 + 2r + (h >> 1)
  uint32_t cw[R][BITS];
  uint4 xl[XS][4 / NXL];  // x loads of the step per x set, NXL MFMA slots each (natural pair order)
};

// DPP row_ror: lane l of each row of 16 lanes receives the value of lane
// (l + 16 - K16) % 16 of the same row
template <int K16>
__device__ __forceinline__ uint4 row_ror(uint4 v) {
  if constexpr (K16 == 0) return v;
  constexpr int ctl = 0x120 + K16;
  return make_uint4((uint32_t)__builtin_amdgcn_mov_dpp((int)v.x, ctl, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_mov_dpp((int)v.y, ctl, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_mov_dpp((int)v.z, ctl, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_mov_dpp((int)v.w, ctl, 0xF, 0xF, false));
}

// One workgroup's share: R blocks of 16 rows of W (rows past the matrix read
// as zero) against up to XR rows of x, K split over its W waves.  Every wave
// runs all R blocks over its K range, so each x load, its lane moves and the
// sum-of-x MFMA serve R blocks: x comes from L2 once per 16 R rows, which
// keeps its traffic (M / 4 of the 4-bit weight bytes per 16 rows) well below
// the weights'.  GS: log2 of the chunks per group.  XR: rows of x carried per
// chunk slot of an x load -- output rows >= XR are discarded, so A-operand
// rows XR.. may hold anything, and one 16-byte load per lane carries
// NXL = 16 / XR chunks (lanes XR s .. XR s + XR - 1 of a row of 16 hold chunk
// slot s); a row rotation moves a slot to lanes 0.. .  XR = 32: two sets of
// 16 x rows (the second 16 rows below the first), each weight chunk loaded
// and unpacked once for both.
template <typename XT, int BITS, int W, int GS, int XR, int R>
struct MBlock {
  static constexpr int CPG = 1 << GS;  // chunks per group (G = 32 CPG)
  static constexpr int NG = 4 / CPG;   // groups per step
  static constexpr int XS = XR == 32 ? 2 : 1;     // sets of x rows
  static constexpr int XRS = XR == 32 ? 16 : XR;  // x rows per slot of one set
  static constexpr int NXL = 16 / XRS;
  static constexpr int ROWS = 16 * R;
  // 8-bit with a group inside each 32-code chunk: a lane-half swap per
  // register pair keeps every MFMA inside one chunk (one group)
  static constexpr bool kSwap = BITS == 8 && GS == 0;
  typedef MStep<NXL, BITS, R, XS> Step;

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
  const uint16_t *sbl;  // LDS: scales [16 R][gpr], then at sbo the biases
  int64_t K, wpr, gpr;
  int nch, n16, h, c_beg, c_end, sbo;
  uint32_t xset;  // bytes from one x set to the next (16 rows)
  // per-lane parts of the load offsets (the step's part is a scalar offset):
  // codes of block b; x of load t, and the chunk of its slot past c0
  uint32_t wv[R], xb[4 / NXL];
  int xj[4 / NXL];

  __device__ void setup(const uint32_t *codes_rows, int64_t nrows, int64_t K_, int kw, int wave,
                        int lane, const uint16_t *sbl_, __amdgpu_buffer_rsrc_t rx_) {
    K = K_;
    nch = (int)(K >> 5);
    wpr = (int64_t)nch * BITS;  // a 32-code chunk is BITS words
    gpr = nch >> GS;
    n16 = lane & 15;
    h = lane >> 4;
    rw = mk_rsrc(codes_rows, nrows * wpr * 4);
    rx = rx_;
    sbl = sbl_;
    sbo = sb_entries(ROWS, gpr);
    xset = (uint32_t)(16 * K * 2);
    // this wave's K range, whole steps of 4 chunks (each a whole number of groups)
    c_beg = wave * (kw >> 5);
    c_end = c_beg + (kw >> 5) < nch ? c_beg + (kw >> 5) : nch;
    // 4-bit: quarter h reads chunk c0 + h (16 bytes each).  8-bit: load r of
    // quarter h reads bytes 64 r + 16 h of the 128 at chunk c0
#pragma unroll
    for (int b = 0; b < R; ++b) wv[b] = (uint32_t)((int64_t)(16 * b + n16) * wpr * 4 + 16 * h);
#pragma unroll
    for (int t = 0; t < 4 / NXL; ++t) xj[t] = slot_chunk(0, t * NXL + n16 / XRS);
  }

  // x rows for the next run: xro is the byte offset of the x row that chunk
  // slot row (n16 % XR) carries (past the x resource: zeros)
  __device__ void set_x(uint32_t xro) {
#pragma unroll
    for (int t = 0; t < 4 / NXL; ++t) {
      const int j = t * NXL + n16 / XRS;  // MFMA slot this lane's load carries
      xb[t] = xro + (uint32_t)slot_xoff(slot_chunk(0, j), j, h) * 2u;
    }
  }

  // Scales and biases of the rows (one contiguous, 16-byte aligned range
  // each) to LDS with loads that write LDS directly: one instruction per wave
  // copies a block of 64 16-byte units (units past the valid rows read zero;
  // each array's LDS area is whole blocks).  Nothing lands in registers, so
  // the caller can issue its step loads behind these and wait for just these
  // (stage_sb_wait) before the barrier.
  static __device__ void stage_sb(const uint16_t *scales_rows, const uint16_t *biases_rows,
                                  int64_t nrows, int64_t gpr_, uint16_t *sb, int wave, int lane) {
    const __amdgpu_buffer_rsrc_t rs = mk_rsrc(scales_rows, nrows * gpr_ * 2);
    const __amdgpu_buffer_rsrc_t rb = bias_rsrc(scales_rows, biases_rows, nrows * gpr_ * 2);
    const int pad = sb_entries(ROWS, gpr_);
    for (int blk = wave; blk < (pad >> 9); blk += W) {
      const int off = (blk * 64 + lane) * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(sb + blk * 512), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(sb + pad + blk * 512), 16, off, 0,
                                               0, 0);
    }
  }

  // After the staging and `later` further loads of this thread: wait for the
  // staging, then redo the one unit that straddles the end of the valid rows
  // (a 16-byte load past the end reads zero as a whole), entry by entry.
  // The caller synchronizes.
  template <int later>
  static __device__ void stage_sb_wait(const uint16_t *scales_rows, const uint16_t *biases_rows,
                                       int64_t nrows, int64_t gpr_, uint16_t *sb) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(later));
    const int valid = (int)(nrows * gpr_);
    if (valid & 7) {  // uniform: only a workgroup with a partial block of rows
      const __amdgpu_buffer_rsrc_t rs = mk_rsrc(scales_rows, nrows * gpr_ * 2);
      const __amdgpu_buffer_rsrc_t rb = bias_rsrc(scales_rows, biases_rows, nrows * gpr_ * 2);
      const int pad = sb_entries(ROWS, gpr_);
      const int e = (valid & ~7) + (int)threadIdx.x;
      if (threadIdx.x < 8 && e < valid) {
        sb[e] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs, e * 2, 0, 0);
        sb[pad + e] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rb, e * 2, 0, 0);
      }
    }
  }

  __device__ void load(int c0, Step &st) const {
    const uint32_t sw = c0 < c_end ? (uint32_t)c0 * (4 * BITS) : kOutside;
#pragma unroll
    for (int b = 0; b < R; ++b)
#pragma unroll
      for (int r = 0; r < BITS / 4; ++r) {
        const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)wv[b], (int)(sw + 64 * r), 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) st.cw[b][4 * r + i] = v[i];
      }
    const int lim = c_end - c0;
#pragma unroll
    for (int xs = 0; xs < XS; ++xs)
#pragma unroll
      for (int t = 0; t < 4 / NXL; ++t) {
        const uint32_t xo = xj[t] < lim ? xb[t] + (uint32_t)xs * xset : kOutside;
        const u32x4v u =
            __builtin_amdgcn_raw_buffer_load_b128(rx, (int)xo, (int)((uint32_t)c0 * 64u), 0);
        st.xl[xs][t] = make_uint4(u[0], u[1], u[2], u[3]);
      }
  }

  // FULL: the step lies inside K (no group past its end to skip)
  template <bool FULL>
  __device__ void compute(int c0, Step &st, f32x4v (&acc)[XS][R], uint32_t vmask,
                          uint32_t vmagic, uint4 ones) const {
    const float off = mm_traits<XT, BITS>::off;
#pragma unroll
    for (int b = 0; b < R; ++b) {
      if constexpr (BITS == 4) {
        transpose4(st.cw[b]);  // quarter h: word h of chunks c0 .. c0+3
      } else if constexpr (kSwap) {
        // quarters (0 1 | 2 3) of pair 0 and pair 1 -> pair 0 of chunk 2r, pair 1 of 2r+1
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            auto v = __builtin_amdgcn_permlane32_swap(st.cw[b][4 * r + i], st.cw[b][4 * r + 2 + i],
                                                      false, false);
            st.cw[b][4 * r + i] = v[0];
            st.cw[b][4 * r + 2 + i] = v[1];
          }
      }
    }
    uint4 xp[XS][4 / NXL];  // x loads in the k order of the B operand
#pragma unroll
    for (int xs = 0; xs < XS; ++xs)
#pragma unroll
      for (int t = 0; t < 4 / NXL; ++t)
        xp[xs][t] = BITS == 4 ? permute_x(st.xl[xs][t]) : st.xl[xs][t];
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      if (!FULL && c0 + q * CPG >= c_end) break;  // past K (uniform)
      f32x4v xg[XS], pg[XS][R];
#pragma unroll
      for (int xs = 0; xs < XS; ++xs) {
        xg[xs] = (f32x4v){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < R; ++b) pg[xs][b] = (f32x4v){0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int jj = 0; jj < CPG; ++jj) {
        const int j = q * CPG + jj;
        uint4 xa[XS];
#pragma unroll
        for (int xs = 0; xs < XS; ++xs) {
          xa[xs] = xp[xs][j / NXL];
          if constexpr (NXL == 2) {
            if (j % 2 == 1) xa[xs] = row_ror<8>(xa[xs]);
          } else if constexpr (NXL == 4) {
            if (j % 4 == 1) xa[xs] = row_ror<12>(xa[xs]);
            if (j % 4 == 2) xa[xs] = row_ror<8>(xa[xs]);
            if (j % 4 == 3) xa[xs] = row_ror<4>(xa[xs]);
          }
          xg[xs] = mfma16<XT>(xa[xs], ones, xg[xs]);
        }
#pragma unroll
        for (int b = 0; b < R; ++b) {
          const uint4 wb = BITS == 4 ? unpack_word(st.cw[b][j], vmask, vmagic)
                                     : unpack_bytes<XT>(st.cw[b][2 * j], st.cw[b][2 * j + 1], vmagic);
#pragma unroll
          for (int xs = 0; xs < XS; ++xs) pg[xs][b] = mfma16<XT>(xa[xs], wb, pg[xs][b]);
        }
      }
#pragma unroll
      for (int b = 0; b < R; ++b) {
        const int li = (16 * b + n16) * (int)gpr + (c0 >> GS) + q;
        const float sc = f16_to_f32(sbl[li]), bi = f16_to_f32(sbl[sbo + li]);
        const float bo = __builtin_fmaf(-off, sc, bi);
#pragma unroll
        for (int xs = 0; xs < XS; ++xs)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[xs][b][e] =
                __builtin_fmaf(bo, xg[xs][e], __builtin_fmaf(sc, pg[xs][b][e], acc[xs][b][e]));
      }
    }
  }

  // D steps of loads in flight per wave: the first D are issued by
  // prologue() (before the caller waits for the staged scales, so the two
  // memory round trips overlap), and each computed step is refilled with the
  // step D ahead.  Every load is issued unconditionally, since a load on only
  // some paths would make the in-order load counter wait for all in flight;
  // past the wave's range the offset lies outside the resource, so the load
  // returns zeros and touches no memory.
  // loads one prologue issues per thread
  static constexpr int kStepLoads = R * (BITS / 4) + XS * 4 / NXL;

  template <int D>
  __device__ void prologue(uint32_t xro, Step (&st)[D]) {
    set_x(xro);
#pragma unroll
    for (int d = 0; d < D; ++d) {
      load(c_beg + 4 * d, st[d]);
      __builtin_amdgcn_sched_barrier(0);  // keep the steady-state load order
    }
  }

  // partial sums of this wave's K range; lane (n16, h) gets in acc[xs][b]
  // output rows m = 16 xs + 4 h + e of x against W row 16 b + n16
  template <int D>
  __device__ void finish(Step (&st)[D], f32x4v (&acc)[XS][R]) const {
    const uint32_t vmask = opaque(0x000F000Fu), vmagic = opaque(mm_traits<XT, BITS>::magic);
    const uint32_t vones = opaque(mm_traits<XT, BITS>::ones);
    const uint4 ones = make_uint4(vones, vones, vones, vones);
#pragma unroll
    for (int xs = 0; xs < XS; ++xs)
#pragma unroll
      for (int b = 0; b < R; ++b) acc[xs][b] = (f32x4v){0.f, 0.f, 0.f, 0.f};
    // steady state: all D buffered steps are whole steps inside the range, so
    // the body has no branch (a branch around a step makes the compiler's
    // load-counter bookkeeping wait for later steps' loads as well)
    // (the scheduling barriers keep each refill where it is issued: sunk to
    // the end of the body, the loads would arrive a step late)
    int c0 = c_beg;
    for (; c0 + 4 * D <= c_end; c0 += 4 * D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        compute<true>(c0 + 4 * d, st[d], acc, vmask, vmagic, ones);
        __builtin_amdgcn_sched_barrier(0);
        load(c0 + 4 * (d + D), st[d]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // the last D steps or fewer (the final one may end past K)
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (c0 + 4 * d < c_end) compute<false>(c0 + 4 * d, st[d], acc, vmask, vmagic, ones);
  }
};

// LDS of a workgroup: the staged scales and biases, and afterwards (behind a
// barrier) the waves' partial sums in the same space
inline size_t qmvm_lds_bytes(int W, int R, int64_t K, int G, int MR = 8) {
  const size_t sb = (size_t)2 * sb_entries(16 * R, K / G) * 2, part = (size_t)W * 16 * R * MR * 4;
  return sb > part ? sb : part;
}

// sum the W waves' partial sums (lanes h < 2 hold output rows 0..7) through
// LDS (part: [W][16 R][8] floats, free for this use); out(n, m, v) receives
// row n of the 16 R, x row m < 8, value v
// MR: x rows kept (8, 16 when every lane's 4 rows count, 32 with two x sets
// of 16: XS = 2)
template <int W, int R, int MR, int XS, typename F>
__device__ __forceinline__ void reduce_out(float *part, int wave, int lane,
                                           const f32x4v (&acc)[XS][R], F out) {
  const int n16 = lane & 15, h = lane >> 4;
  if (h < MR / XS / 4) {
#pragma unroll
    for (int xs = 0; xs < XS; ++xs)
#pragma unroll
      for (int b = 0; b < R; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          part[(wave * 16 * R + 16 * b + n16) * MR + 16 * xs + 4 * h + e] = acc[xs][b][e];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * R * MR; i += 64 * W) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) v += part[w * 16 * R * MR + i];
    out(i / MR, i % MR, v);
  }
}

// S > 1 (XR = 16 or 32): x has up to XR S rows, run as S slices of XR rows;
// the S slices of one block of W rows are consecutive workgroups of one XCD
// (block b runs on XCD b % 8), so that block is read from HBM once and the
// other slices find it in that XCD's L2.  Workgroup b covers rows
// [b * stride, b * stride + stride), stride <= 16 R (rows past the stride or
// past N read as zero and are not stored).
template <typename XT, int BITS, int W, int GS, int XR, int R>
__global__ __launch_bounds__(64 * W) void qmvm_kernel(const uint16_t *__restrict__ x, int M,
                                                      const uint32_t *__restrict__ codes,
                                                      const uint16_t *__restrict__ scales,
                                                      const uint16_t *__restrict__ biases,
                                                      int64_t N, int64_t K, int kw,
                                                      uint16_t *__restrict__ y, int S, int stride) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];  // [2][16 R][gpr]; then partials
  typedef MBlock<XT, BITS, W, GS, XR, R> Blk;
  constexpr int MR = XR >= 16 ? XR : 8;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t rb = blockIdx.x;
  if (S > 1) {
    const int64_t k = blockIdx.x >> 3;
    const int sl = (int)(k % S);
    rb = (k / S) * 8 + (blockIdx.x & 7);
    x += (int64_t)sl * XR * K;
    y += (int64_t)sl * XR * N;
    M = M - XR * sl < XR ? M - XR * sl : XR;
  }
  const int64_t row0 = rb * stride;
  if (row0 >= N) return;  // padding of the slice mapping (uniform, before any barrier)
  const int64_t nrows = N - row0 < stride ? N - row0 : stride;
  const int64_t gpr = (K >> 5) >> GS;
  Blk blk;
  blk.setup(codes + row0 * (K >> 5) * BITS, nrows, K, kw, wave, lane, lds,
            mk_rsrc(x, (int64_t)M * K * 2));  // rows of x past M read as zero
  const uint32_t xro = (uint32_t)((int64_t)((lane & 15) % Blk::XRS) * K * 2);
  // 4-bit single-block workgroups of 8 waves (long rows, see qmvm_shape) keep
  // a third step in flight: measured at 4096 x 14336, M = 2 .. 8, 11.3 .. 14.2
  // us against 12.2 .. 14.3 with two (and 11.5 .. 14.9 on 16 waves)
  constexpr int D = BITS == 4 && R == 1 && W == 8 && XR < 16 ? 3 : kDepth<BITS>;
  typename Blk::Step st[D];
  // staging first, then the first steps' loads: one round trip covers both
  Blk::stage_sb(scales + row0 * gpr, biases ? biases + row0 * gpr : nullptr, nrows, gpr, lds, wave, lane);
  __builtin_amdgcn_sched_barrier(0);
  blk.template prologue<D>(xro, st);
  Blk::template stage_sb_wait<D * Blk::kStepLoads>(scales + row0 * gpr, biases ? biases + row0 * gpr : nullptr,
                                                   nrows, gpr, lds);
  __syncthreads();
  f32x4v acc[Blk::XS][R];
  blk.template finish<D>(st, acc);
  __syncthreads();  // every wave is done with the staged scales
  reduce_out<W, R, MR, Blk::XS>(reinterpret_cast<float *>(lds), wave, lane, acc, [&](int nn, int m, float v) {
    if (m < M && nn < nrows) y[(int64_t)m * N + row0 + nn] = xtraits<XT>::from_f32(v);
  });
}

// Mixture-of-experts gather ("Quantization", metalworking, gather variants
// for MoE experts): y[t, j, :] = x[t] @ W_{ids[t, j]}^T.  One workgroup per
// (16 R rows, expert e) collects the (token, slot) pairs routed to e and runs
// them in batches through the matrix cores (with WIDE, 16 x rows while more
// than 8 pairs are left; else 8, the lighter form with two K chunks per MFMA
// slot), so each expert's rows are read once per batch of tokens that chose
// it (experts no token chose are never read).  Pairs whose id is outside [0, E) get zero
// rows, written by the workgroups of expert 0.
constexpr int kGTile = 256;  // ids scanned per round

template <typename XT, int BITS, int W, int GS, int R, bool WIDE>
__global__ __launch_bounds__(64 * W) void gather_qmvm_kernel(
    const uint16_t *__restrict__ x, int64_t T, const uint32_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ biases, int64_t E, int64_t N,
    int64_t K, const int32_t *__restrict__ ids, int topk, int kw, uint16_t *__restrict__ y) {
  __shared__ int list[kGTile];
  __shared__ int count;  // pairs of the current round in list
  __shared__ int later;  // set if this expert has pairs past the first round
  __shared__ __attribute__((aligned(16))) float part[W * 16 * R * (WIDE ? 16 : 8)];
  extern __shared__ __attribute__((aligned(16))) uint16_t sbl[];  // [2][16 R][gpr]
  typedef MBlock<XT, BITS, W, GS, 8, R> Blk;
  typedef MBlock<XT, BITS, W, GS, 16, R> Blk16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int e = blockIdx.y;
  const int64_t row0 = (int64_t)blockIdx.x * Blk::ROWS;
  const int64_t nrows = N - row0 < Blk::ROWS ? N - row0 : Blk::ROWS;
  const int64_t gpr = (K >> 5) >> GS, wpe = N * (K >> 5) * BITS;
  const int64_t total = T * topk;

  // pairs with an id outside the table: zero rows (expert-0 workgroups)
  if (e == 0)
    for (int64_t p = threadIdx.x; p < total; p += 64 * W) {
      const int32_t id = ids[p];
      if (id < 0 || id >= E)
        for (int nn = 0; nn < nrows; ++nn) y[p * N + row0 + nn] = 0;
    }
  // does any pair choose this expert?  (if not, nothing of it is read)  The
  // same scan lists the first round's pairs.
  if (threadIdx.x == 0) {
    count = 0;
    later = 0;
  }
  __syncthreads();
  for (int64_t p = threadIdx.x; p < total; p += 64 * W)
    if (ids[p] == e) {
      if (p < kGTile) list[atomicAdd(&count, 1)] = (int)p;
      else later = 1;
    }
  __syncthreads();
  if (count == 0 && later == 0) return;

  const uint32_t *wrows = codes + e * wpe + row0 * (K >> 5) * BITS;
  const __amdgpu_buffer_rsrc_t rx = mk_rsrc(x, T * K * 2);
  Blk blk;
  blk.setup(wrows, nrows, K, kw, wave, lane, sbl, rx);
  Blk::stage_sb(scales + (e * N + row0) * gpr, biases ? biases + (e * N + row0) * gpr : nullptr, nrows, gpr, sbl,
                wave, lane);
  Blk::template stage_sb_wait<0>(scales + (e * N + row0) * gpr, biases ? biases + (e * N + row0) * gpr : nullptr,
                                 nrows, gpr, sbl);
  constexpr int D = kDepth<BITS>;
  for (int64_t t0 = 0; t0 < total; t0 += kGTile) {
    if (t0 > 0) {  // uniform; the first round's list is already built
      if (threadIdx.x == 0) count = 0;
      __syncthreads();
      for (int i = threadIdx.x; i < kGTile; i += 64 * W) {
        const int64_t p = t0 + i;
        if (p < total && ids[p] == e) list[atomicAdd(&count, 1)] = (int)i;
      }
    }
    __syncthreads();  // publishes the list (and, first, the staged scales)
    const int n = count;
    for (int b0 = 0; b0 < n;) {
      // slot row m = n16 % (batch rows) carries pair list[b0 + m]; missing
      // pairs read past the x resource (zeros)
      const auto xrow = [&](int m) {
        return b0 + m < n ? (uint32_t)(((t0 + list[b0 + m]) / topk) * K * 2)
                          : (uint32_t)(T * K * 2);
      };
      const auto store = [&](int nn, int mm, float v) {
        if (b0 + mm < n && row0 + nn < N)
          y[(t0 + list[b0 + mm]) * N + row0 + nn] = xtraits<XT>::from_f32(v);
      };
      f32x4v acc[1][R];
      if (WIDE && n - b0 > 8) {  // uniform
        Blk16 wide;
        wide.setup(wrows, nrows, K, kw, wave, lane, sbl, rx);
        typename Blk16::Step st[D];
        wide.template prologue<D>(xrow(lane & 15), st);
        wide.template finish<D>(st, acc);
        reduce_out<W, R, 16, 1>(part, wave, lane, acc, store);
        __syncthreads();  // part and list reused
        b0 += 16;
      } else {
        typename Blk::Step st[D];
        blk.template prologue<D>(xrow(lane & 7), st);
        blk.template finish<D>(st, acc);
        reduce_out<W, R, 8, 1>(part, wave, lane, acc, store);
        __syncthreads();
        b0 += 8;
      }
    }
  }
}

template <typename XT, int BITS, int W, int XR, int R>
hipError_t qmvm_go(const void *x, int M, const uint32_t *codes, const uint16_t *scales,
                   const uint16_t *biases, int64_t N, int64_t K, int G, void *y, hipStream_t s) {
  const int64_t steps = (K + kStepK - 1) / kStepK;
  const int kw = (int)((steps + W - 1) / W) * kStepK;  // k per wave, whole steps
  const int S = XR >= 16 ? (M + XR - 1) / XR : 1;  // slices of XR x rows
  // rows per workgroup: 16 R, except for tall matrices with one slice, where
  // the rows are dealt evenly over a whole number of workgroups per compute
  // unit (14336 rows: 512 workgroups of 28 rather than 448 of 32, which left
  // 192 compute units two workgroups and 64 one; each compute unit's
  // second workgroup cost about 4.5 us; with four blocks, 256 workgroups of
  // 56 rather than 224 of 64: M = 16, 4-bit 14.9 -> 14.5 us, 8-bit 18.5 -> 17.7)
  int stride = 16 * R;
  if (S == 1 && (R == 2 || R == 4)) {
    const int64_t cus = device_cus();
    const int64_t per_cu = (N + 16 * R * cus - 1) / (16 * R * cus);
    stride = (int)((N + per_cu * cus - 1) / (per_cu * cus));
  }
  const int64_t blocks = (N + stride - 1) / stride;
  const int64_t grid_blocks = S > 1 ? (blocks + 7) / 8 * 8 * S : blocks;
  if (grid_blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)grid_blocks), block(64 * W);
  const size_t lds = qmvm_lds_bytes(W, R, K, G, XR >= 16 ? XR : 8);
  switch (G) {
    case 32: hipLaunchKernelGGL((qmvm_kernel<XT, BITS, W, 0, XR, R>), grid, block, lds, s, (const uint16_t *)x, M, codes, scales, biases, N, K, kw, (uint16_t *)y, S, stride); break;
    case 64: hipLaunchKernelGGL((qmvm_kernel<XT, BITS, W, 1, XR, R>), grid, block, lds, s, (const uint16_t *)x, M, codes, scales, biases, N, K, kw, (uint16_t *)y, S, stride); break;
    case 128: hipLaunchKernelGGL((qmvm_kernel<XT, BITS, W, 2, XR, R>), grid, block, lds, s, (const uint16_t *)x, M, codes, scales, biases, N, K, kw, (uint16_t *)y, S, stride); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// staged scales and biases of a gather workgroup of R blocks
inline size_t gather_lds_bytes(int R, int64_t K, int G) {
  return (size_t)2 * sb_entries(16 * R, K / G) * 2;
}

template <typename XT, int BITS, int R, int W, bool WIDE = true>
hipError_t gather_go(const void *x, int64_t T, const uint32_t *codes, const uint16_t *scales,
                     const uint16_t *biases, int64_t E, int64_t N, int64_t K,
                     const int32_t *ids, int topk, int G, void *y, hipStream_t s) {
  const int64_t steps = (K + kStepK - 1) / kStepK;
  const int kw = (int)((steps + W - 1) / W) * kStepK;
  const int64_t blocks = (N + 16 * R - 1) / (16 * R);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks, (unsigned)E), block(64 * W);
  const size_t lds = gather_lds_bytes(R, K, G);
  switch (G) {
    case 32: hipLaunchKernelGGL((gather_qmvm_kernel<XT, BITS, W, 0, R, WIDE>), grid, block, lds, s, (const uint16_t *)x, T, codes, scales, biases, E, N, K, ids, topk, kw, (uint16_t *)y); break;
    case 64: hipLaunchKernelGGL((gather_qmvm_kernel<XT, BITS, W, 1, R, WIDE>), grid, block, lds, s, (const uint16_t *)x, T, codes, scales, biases, E, N, K, ids, topk, kw, (uint16_t *)y); break;
    case 128: hipLaunchKernelGGL((gather_qmvm_kernel<XT, BITS, W, 2, R, WIDE>), grid, block, lds, s, (const uint16_t *)x, T, codes, scales, biases, E, N, K, ids, topk, kw, (uint16_t *)y); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// dynamic LDS of one workgroup at most (scales and biases of its rows)
constexpr size_t kMaxStagedLds = 64 * 1024;

}  // namespace

bool qmvm_supported(int M, int bits, int64_t N, int64_t K, int G) {
  return M >= 2 && M <= kQmvmMaxRows && (bits == 4 || bits == 8) && N >= 1 && K >= 32 &&
         32 * K * 2 <= 0x7FFFFFFF && qmvm_lds_bytes(16, 1, K, G, 32) <= kMaxStagedLds;
}

bool qmvm_preferred(int64_t M, int bits, int64_t N, int64_t K, int G) {
  // Past 8 rows each slice of x rows costs about one pass over W (11-14 us at
  // 14336 x 4096 and 4096 x 14336, 4-bit and 8-bit, on the MI355X), while the
  // prefill kernel computes whole 256 x 256 tiles, ceil(N / 256) of them per
  // 256 rows: at most 256 rows it takes 62-68 us at 14336 x 4096 and about
  // 200 us at 4096 x 14336 (16 tiles).  Measured crossover: M = 96 .. 128 at
  // N = 14336; with fewer tiles than an eighth of the compute units the
  // slices win up to 256 rows.
  if (M > kQmvmMaxRows || !qmvm_supported((int)M, bits, N, K, G)) return false;
  const int64_t qmm_tiles = (M + 255) / 256 * ((N + 255) / 256);
  return M <= 64 || qmm_tiles * 8 < device_cus();
}

void qmvm_shape(int M, int bits, int64_t N, int64_t K, int G, int &R, int &W, int &XR) {
  // Past 16 rows, two sets of 16 x rows per wave (each weight chunk loaded
  // and unpacked once for 32 rows of x) when the slices of 32 still fill the
  // chip with two row blocks per workgroup; else slices of 16.  Measured at
  // 14336 x 4096, 4-bit: M = 17 / 32 / 128 take 19.8 / 24.6 / 72.6 us in
  // slices of 32, 27.1 / 28.0 / 83.9 us in slices of 16; at 4096 x 14336,
  // M = 17 .. 32, slices of 16 are faster (23.6 .. 24.4 against 24.9 .. 33.6).
  XR = M <= 4 ? 4 : M <= 8 ? 8 : M <= 16 ? 16
       : (N + 31) / 32 * ((M + 31) / 32) >= device_cus() ? 32 : 16;
  const int64_t S = XR >= 16 ? (M + XR - 1) / XR : 1;  // slices of XR x rows
  if (XR >= 16) {
    // 16 or 32 rows per slot: four blocks of 16 rows over 4 waves while the
    // 64-row workgroups still give at least 3/4 of one per compute unit (each
    // x load then serves 64 rows of W: at 14336 x 4096, M = 16 / 64, 4-bit
    // 15.9 / 43.9 -> 14.9 / 33.4 us, 8-bit 20.6 / 50.3 -> 18.6 / 41.6; 8
    // waves were slower; at 4096 x 14336, 64 or 128 workgroups, 1.3-1.8x
    // slower than two blocks)
    if ((N + 63) / 64 * S * 4 >= 3 * device_cus() &&
        qmvm_lds_bytes(4, 4, K, G, XR) <= kMaxStagedLds) {
      R = 4;
      W = 4;
      return;
    }
    // else two blocks of 16 rows over 4 waves whenever that still gives a
    // workgroup per compute unit (measured best at 14336 x 4096 from M = 9
    // and at 4096 x 14336 from M = 17, both widths)
    if ((N + 31) / 32 * S >= device_cus() && qmvm_lds_bytes(4, 2, K, G, XR) <= kMaxStagedLds) {
      R = 2;
      W = 4;
      return;
    }
  }
  // Tall matrices: up to 2 blocks of 16 rows per workgroup (half the x loads
  // per weight byte), rows dealt evenly (qmvm_go), K split over 4 waves
  // (measured at 14336 x 4096, M = 2 / 8: 4-bit 12.0 / 12.1 us against
  // 12.8 / 13.7 with 8 waves and 32-row workgroups; 8-bit 13.7 / 14.9 against
  // 14.1 / 16.0).  Otherwise one block, K split over W waves so that the grid
  // has about four waves per SIMD (each wave then runs a few steps).
  // Measured on the MI355X at N x K = 14336 x 4096 and 4096 x 14336,
  // M = 2..8: more blocks per workgroup leave too few waves, deeper load
  // pipelines gain nothing; 8-bit steps carry twice the bytes and run best
  // with half the waves.
  const int64_t target = 4 * 4 * (int64_t)device_cus();
  R = XR < 16 && N >= 8192 && qmvm_lds_bytes(4, 2, K, G) <= kMaxStagedLds ? 2 : 1;
  if (R == 2) {
    W = 4;
    return;
  }
  // workgroups: row blocks, times the slices
  const int64_t rowblocks = (N + 15) / 16 * S;
  W = rowblocks * 2 >= target ? 2
      : rowblocks * 4 >= target ? 4
      : rowblocks * 8 >= target ? 8 : 16;
  if (bits == 8 && W > 2) W /= 2;
  // Long rows at 4-bit: halve the waves when that gives each wave 8 steps or
  // more and still leaves 2 waves per SIMD (4096 x 14336: 16 waves of 7 steps
  // -> 8 waves of 14, with three steps in flight, qmvm_kernel; M = 2 / 4 / 8
  // 11.3 / 11.8 / 14.2 us against 11.5 / 12.6 / 14.9)
  const int64_t steps = (K + kStepK - 1) / kStepK;
  if (bits == 4 && XR < 16 && W == 16 && (steps + 15) / 16 < 8 && (steps + 7) / 8 >= 8 &&
      rowblocks * 8 >= target / 2)
    W = 8;
}

hipError_t launch_qmvm(const void *x, int x_dtype, int M, const uint32_t *codes,
                       const uint16_t *scales, const uint16_t *biases, int64_t N, int64_t K, int G,
                       int bits, void *y, hipStream_t s) {
  int R, W, XR;
  qmvm_shape(M, bits, N, K, G, R, W, XR);
#define AQ_QMVM_W(T, B, XR, RR) \
  switch (W) { \
    case 2: return qmvm_go<T, B, 2, XR, RR>(x, M, codes, scales, biases, N, K, G, y, s); \
    case 4: return qmvm_go<T, B, 4, XR, RR>(x, M, codes, scales, biases, N, K, G, y, s); \
    case 8: return qmvm_go<T, B, 8, XR, RR>(x, M, codes, scales, biases, N, K, G, y, s); \
    default: return qmvm_go<T, B, 16, XR, RR>(x, M, codes, scales, biases, N, K, G, y, s); \
  }
#define AQ_QMVM_R(T, B, XR) \
  if constexpr (XR >= 16) { \
    if (R == 4) return qmvm_go<T, B, 4, XR, 4>(x, M, codes, scales, biases, N, K, G, y, s); \
  } \
  if (R == 2) { \
    return qmvm_go<T, B, 4, XR, 2>(x, M, codes, scales, biases, N, K, G, y, s); \
  } else { AQ_QMVM_W(T, B, XR, 1) }
#define AQ_QMVM(T) \
  if (bits == 4) { \
    if (XR == 4) { AQ_QMVM_R(T, 4, 4) } else if (XR == 8) { AQ_QMVM_R(T, 4, 8) } \
    else if (XR == 16) { AQ_QMVM_R(T, 4, 16) } else { AQ_QMVM_R(T, 4, 32) } \
  } else { \
    if (XR == 4) { AQ_QMVM_R(T, 8, 4) } else if (XR == 8) { AQ_QMVM_R(T, 8, 8) } \
    else if (XR == 16) { AQ_QMVM_R(T, 8, 16) } else { AQ_QMVM_R(T, 8, 32) } \
  }
  if (x_dtype == X_BF16) { AQ_QMVM(bf16_t) }
  if (x_dtype == X_F16) { AQ_QMVM(f16_t) }
#undef AQ_QMVM
#undef AQ_QMVM_R
#undef AQ_QMVM_W
  return hipErrorInvalidValue;
}


bool gather_qmvm_supported(int bits, int64_t K, int G) {
  return (bits == 4 || bits == 8) && K >= 32 && gather_lds_bytes(1, K, G) <= kMaxStagedLds;
}

hipError_t launch_gather_qmvm(const void *x, int x_dtype, int64_t T, const uint32_t *codes,
                              const uint16_t *scales, const uint16_t *biases, int64_t E, int64_t N,
                              int64_t K, const int32_t *ids, int topk, int G, int bits,
                              void *y, hipStream_t s) {
  // 4 blocks of 16 rows per workgroup, K split over 2 waves (the x rows of a
  // batch are loaded once per 64 rows; the grid is (rows / 64) x experts),
  // fewer blocks if the staged scales would not fit.  With at most one pair
  // per expert on average (decode of a few tokens) each workgroup has a
  // single batch and the launch is latency-bound: 2 blocks over 4 waves give
  // the touched experts four times the waves (measured 15-36% faster at 1-8
  // tokens of 64 experts, top-6; slower from about 3 pairs per expert on).
  // That launch leaves out the 16-row batches: they serve experts with more
  // than 8 pairs, and their registers cost it about 1 us.
  const bool few = T * topk <= E;
#define AQ_GATHER_B(XT, B) \
  if (few && gather_lds_bytes(2, K, G) <= kMaxStagedLds) return gather_go<XT, B, 2, 4, false>(x, T, codes, scales, biases, E, N, K, ids, topk, G, y, s); \
  if (gather_lds_bytes(4, K, G) <= kMaxStagedLds) return gather_go<XT, B, 4, 2>(x, T, codes, scales, biases, E, N, K, ids, topk, G, y, s); \
  if (gather_lds_bytes(2, K, G) <= kMaxStagedLds) return gather_go<XT, B, 2, 2>(x, T, codes, scales, biases, E, N, K, ids, topk, G, y, s); \
  return gather_go<XT, B, 1, 2>(x, T, codes, scales, biases, E, N, K, ids, topk, G, y, s);
#define AQ_GATHER(XT) \
  if (bits == 4) { AQ_GATHER_B(XT, 4) } else { AQ_GATHER_B(XT, 8) }
  if (x_dtype == X_BF16) { AQ_GATHER(bf16_t) }
  if (x_dtype == X_F16) { AQ_GATHER(f16_t) }
#undef AQ_GATHER
#undef AQ_GATHER_B
  return hipErrorInvalidValue;
}

}  // namespace aq

