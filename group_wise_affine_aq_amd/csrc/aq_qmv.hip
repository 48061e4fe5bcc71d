// aq_qmv.hip -- quantized matrix-vector kernels (decode, 1 <= M <= 8) and the
// mixture-of-experts gather variant, for gfx950.
//
// The operation is y = x @ W^T with W given as packed codes + per-group fp16
// scale/bias and dequantized in registers on every use ("Quantization",
// metalworking MLX notes: QMV is a bandwidth-shaped reduction that
// dequantizes in registers; "Tutorial 10: Quantization", s.5, transpose=True).
//
// Design (MI355X): the weights are streamed from HBM exactly once.
//  * A workgroup of 4 waves owns 4*R consecutive rows of W; each wave owns R
//    of them.  The lanes of a wave split K into 32-code chunks (chunk c of a
//    row = BITS words): lane l takes chunks l, l+64, l+128, ... so every load
//    instruction of a wave reads 64 adjacent chunks of one row (fully
//    coalesced 16-byte loads for 4- and 8-bit codes).
//  * x (M rows) is staged in LDS once per workgroup and K-slice, already
//    permuted into the pair order the unpacked codes come out in, laid out
//    quarter-major so 64 lanes reading 16 bytes each hit 64 distinct banks.
//    The per-chunk sums of x sit next to it.
//  * Codes become packed 16-bit pairs with one AND-OR per pair: OR-ing a code
//    q < 1024 into the fp16 exponent pattern of 1024.0 gives exactly 1024 + q
//    (bf16: 128.0, q < 128).  One v_dot2 per pair accumulates
//    D = sum x * (OFF + q) in binary32; the group identity
//      sum_k x_k (q_k s + b) = s * D + (b - OFF*s) * sum_k x_k
//    applies scale and bias once per chunk and row.  For bf16 with 8-bit
//    codes (q up to 255 does not fit that trick) the codes go through
//    v_cvt_f32_ubyte and OFF = 0.
//  * Two passes of loads are kept in flight per wave (software pipelining);
//    partial sums are reduced across the wave with DPP at the end.
#include <type_traits>

#include "aq_device.hpp"
#include "aq_internal.hpp"

namespace aq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunkLdsBytes = 72;   // 32 x values (64 B) + two partial sums (8 B), per row
constexpr int kLdsBudget = 80 * 1024;
constexpr int kGatherTile = 256;      // ids scanned per round in the gather kernel

template <int BITS, typename XT>
struct pairing {
  static constexpr bool is_f16 = std::is_same<XT, f16_t>::value;
  // bf16 cannot represent 128 + q for q >= 128: convert through binary32 instead
  static constexpr bool cvt = !is_f16 && BITS == 8;
  // b | 32: word j holds P = 32/BITS codes; pairs are (i, i + P/2) so one
  // shift + AND-OR serves two codes.  Otherwise pairs are (2p, 2p+1).
  static constexpr bool split = (32 % BITS == 0) && !cvt;
  static constexpr uint32_t magic = is_f16 ? 0x64006400u : 0x43004300u;
  static constexpr float offset = cvt ? 0.f : (is_f16 ? 1024.f : 128.f);
  // 4-bit codes with fp16: the upper nibble of each byte is masked in place
  // (bits 4..7 of the fp16 mantissa), giving 1024 + 16q exactly, so a word
  // needs one shift instead of three.  Those pairs ("odd" codes 1,3,5,7 of a
  // word) accumulate separately and are rescaled by 1/16.
  static constexpr bool nibble = is_f16 && BITS == 4;
};

// chunk position (0..31) of the x value placed in slot t of the permuted chunk
template <int BITS, typename XT>
__device__ __forceinline__ constexpr int perm_src(int t) {
  if constexpr (!pairing<BITS, XT>::split) {
    return t;
  } else {
    constexpr int P = 32 / BITS, H = P / 2;
    const int p = t >> 1, half = t & 1;
    return (p / H) * P + (p % H) + half * H;
  }
}

// The OR constant of the pair conversion, materialised in a VGPR: a VOP3
// instruction on gfx9 takes no literal and reads at most one SGPR, so with
// the constant in a register (w >> sh) & mask | magic is two instructions
// (shift, v_and_or_b32) instead of three.
__device__ __forceinline__ uint32_t vgpr_const(uint32_t c) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

// 16 packed pairs (OFF + q) of one chunk, in the order perm_src describes
template <int BITS, typename XT>
__device__ __forceinline__ void unpack_pairs(const uint32_t *w, uint32_t *qp, uint32_t magic) {
  using PR = pairing<BITS, XT>;
  if constexpr (PR::nibble) {
    // word j -> pairs 4j..4j+3 = (q0,q4), 16*(q1,q5), (q2,q6), 16*(q3,q7)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w8 = w[j] >> 8;
      qp[4 * j] = (w[j] & 0x000F000Fu) | magic;
      qp[4 * j + 1] = (w[j] & 0x00F000F0u) | magic;
      qp[4 * j + 2] = (w8 & 0x000F000Fu) | magic;
      qp[4 * j + 3] = (w8 & 0x00F000F0u) | magic;
    }
  } else if constexpr (PR::split) {
    constexpr int P = 32 / BITS, H = P / 2;
    constexpr uint32_t m2 = ((1u << BITS) - 1u) * 0x10001u;
#pragma unroll
    for (int j = 0; j < BITS; ++j)
#pragma unroll
      for (int i = 0; i < H; ++i) qp[j * H + i] = ((w[j] >> (BITS * i)) & m2) | magic;
  } else if constexpr (PR::cvt) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t f0 = __builtin_bit_cast(uint32_t, (float)(w[j] & 0xFFu));
      const uint32_t f1 = __builtin_bit_cast(uint32_t, (float)((w[j] >> 8) & 0xFFu));
      const uint32_t f2 = __builtin_bit_cast(uint32_t, (float)((w[j] >> 16) & 0xFFu));
      const uint32_t f3 = __builtin_bit_cast(uint32_t, (float)(w[j] >> 24));
      // integers below 256 are exact in bf16: keep the upper halves
      qp[2 * j] = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
      qp[2 * j + 1] = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
    }
  } else {
#pragma unroll
    for (int p = 0; p < 16; ++p)
      qp[p] = chunk_code<BITS>(w, 2 * p) | (chunk_code<BITS>(w, 2 * p + 1) << 16) | magic;
  }
}

// A global-memory pointer that is the same in every lane, moved to scalar
// registers (and kept in the global address space) so loads use the
// scalar-base + 32-bit lane-offset addressing form.
typedef const __attribute__((address_space(1))) char gchar;
__device__ __forceinline__ gchar *uniform_ptr(const void *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<gchar *>(((uint64_t)hi << 32) | lo);
}
template <typename T>
__device__ __forceinline__ T gload(gchar *base, uint32_t off) {
  return *reinterpret_cast<const __attribute__((address_space(1))) T *>(base + off);
}
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
// the BITS words of one chunk at byte offset `off` of a uniform row pointer
template <int BITS>
__device__ __forceinline__ void load_chunk_g(gchar *row, uint32_t off, uint32_t *w) {
  if constexpr (BITS % 4 == 0) {
#pragma unroll
    for (int j = 0; j < BITS / 4; ++j) {
      const u32x4v v = gload<u32x4v>(row, off + 16 * j);
      w[4 * j] = v[0]; w[4 * j + 1] = v[1]; w[4 * j + 2] = v[2]; w[4 * j + 3] = v[3];
    }
  } else if constexpr (BITS % 2 == 0) {
#pragma unroll
    for (int j = 0; j < BITS / 2; ++j) {
      const u32x2v v = gload<u32x2v>(row, off + 8 * j);
      w[2 * j] = v[0]; w[2 * j + 1] = v[1];
    }
  } else {
#pragma unroll
    for (int j = 0; j < BITS; ++j) w[j] = gload<uint32_t>(row, off + 4 * j);
  }
}

template <int BITS, int R>
struct PassData {
  uint32_t w[R][BITS];
  uint32_t s[R], b[R];  // fp16 bit patterns; combined only when consumed, so
                        // the loads of later steps stay in flight
};

struct Weights {
  const uint32_t *codes;
  const uint16_t *scales;
  const uint16_t *biases;  // null: every bias is +0
};

// A buffer resource over `bytes` bytes at a base that is the same in every
// lane (moved to scalar registers).  Loads at offsets past `bytes` return 0
// without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void *base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(((uint64_t)hi << 32) | lo), 0,
                                           bytes, 0x00020000);
}

// The fp16 bias at byte offset goff of a row's biases.  Without a bias array
// the resource has size 0, so the load returns 0 (+0.0) without touching
// memory and the kernels need no second code path.
__device__ __forceinline__ uint32_t load_bias(const Weights &wt, int64_t so, int64_t ng,
                                              uint32_t goff) {
  const __amdgpu_buffer_rsrc_t r =
      uniform_rsrc(wt.biases ? wt.biases + so : wt.scales, wt.biases ? (int)(ng * 2) : 0);
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)goff, 0, 0);
}

template <int BITS, int MB, typename XT, int R>
struct QmvCore {
  using PR = pairing<BITS, XT>;

  const Weights wt;
  const int64_t N, K;
  const int nch;     // chunks per row, K / 32
  const int gshift;  // chunk index -> group index: c >> gshift (G = 32 << gshift)

  __device__ QmvCore(const Weights &w, int64_t n, int64_t k, int G)
      : wt(w), N(n), K(k), nch((int)(k >> 5)), gshift(__builtin_ctz((unsigned)G) - 5) {}

  // rows [row0, row0 + R) of W (clamped to the last row; row0 is uniform
  // across the wave), chunk `chunk` (clamped to the last chunk: padding
  // lanes re-read it and multiply zeros)
  __device__ __forceinline__ void load_pass(PassData<BITS, R> &d, int64_t row0, int chunk) const {
    const uint32_t c = (uint32_t)(chunk < nch - 1 ? chunk : nch - 1);
    const uint32_t coff = c * (uint32_t)(BITS * 4);     // byte offset in the row
    const uint32_t goff = (c >> gshift) * 2u;            // byte offset of the group
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int64_t n = row0 + r;
      n = n < N ? n : N - 1;
      gchar *rc = uniform_ptr(wt.codes + n * ((int64_t)nch * BITS));
      const int64_t so = n * (int64_t)(nch >> gshift);
      load_chunk_g<BITS>(rc, coff, d.w[r]);
      d.s[r] = gload<uint16_t>(uniform_ptr(wt.scales + so), goff);
      d.b[r] = load_bias(wt, so, nch >> gshift, goff);
    }
  }

  // one chunk per lane: acc[r][m] += sum over the chunk of x[m, k] * w^[r, k]
  __device__ __forceinline__ void compute_pass(const PassData<BITS, R> &d, const uint8_t *xlds,
                                               const float *xsum, int CP, int c_local, int M,
                                               float (&acc)[R][MB]) const {
    uint32_t qp[R][16];
    float sf[R], bo[R];
    const uint32_t magic = vgpr_const(PR::magic);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      unpack_pairs<BITS, XT>(d.w[r], qp[r], magic);
      sf[r] = f16_to_f32((uint16_t)d.s[r]);
      bo[r] = __builtin_fmaf(-PR::offset, sf[r], f16_to_f32((uint16_t)d.b[r]));
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      if (m < M) {
        uint32_t xv[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 v = *reinterpret_cast<const uint4 *>(xlds + ((size_t)(m * 4 + j) * CP + c_local) * 16);
          xv[4 * j] = v.x; xv[4 * j + 1] = v.y; xv[4 * j + 2] = v.z; xv[4 * j + 3] = v.w;
        }
        if constexpr (PR::nibble) {
          // sums of x over the even and odd codes of each word
          const float2 xs = reinterpret_cast<const float2 *>(xsum)[m * CP + c_local];
#pragma unroll
          for (int r = 0; r < R; ++r) {
            float de = 0.f, dodd = 0.f;
#pragma unroll
            for (int p = 0; p < 16; p += 2) {
              de = dot2(XT{}, xv[p], qp[r][p], de);
              dodd = dot2(XT{}, xv[p + 1], qp[r][p + 1], dodd);
            }
            // sum x (q s + b) = s De + (s/16) Dodd + (b - 1024 s) Xe + (b - 64 s) Xo
            const float bodd = __builtin_fmaf(960.f, sf[r], bo[r]);
            float a = __builtin_fmaf(bo[r], xs.x, acc[r][m]);
            a = __builtin_fmaf(bodd, xs.y, a);
            a = __builtin_fmaf(sf[r], de, a);
            acc[r][m] = __builtin_fmaf(sf[r] * 0.0625f, dodd, a);
          }
        } else {
          const float xs = reinterpret_cast<const float2 *>(xsum)[m * CP + c_local].x;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            float dsum = 0.f;
#pragma unroll
            for (int p = 0; p < 16; ++p) dsum = dot2(XT{}, xv[p], qp[r][p], dsum);
            acc[r][m] = __builtin_fmaf(sf[r], dsum, __builtin_fmaf(bo[r], xs, acc[r][m]));
          }
        }
      }
    }
  }

  // reduce the lane partials of rows [row0, row0 + R) and store them
  __device__ __forceinline__ void finish(float (&acc)[R][MB], int64_t row0, int M,
                                         uint16_t *const (&yr)[MB], int lane) const {
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        if (m < M) {
          const float v = wave_sum(acc[r][m]);
          if (lane == 0 && row0 + r < N) yr[m][row0 + r] = xtraits<XT>::from_f32(v);
        }
        acc[r][m] = 0.f;
      }
    }
  }
};

// One chunk of one row against x held in registers (the M = 1 kernel):
// returns acc + sum over the chunk of x[k] * (q[k] * s + b).
template <int BITS, typename XT>
__device__ __forceinline__ float chunk_dot(const uint32_t *w, uint32_t s16, uint32_t b16,
                                           const uint32_t (&xv)[16], float2 xs, float acc,
                                           uint32_t magic) {
  using PR = pairing<BITS, XT>;
  uint32_t qp[16];
  unpack_pairs<BITS, XT>(w, qp, magic);
  const float sf = f16_to_f32((uint16_t)s16);
  const float bo = __builtin_fmaf(-PR::offset, sf, f16_to_f32((uint16_t)b16));
  if constexpr (PR::nibble) {
    float de = 0.f, dodd = 0.f;
#pragma unroll
    for (int p = 0; p < 16; p += 2) {
      de = dot2(XT{}, xv[p], qp[p], de);
      dodd = dot2(XT{}, xv[p + 1], qp[p + 1], dodd);
    }
    // sum x (q s + b) = s De + (s/16) Dodd + (b - 1024 s) Xe + (b - 64 s) Xo
    float a = __builtin_fmaf(bo, xs.x, acc);
    a = __builtin_fmaf(__builtin_fmaf(960.f, sf, bo), xs.y, a);
    a = __builtin_fmaf(sf, de, a);
    return __builtin_fmaf(sf * 0.0625f, dodd, a);
  } else {
    float d = 0.f;
#pragma unroll
    for (int p = 0; p < 16; ++p) d = dot2(XT{}, xv[p], qp[p], d);
    return __builtin_fmaf(sf, d, __builtin_fmaf(bo, xs.x, acc));
  }
}

// Two-phase staging for the streaming kernel: the x loads are issued before
// the first weight loads, so waiting for x (the in-order load counter)
// never waits for the weights behind it.  Each thread owns chunks
// t, t + 256, ... of the M x CP staged chunks, at most XS of them.
template <int XS>
struct XStage {
  uint4 v[XS][4];
};

template <int BITS, int MB, typename XT, int NT, int XS>
__device__ __forceinline__ void stage_x_load(const uint16_t *const (&xr)[MB], int M, int nvalid,
                                             int CP, XStage<XS> &st) {
#pragma unroll
  for (int i = 0; i < XS; ++i) {
    const int t = threadIdx.x + i * NT;
    const int m = t / CP, c = t - m * CP;
    if (t < M * CP && c < nvalid) {
      const uint16_t *src = nullptr;
#pragma unroll
      for (int mm = 0; mm < MB; ++mm)
        if (mm == m) src = xr[mm];
      const uint4 *p = reinterpret_cast<const uint4 *>(src + (int64_t)c * 32);
#pragma unroll
      for (int q = 0; q < 4; ++q) st.v[i][q] = p[q];
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) st.v[i][q] = make_uint4(0, 0, 0, 0);
    }
  }
}

template <int BITS, int MB, typename XT, int NT, int XS>
__device__ __forceinline__ void stage_x_store(int M, int CP, const XStage<XS> &st, uint8_t *xlds,
                                              float *xsum) {
#pragma unroll
  for (int i = 0; i < XS; ++i) {
    const int t = threadIdx.x + i * NT;
    if (t >= M * CP) break;
    const int m = t / CP, c = t - m * CP;
    uint16_t v[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t uu[4] = {st.v[i][q].x, st.v[i][q].y, st.v[i][q].z, st.v[i][q].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * q + 2 * e] = (uint16_t)(uu[e] & 0xFFFFu);
        v[8 * q + 2 * e + 1] = (uint16_t)(uu[e] >> 16);
      }
    }
    float s_even = 0.f, s_odd = 0.f;
#pragma unroll
    for (int k = 0; k < 32; k += 2) {
      s_even += xtraits<XT>::to_f32(v[k]);
      s_odd += xtraits<XT>::to_f32(v[k + 1]);
    }
    uint32_t out[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      out[k] = (uint32_t)v[perm_src<BITS, XT>(2 * k)] | ((uint32_t)v[perm_src<BITS, XT>(2 * k + 1)] << 16);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint4 *>(xlds + ((size_t)(m * 4 + j) * CP + c) * 16) =
          make_uint4(out[4 * j], out[4 * j + 1], out[4 * j + 2], out[4 * j + 3]);
    reinterpret_cast<float2 *>(xsum)[m * CP + c] =
        pairing<BITS, XT>::nibble ? make_float2(s_even, s_odd) : make_float2(s_even + s_odd, 0.f);
  }
}

// Stage x rows (pointers xr[0..M-1]) for chunks [c0, c0 + nvalid) of K into
// LDS in the permuted, quarter-major layout; chunks nvalid..CP-1 are zero.
template <int BITS, int MB, typename XT>
__device__ __forceinline__ void stage_x(const uint16_t *const (&xr)[MB], int M, int64_t c0,
                                        int nvalid, int CP, uint8_t *xlds, float *xsum) {
  for (int t = threadIdx.x; t < M * CP; t += kThreads) {
    const int m = t / CP, c = t - m * CP;
    uint32_t out[16];
    float s_even = 0.f, s_odd = 0.f;
    if (c < nvalid) {
      const uint16_t *src = nullptr;
#pragma unroll
      for (int mm = 0; mm < MB; ++mm)
        if (mm == m) src = xr[mm];
      const uint4 *p = reinterpret_cast<const uint4 *>(src + (c0 + c) * 32);
      uint16_t v[32];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 u = p[q];
        const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[8 * q + 2 * e] = (uint16_t)(uu[e] & 0xFFFFu);
          v[8 * q + 2 * e + 1] = (uint16_t)(uu[e] >> 16);
        }
      }
#pragma unroll
      for (int i = 0; i < 32; i += 2) {
        s_even += xtraits<XT>::to_f32(v[i]);
        s_odd += xtraits<XT>::to_f32(v[i + 1]);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i)
        out[i] = (uint32_t)v[perm_src<BITS, XT>(2 * i)] | ((uint32_t)v[perm_src<BITS, XT>(2 * i + 1)] << 16);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) out[i] = 0;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint4 *>(xlds + ((size_t)(m * 4 + j) * CP + c) * 16) =
          make_uint4(out[4 * j], out[4 * j + 1], out[4 * j + 2], out[4 * j + 3]);
    // nibble path: (sum over even codes, sum over odd codes); otherwise (total, 0)
    reinterpret_cast<float2 *>(xsum)[m * CP + c] =
        pairing<BITS, XT>::nibble ? make_float2(s_even, s_odd) : make_float2(s_even + s_odd, 0.f);
  }
}

// Full K reduction for one workgroup's rows against M staged x rows, slice
// by slice (x re-staged per slice when M*K does not fit in LDS at once);
// writes y rows yr[m][n].
template <int BITS, int MB, typename XT, int R>
__device__ __forceinline__ void qmv_rows(const Weights &wt, int64_t N, int64_t K, int G,
                                         int rowblk, const uint16_t *const (&xr)[MB],
                                         uint16_t *const (&yr)[MB], int M, int CPmax,
                                         uint8_t *smem) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t row0 = (int64_t)rowblk * (kWaves * R) + wave * R;
  const QmvCore<BITS, MB, XT, R> core(wt, N, K, G);
  uint8_t *xlds = smem;
  float *xsum = reinterpret_cast<float *>(smem + (size_t)M * CPmax * 64);

  float acc[R][MB];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[r][m] = 0.f;

  const int64_t nchunks = K >> 5;
  for (int64_t c0 = 0; c0 < nchunks; c0 += CPmax) {
    const int nvalid = (int)((nchunks - c0) < CPmax ? (nchunks - c0) : CPmax);
    const int CP = (nvalid + 63) & ~63;  // padded to whole passes
    const int cpl = CP >> 6;
    PassData<BITS, R> A, B;
    core.load_pass(A, row0, (int)c0 + lane);
    __syncthreads();  // previous slice fully consumed
    stage_x<BITS, MB, XT>(xr, M, c0, nvalid, CP, xlds, xsum);
    __syncthreads();
    for (int p = 0; p < cpl; p += 2) {
      const bool has1 = p + 1 < cpl;
      if (has1) core.load_pass(B, row0, (int)c0 + (p + 1) * 64 + lane);
      core.compute_pass(A, xlds, xsum, CP, p * 64 + lane, M, acc);
      if (has1) {
        if (p + 2 < cpl) core.load_pass(A, row0, (int)c0 + (p + 2) * 64 + lane);
        core.compute_pass(B, xlds, xsum, CP, (p + 1) * 64 + lane, M, acc);
      }
    }
  }
  core.finish(acc, row0, M, yr, lane);
}

template <int BITS, int MB, typename XT, int R>
__global__ __launch_bounds__(kThreads) void qmv_kernel(const uint16_t *__restrict__ x, int M,
                                                       Weights wt, int64_t N, int64_t K, int G,
                                                       uint16_t *__restrict__ y, int CPmax) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const uint16_t *xr[MB];
  uint16_t *yr[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    xr[m] = x + (int64_t)(m < M ? m : 0) * K;
    yr[m] = y + (int64_t)(m < M ? m : 0) * N;
  }
  qmv_rows<BITS, MB, XT, R>(wt, N, K, G, blockIdx.x, xr, yr, M, CPmax, smem);
}

// Persistent streaming variant for the case where all of x fits in LDS:
// x is staged once per workgroup, then every wave walks its units (R rows
// each, units gw, gw + TW, ... over all TW waves of the grid) as one flat
// sequence of (unit, pass) steps.  A D-deep ring of register buffers keeps
// the loads of the next D steps in flight across unit boundaries, so a wave
// never waits for HBM latency between rows.  Finished rows are parked in LDS
// and written out after the loop: a global store inside it would share the
// in-order memory counter with the loads and force the compiler to drain
// every load in flight.
constexpr int kStreamRound = 32;  // units per wave between output flushes

template <int BITS, int MB, typename XT, int R, int D, int W, int XS>
__global__ __launch_bounds__(64 * W) void qmv_stream_kernel(const uint16_t *__restrict__ x,
                                                              int M, Weights wt, int64_t N,
                                                              int64_t K, int G,
                                                              uint16_t *__restrict__ y, int CP) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const uint16_t *xr[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) xr[m] = x + (int64_t)(m < M ? m : 0) * K;
  const QmvCore<BITS, MB, XT, R> core(wt, N, K, G);
  const int64_t TW = (int64_t)gridDim.x * W, gw = (int64_t)blockIdx.x * W + wave;
  const int64_t U = (N + R - 1) / R;
  const int cpl = CP >> 6;
  const int nunits = gw < U ? (int)((U - 1 - gw) / TW + 1) : 0;

  uint8_t *xlds = smem;
  float *xsum = reinterpret_cast<float *>(smem + (size_t)M * CP * 64);
  uint16_t *obuf = reinterpret_cast<uint16_t *>(smem + (size_t)M * CP * kChunkLdsBytes) +
                   (size_t)wave * kStreamRound * R * MB;

  PassData<BITS, R> buf[D];
  float acc[R][MB];
  bool staged = false;
  XStage<XS> xst;
  stage_x_load<BITS, MB, XT, 64 * W, XS>(xr, M, (int)(K >> 5), CP, xst);
  for (int u0 = 0; u0 < nunits || !staged; u0 += kStreamRound) {
    const int nu = nunits - u0 < kStreamRound ? nunits - u0 : kStreamRound;
    const int64_t S = nu > 0 ? (int64_t)nu * cpl : 0;
    int li = 0, lp = 0;  // next (unit, pass) of this round to load
    auto load_next = [&](PassData<BITS, R> &bb) {
      int i = li, p = lp;
      if (i >= nu) { i = nu - 1; p = cpl - 1; }  // past the end: harmless re-read
      core.load_pass(bb, (gw + (int64_t)(u0 + i) * TW) * R, p * 64 + lane);
      if (++lp == cpl) { lp = 0; ++li; }
    };
    // always D loads (past the end they re-read the last chunk): a fixed
    // count keeps the in-order load counter exact at the loop head
    // (issued in consumption order: the scheduler may not regroup them)
    if (nu > 0) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        load_next(buf[d]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (!staged) {  // the first weight loads are in flight while x is stored
      stage_x_store<BITS, MB, XT, 64 * W, XS>(M, CP, xst, xlds, xsum);
      __syncthreads();
      staged = true;
      if (nunits == 0) return;
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MB; ++m) acc[r][m] = 0.f;
    int ci = 0, cp = 0;  // (unit, pass) being computed
    auto consume = [&](PassData<BITS, R> &bb) {
      core.compute_pass(bb, xlds, xsum, CP, cp * 64 + lane, M, acc);
      if (cp == cpl - 1) {  // unit complete: reduce, park in LDS
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int m = 0; m < MB; ++m) {
            if (m < M) {
              const float v = wave_sum(acc[r][m]);
              if (lane == 0) obuf[(ci * R + r) * MB + m] = xtraits<XT>::from_f32(v);
            }
            acc[r][m] = 0.f;
          }
      }
      if (++cp == cpl) { cp = 0; ++ci; }
    };
    int64_t t = 0;
    for (; t + D <= S; t += D) {  // whole rings: no per-step guards
#pragma unroll
      for (int d = 0; d < D; ++d) {
        consume(buf[d]);
        load_next(buf[d]);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d)  // tail: already loaded
      if (t + d < S) consume(buf[d]);
    __builtin_amdgcn_wave_barrier();
    for (int e = lane; e < nu * R * MB; e += 64) {
      const int m = e % MB, r = (e / MB) % R, i = e / (MB * R);
      const int64_t n = (gw + (int64_t)(u0 + i) * TW) * R + r;
      if (m < M && n < N) y[(int64_t)m * N + n] = obuf[e];
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Decode kernel for M = 1 and K <= 64 * 32 * CPL: every lane keeps its CPL x
// chunks (the chunks l, l + 64, ... it multiplies in every row) in
// registers, copied once from the workgroup's LDS copy of x.  The ring of
// D = CPL * UD load buffers holds whole rows, so the pass of every ring slot
// is a compile-time constant.  Rows are dealt to waves round-robin (row gw,
// gw + TW, ...), D steps of loads stay in flight across row boundaries,
// finished rows are parked in LDS and written after the loop (as in the
// M <= 8 streaming kernel).
// A row's scales and biases arrive with SL 4-byte loads of each per lane
// (SL * 128 groups), issued just ahead of the row's first code load; when
// that chunk is consumed the wave writes them into its LDS table as one
// dword per group (scale | bias << 16), from which every chunk of the row
// reads its group.  That replaces two 2-byte loads per chunk (3 vector
// memory instructions per 1 KB of codes become 1 + 2 SL / CPL).  With an
// odd number of groups per row, every other row starts 2 bytes into a
// dword: its loads start at the dword boundary below, so dword j holds
// groups 2 j - 1 and 2 j, and the table entries move down by one (the
// table keeps two spare entries in front for that).
template <int BITS, typename XT, int CPL, int UD, int W, int SL>
__global__ __launch_bounds__(64 * W) void qmv1_kernel(const uint16_t *__restrict__ x, Weights wt,
                                                      int64_t N, int64_t K, int G,
                                                      uint16_t *__restrict__ y) {
  constexpr int D = CPL * UD, CP = 64 * CPL;
  constexpr int XS = (CP + 64 * W - 1) / (64 * W);
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const uint16_t *xr[1] = {x};
  const QmvCore<BITS, 1, XT, 1> core(wt, N, K, G);
  const int64_t TW = (int64_t)gridDim.x * W, gw = (int64_t)blockIdx.x * W + wave;
  const int nunits = gw < N ? (int)((N - 1 - gw) / TW + 1) : 0;
  const int ng = core.nch >> core.gshift;  // groups per row, at most SL * 128

  uint8_t *xlds = smem;
  float *xsum = reinterpret_cast<float *>(smem + (size_t)CP * 64);
  uint16_t *obuf = reinterpret_cast<uint16_t *>(smem + (size_t)CP * kChunkLdsBytes) +
                   (size_t)wave * kStreamRound;
  uint32_t *sbt = reinterpret_cast<uint32_t *>(smem + (size_t)CP * kChunkLdsBytes +
                                               (size_t)W * kStreamRound * 2) +
                  (size_t)wave * (SL * 128 + 2);  // group g at entry 2 + g

  // codes of one chunk of a row (chunk clamped to the last: padding lanes
  // re-read it and multiply zeros)
  auto load_codes = [&](PassData<BITS, 1> &d, int64_t row, int chunk) {
    const uint32_t c = (uint32_t)(chunk < core.nch - 1 ? chunk : core.nch - 1);
    load_chunk_g<BITS>(uniform_ptr(wt.codes + row * ((int64_t)core.nch * BITS)),
                       c * (uint32_t)(BITS * 4), d.w[0]);
  };
  // lane l, load r: groups 2 j - odd and 2 j - odd + 1 of the row, j = l + 64 r,
  // odd = 1 when the row starts 2 bytes into a dword (the scale and bias
  // arrays are 16-byte aligned, so both rows start alike); returns odd.  The
  // range is whole dwords, so a row ending mid-dword still reads its last
  // group (the other half, past the row, lies in the same aligned dword as
  // the array's own bytes and is never used).
  auto stage_load = [&](int64_t row, uint32_t (&ss)[SL], uint32_t (&bb)[SL]) -> int {
    const int64_t so = row * ng;
    const int odd = (int)(so & 1);
    const int bytes = ((ng + odd) * 2 + 3) & ~3;
    const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(wt.scales + so - odd, bytes);
    const __amdgpu_buffer_rsrc_t rb = uniform_rsrc(wt.biases ? wt.biases + so - odd : wt.scales,
                                                   wt.biases ? bytes : 0);
#pragma unroll
    for (int r = 0; r < SL; ++r) {
      ss[r] = __builtin_amdgcn_raw_buffer_load_b32(rs, (lane + 64 * r) * 4, 0, 0);
      bb[r] = __builtin_amdgcn_raw_buffer_load_b32(rb, (lane + 64 * r) * 4, 0, 0);
    }
    return odd;
  };
  auto stage_store = [&](const uint32_t (&ss)[SL], const uint32_t (&bb)[SL], int odd) {
    uint32_t *t = sbt + 2 - odd;
#pragma unroll
    for (int r = 0; r < SL; ++r) {
      const int j = lane + 64 * r;
      t[2 * j] = __builtin_amdgcn_perm(bb[r], ss[r], 0x05040100u);      // low halves
      t[2 * j + 1] = __builtin_amdgcn_perm(bb[r], ss[r], 0x07060302u);  // high halves
    }
  };

  // x loads first, then the first PRE weight loads, then the wait for x:
  // the two round trips overlap.  Those first loads are unconditional (a
  // wave without rows re-reads row N - 1 and stores nothing), so the wait
  // for x leaves weight loads in flight on every path; the scheduling
  // barriers keep that order.  Rows of 5 or more chunks per lane issue only
  // 4 of them before the wait and the rest after it: x's own fetch queues
  // behind every weight request the chip has issued, and with the whole
  // first row requested up front it lands later (4096 x 14336, 4-bit:
  // 8.46 .. 8.57 us against 8.83 .. 8.97 with all 7 up front, 8.53 with 2,
  // 8.7 with 5 or 6).
  XStage<XS> xst;
  stage_x_load<BITS, 1, XT, 64 * W, XS>(xr, 1, (int)(K >> 5), CP, xst);
  __builtin_amdgcn_sched_barrier(0);
  PassData<BITS, 1> buf[D];
  uint32_t stg_s[UD][SL], stg_b[UD][SL];  // staged scale / bias dwords of the rows in flight
  int stg_odd[UD];
  constexpr int PRE = D < 5 ? D : 4;
  auto fill = [&](int d) {  // slot d of the first round
    const int nu = nunits < kStreamRound ? nunits : kStreamRound;
    const int i = d / CPL < nu ? d / CPL : (nu > 0 ? nu - 1 : 0);
    int64_t row = gw + (int64_t)i * TW;
    row = row < N ? row : N - 1;
    if (d % CPL == 0) stg_odd[d / CPL] = stage_load(row, stg_s[d / CPL], stg_b[d / CPL]);
    load_codes(buf[d], row, (d % CPL) * 64 + lane);
  };
#pragma unroll
  for (int d = 0; d < PRE; ++d) {
    fill(d);
    __builtin_amdgcn_sched_barrier(0);
  }
  uint32_t xv[CPL][16];
  float2 xs[CPL];
  stage_x_store<BITS, 1, XT, 64 * W, XS>(1, CP, xst, xlds, xsum);
  __syncthreads();
  if (nunits == 0) return;
#pragma unroll
  for (int d = PRE; d < D; ++d) {
    fill(d);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int p = 0; p < CPL; ++p) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 v = *reinterpret_cast<const uint4 *>(xlds + ((size_t)j * CP + p * 64 + lane) * 16);
      xv[p][4 * j] = v.x; xv[p][4 * j + 1] = v.y; xv[p][4 * j + 2] = v.z; xv[p][4 * j + 3] = v.w;
    }
    xs[p] = reinterpret_cast<const float2 *>(xsum)[p * 64 + lane];
  }
  const uint32_t magic = vgpr_const(pairing<BITS, XT>::magic);
  for (int u0 = 0; u0 < nunits; u0 += kStreamRound) {
    const int nu = nunits - u0 < kStreamRound ? nunits - u0 : kStreamRound;
    auto row_of = [&](int i) -> int64_t {
      i = i < nu ? i : nu - 1;  // past the end: harmless re-read of the last row
      return gw + (int64_t)(u0 + i) * TW;
    };
    if (u0 > 0) {  // the first round was filled above
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (d % CPL == 0)
          stg_odd[d / CPL] = stage_load(row_of(d / CPL), stg_s[d / CPL], stg_b[d / CPL]);
        load_codes(buf[d], row_of(d / CPL), (d % CPL) * 64 + lane);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    float acc = 0.f;
    auto consume = [&](const PassData<BITS, 1> &bb, int p, int unit) {
      const int c = p * 64 + lane < core.nch - 1 ? p * 64 + lane : core.nch - 1;
      const uint32_t sb = sbt[2 + (c >> core.gshift)];
      acc = chunk_dot<BITS, XT>(bb.w[0], sb & 0xFFFFu, sb >> 16, xv[p], xs[p], acc, magic);
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
        if (d % CPL == 0) stage_store(stg_s[d / CPL], stg_b[d / CPL], stg_odd[d / CPL]);
        consume(buf[d], d % CPL, i + d / CPL);
        if (d % CPL == 0)
          stg_odd[d / CPL] = stage_load(row_of(i + UD + d / CPL), stg_s[d / CPL], stg_b[d / CPL]);
        load_codes(buf[d], row_of(i + UD + d / CPL), (d % CPL) * 64 + lane);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d)  // the last < UD rows: already loaded
      if (i + d / CPL < nu) {
        if (d % CPL == 0) stage_store(stg_s[d / CPL], stg_b[d / CPL], stg_odd[d / CPL]);
        consume(buf[d], d % CPL, i + d / CPL);
      }
    __builtin_amdgcn_wave_barrier();
    for (int e = lane; e < nu; e += 64) y[gw + (int64_t)(u0 + e) * TW] = obuf[e];
    __builtin_amdgcn_wave_barrier();
  }
}

// One workgroup per (row block, expert).  It scans the ids, collects the
// (token, slot) pairs routed to its expert and runs them through the
// matrix-vector core in batches of up to MB tokens, so each expert's rows
// are read once per call for every batch of tokens that chose it (experts no
// token chose are never read).
template <int BITS, int MB, typename XT, int R>
__global__ __launch_bounds__(kThreads) void gather_qmv_kernel(
    const uint16_t *__restrict__ x, int64_t T, Weights wt, int64_t E, int64_t N, int64_t K,
    const int32_t *__restrict__ ids, int topk, int G, uint16_t *__restrict__ y, int CPmax) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int *list = reinterpret_cast<int *>(smem + (size_t)MB * CPmax * kChunkLdsBytes);
  int *count = list + kGatherTile;
  const int e = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t wpe = N * ((K >> 5) * BITS), spe = N * (K / G);
  const Weights we{wt.codes + e * wpe, wt.scales + e * spe,
                   wt.biases ? wt.biases + e * spe : nullptr};
  const int64_t total = T * topk;

  for (int64_t t0 = 0; t0 < total; t0 += kGatherTile) {
    __syncthreads();
    if (threadIdx.x == 0) *count = 0;
    __syncthreads();
    const int64_t i = t0 + threadIdx.x;
    const int id = i < total ? ids[i] : -1;
    if (i < total && id == e) list[atomicAdd(count, 1)] = (int)(i - t0);
    // ids outside [0, E): the expert-0 workgroups zero those output rows
    if (e == 0 && i < total && (id < 0 || id >= E)) {
      for (int r = 0; r < kWaves * R; ++r) {
        const int64_t n = (int64_t)blockIdx.x * kWaves * R + r;
        if (n < N) y[i * N + n] = 0;
      }
    }
    __syncthreads();
    const int cnt = *count;
    // keep the order of the pairs deterministic within the batch
    for (int b0 = 0; b0 < cnt; b0 += MB) {
      const int Mb = cnt - b0 < MB ? cnt - b0 : MB;
      const uint16_t *xr[MB];
      uint16_t *yr[MB];
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const int64_t pair = t0 + list[b0 + (m < Mb ? m : 0)];
        xr[m] = x + (pair / topk) * K;
        yr[m] = y + pair * N;
      }
      qmv_rows<BITS, MB, XT, R>(we, N, K, G, blockIdx.x, xr, yr, Mb, CPmax, smem);
    }
  }
  (void)wave;
  (void)lane;
}

// ---- host side -------------------------------------------------------------------------

inline int slice_chunks(int64_t K, int rows) {
  const int64_t nchunks = K >> 5;
  int64_t cap = kLdsBudget / ((int64_t)rows * kChunkLdsBytes);
  cap = cap / 64 * 64;
  if (cap < 64) cap = 64;
  const int64_t need = (nchunks + 63) / 64 * 64;
  return (int)(need < cap ? need : cap);
}

template <typename KernelT>
hipError_t allow_lds(KernelT kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

constexpr int kRows = 2;  // rows per wave, sliced kernel and gather
constexpr int kStreamWaves = 16;  // one 16-wave workgroup per CU shares one x copy
constexpr int kStreamLdsMax = 96 * 1024;


constexpr int kStreamCtasPerCu = 1;
template <int MB> struct stream_shape;
template <> struct stream_shape<1> { static constexpr int R = 1, D = 4; };
template <> struct stream_shape<2> { static constexpr int R = 2, D = 4; };
template <> struct stream_shape<4> { static constexpr int R = 4, D = 2; };
template <> struct stream_shape<8> { static constexpr int R = 4, D = 2; };

}  // namespace

// M = 1 kernel shape: CPL 64-chunk passes per row, UD rows in flight per
// wave, W waves per workgroup, SL staging loads of scales (and of biases) per
// lane and row, and at most WPC workgroups per CU (0: as many as fit).
// Measured on the MI355X (4-bit, cold weights; µs): at K = 4096 fewer waves
// than fit run faster -- 14336 rows: 4-wave workgroups, 3 per CU (3072
// waves) 7.88 .. 8.07, against 8.31 .. 8.42 with 6144 waves (8-wave
// workgroups, all that fit) and 8.05 .. 8.21 with 4096; 4096 rows: one
// 16-wave workgroup per CU, a row per wave, 4.08 .. 4.12, against
// 4.38 .. 4.51 with 2 rows in flight per wave on 8-wave workgroups;
// 1024 rows: one or two rows in flight per wave, 3.14 .. 3.20 either way.
// At K = 14336 (4096 rows, 2 waves per SIMD), 8-wave workgroups
// 8.59 .. 8.75 us against 8.59 .. 8.95 with 4 waves (two rows in flight per
// wave 10.4 .. 10.6), and SL = 2 at G = 64 about 0.05 .. 0.1 us ahead of
// SL = 4.
void qmv1_shape(int64_t N, int64_t K, int G, int &cpl, int &ud, int &w, int &sl, int &wpc) {
  cpl = (int)((K / 32 + 63) / 64);
  ud = cpl == 1 ? 4 : (cpl == 2 && N <= 2048 ? 2 : 1);  // (1 and 2 measured alike at 1024 rows)
  wpc = 0;
  if (cpl == 2 && N > 8192) {
    w = 4;
    wpc = 3;
  } else if (cpl == 2 && N > 2048) {
    w = 16;
    wpc = 1;
  } else {
    // from 5 chunks per lane on, x in registers leaves room for 2 waves per
    // SIMD: one workgroup of 8 waves per CU stages x once for all of them
    w = cpl >= 5 ? 8 : 4;
  }
  // 4-byte staging loads per lane: 128 groups each, in powers of two
  const int groups = (64 * cpl * 32) / G;
  sl = groups <= 128 ? 1 : (groups <= 256 ? 2 : 4);
}

namespace {

template <int BITS, typename XT, int CPL, int UD, int W, int SL>
hipError_t qmv1_launch(const void *x, const Weights &wt, int64_t N, int64_t K, int G, void *y,
                       int wpc, hipStream_t s) {
  auto kern = qmv1_kernel<BITS, XT, CPL, UD, W, SL>;
  const size_t lds = (size_t)64 * CPL * kChunkLdsBytes + (size_t)W * kStreamRound * 2 +
                     (size_t)W * (SL * 128 + 2) * 4;
  static int per_cu = 0;  // resident workgroups per CU for this instantiation
  if (per_cu == 0) {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, reinterpret_cast<const void *>(kern),
                                                     64 * W, lds) != hipSuccess || v <= 0)
      v = 1;
    per_cu = v;
  }
  const int64_t want = (N + W - 1) / W;
  const int64_t cap = (int64_t)device_cus() * (wpc > 0 && wpc < per_cu ? wpc : per_cu);
  const dim3 grid((unsigned)(want < cap ? want : cap));
  hipLaunchKernelGGL(kern, grid, dim3(64 * W), lds, s, (const uint16_t *)x, wt, N, K, G,
                     (uint16_t *)y);
  return hipGetLastError();
}

// CPL chunks per lane with the launch shape qmv1_shape picks
template <int BITS, typename XT, int CPL, int UD, int W>
hipError_t qmv1_launch_sl(int sl, int wpc, const void *x, const Weights &wt, int64_t N, int64_t K,
                          int G, void *y, hipStream_t s) {
  constexpr int SLMAX = CPL <= 2 ? 1 : (CPL <= 4 ? 2 : 4);
  if (sl == 1) return qmv1_launch<BITS, XT, CPL, UD, W, 1>(x, wt, N, K, G, y, wpc, s);
  if (SLMAX >= 2 && sl == 2)
    return qmv1_launch<BITS, XT, CPL, UD, W, (SLMAX >= 2 ? 2 : 1)>(x, wt, N, K, G, y, wpc, s);
  return qmv1_launch<BITS, XT, CPL, UD, W, SLMAX>(x, wt, N, K, G, y, wpc, s);
}

template <int BITS, typename XT>
hipError_t qmv1_dispatch(const void *x, const Weights &wt, int64_t N, int64_t K, int G, void *y,
                         hipStream_t s) {
  int cpl, ud, w, sl, wpc;
  qmv1_shape(N, K, G, cpl, ud, w, sl, wpc);
#define AQ_QMV1(C, U, WW) return qmv1_launch_sl<BITS, XT, C, U, WW>(sl, wpc, x, wt, N, K, G, y, s)
  switch (cpl) {
    case 1: AQ_QMV1(1, 4, 4);
    case 2:
      if (w == 16) AQ_QMV1(2, 1, 16);
      if (ud == 1) AQ_QMV1(2, 1, 4);
      AQ_QMV1(2, 2, 4);
    case 3: AQ_QMV1(3, 1, 4);
    case 4: AQ_QMV1(4, 1, 4);
    case 5: AQ_QMV1(5, 1, 8);
    case 6: AQ_QMV1(6, 1, 8);
    case 7: AQ_QMV1(7, 1, 8);
    case 8: AQ_QMV1(8, 1, 8);
  }
#undef AQ_QMV1
  return hipErrorInvalidValue;
}

template <int BITS, int MB, typename XT>
hipError_t qmv_launch(const void *x, int M, const Weights &wt, int64_t N, int64_t K, int G,
                      void *y, hipStream_t s) {
  if (MB == 1 && K <= 8 * 2048) return qmv1_dispatch<BITS, XT>(x, wt, N, K, G, y, s);
  const int64_t need = ((K >> 5) + 63) / 64 * 64;
  constexpr int R = stream_shape<MB>::R, D = stream_shape<MB>::D;
  constexpr int W = kStreamWaves, XS = 2;  // M * CP <= XS * 64 * W staged chunks
  const size_t stream_lds = (size_t)M * need * kChunkLdsBytes +
                            (size_t)W * kStreamRound * R * MB * sizeof(uint16_t);
  if (stream_lds <= (size_t)kStreamLdsMax && M * need <= XS * 64 * W) {
    auto kern = qmv_stream_kernel<BITS, MB, XT, R, D, W, XS>;
    hipError_t e = allow_lds(kern, stream_lds);
    if (e != hipSuccess) return e;
    const int64_t units = (N + R - 1) / R;
    const int64_t want = (units + W - 1) / W;
    const int64_t cap = (int64_t)device_cus() * kStreamCtasPerCu;
    const dim3 grid((unsigned)(want < cap ? want : cap));
    hipLaunchKernelGGL(kern, grid, dim3(64 * W), stream_lds, s, (const uint16_t *)x, M, wt, N,
                       K, G, (uint16_t *)y, (int)need);
    return hipGetLastError();
  }
  const int CP = slice_chunks(K, M);
  const size_t lds = (size_t)M * CP * kChunkLdsBytes;
  auto kern = qmv_kernel<BITS, MB, XT, kRows>;
  hipError_t e = allow_lds(kern, lds);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((N + kWaves * kRows - 1) / (kWaves * kRows)));
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, s, (const uint16_t *)x, M, wt, N, K, G,
                     (uint16_t *)y, CP);
  return hipGetLastError();
}

template <int MB, typename XT>
hipError_t qmv_bits(const void *x, int M, const Weights &wt, int64_t N, int64_t K, int G,
                    int bits, void *y, hipStream_t s) {
  switch (bits) {
    case 2: return qmv_launch<2, MB, XT>(x, M, wt, N, K, G, y, s);
    case 3: return qmv_launch<3, MB, XT>(x, M, wt, N, K, G, y, s);
    case 4: return qmv_launch<4, MB, XT>(x, M, wt, N, K, G, y, s);
    case 5: return qmv_launch<5, MB, XT>(x, M, wt, N, K, G, y, s);
    case 6: return qmv_launch<6, MB, XT>(x, M, wt, N, K, G, y, s);
    case 7: return qmv_launch<7, MB, XT>(x, M, wt, N, K, G, y, s);
    case 8: return qmv_launch<8, MB, XT>(x, M, wt, N, K, G, y, s);
  }
  return hipErrorInvalidValue;
}

template <typename XT>
hipError_t qmv_m(const void *x, int M, const Weights &wt, int64_t N, int64_t K, int G, int bits,
                 void *y, hipStream_t s) {
  if (M == 1) return qmv_bits<1, XT>(x, M, wt, N, K, G, bits, y, s);
  if (M == 2) return qmv_bits<2, XT>(x, M, wt, N, K, G, bits, y, s);
  if (M <= 4) return qmv_bits<4, XT>(x, M, wt, N, K, G, bits, y, s);
  return qmv_bits<8, XT>(x, M, wt, N, K, G, bits, y, s);
}

constexpr int kGatherMB = 8;

template <int BITS, typename XT>
hipError_t gather_launch(const void *x, int64_t T, const Weights &wt, int64_t E, int64_t N,
                         int64_t K, const int32_t *ids, int topk, int G, void *y, hipStream_t s) {
  const int CP = slice_chunks(K, kGatherMB);
  const size_t lds = (size_t)kGatherMB * CP * kChunkLdsBytes + (kGatherTile + 1) * sizeof(int);
  auto kern = gather_qmv_kernel<BITS, kGatherMB, XT, kRows>;
  hipError_t e = allow_lds(kern, lds);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((N + kWaves * kRows - 1) / (kWaves * kRows)), (unsigned)E);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, s, (const uint16_t *)x, T, wt, E, N, K, ids,
                     topk, G, (uint16_t *)y, CP);
  return hipGetLastError();
}

template <typename XT>
hipError_t gather_bits(const void *x, int64_t T, const Weights &wt, int64_t E, int64_t N,
                       int64_t K, const int32_t *ids, int topk, int G, int bits, void *y,
                       hipStream_t s) {
  switch (bits) {
    case 2: return gather_launch<2, XT>(x, T, wt, E, N, K, ids, topk, G, y, s);
    case 3: return gather_launch<3, XT>(x, T, wt, E, N, K, ids, topk, G, y, s);
    case 4: return gather_launch<4, XT>(x, T, wt, E, N, K, ids, topk, G, y, s);
    case 5: return gather_launch<5, XT>(x, T, wt, E, N, K, ids, topk, G, y, s);
    case 6: return gather_launch<6, XT>(x, T, wt, E, N, K, ids, topk, G, y, s);
    case 7: return gather_launch<7, XT>(x, T, wt, E, N, K, ids, topk, G, y, s);
    case 8: return gather_launch<8, XT>(x, T, wt, E, N, K, ids, topk, G, y, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_qmv(const void *x, int x_dtype, int M, const uint32_t *codes,
                      const uint16_t *scales, const uint16_t *biases, int64_t N, int64_t K, int G,
                      int bits, void *y, hipStream_t s) {
  const Weights wt{codes, scales, biases};
  if (x_dtype == X_F16) return qmv_m<f16_t>(x, M, wt, N, K, G, bits, y, s);
  if (x_dtype == X_BF16) return qmv_m<bf16_t>(x, M, wt, N, K, G, bits, y, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gather_qmv(const void *x, int x_dtype, int64_t T, const uint32_t *codes,
                             const uint16_t *scales, const uint16_t *biases, int64_t E, int64_t N,
                             int64_t K, const int32_t *ids, int topk, int G, int bits, void *y,
                             hipStream_t s) {
  const Weights wt{codes, scales, biases};
  if (x_dtype == X_F16) return gather_bits<f16_t>(x, T, wt, E, N, K, ids, topk, G, bits, y, s);
  if (x_dtype == X_BF16) return gather_bits<bf16_t>(x, T, wt, E, N, K, ids, topk, G, bits, y, s);
  return hipErrorInvalidValue;
}

}  // namespace aq
