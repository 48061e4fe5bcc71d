// aq_qmm.hip -- quantized matrix-matrix product (prefill) on the gfx950 matrix
// cores.
//
// The operation is Y = X @ W^T with W in packed form ("Quantization",
// metalworking MLX notes, QMM: dequantize weight tiles into on-chip memory,
// then a tiled GEMM against them).  On MI355X:
//  * one 256-thread workgroup computes a 256 x 224 tile of Y (2048 x 28672
//    is exactly 1024 tiles, four full rounds of the 256 CUs); its 4 waves are
//    stacked along M, each owning a 64 x 224 sub-tile made of 2 x 7 blocks of
//    v_mfma_f32_32x32x16_{bf16,f16} with binary32 accumulation (on gfx950
//    the 32x32x16 form sustains about 1.7x the rate of 16x16x32);
//  * per K step of 64 the X tile is copied to LDS and the W tile is read as
//    packed codes, dequantized in registers (q*s + b in binary32, rounded to
//    nearest even into the activation type -- exactly what aq_dequantize
//    returns) and written to LDS, so each weight is dequantized once per 256
//    rows of X; both LDS tiles use a 144-byte row pitch so the 16-byte
//    fragment reads of 16 lanes fall into disjoint banks;
//  * the LDS tiles are double-buffered: the global loads for step k+1 are in
//    flight while the matrix cores work on step k;
//  * tiles are ordered so that the workgroups resident on one XCD (blocks
//    are dealt to the 8 XCDs round-robin) share one row-tile of X in that
//    XCD's L2.
#include "aq_device.hpp"
#include "aq_internal.hpp"

namespace aq {
namespace {

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8v __attribute__((ext_vector_type(8)));
typedef float f32x16v __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 224, BK = 64;
constexpr int WM = 64, WN = 224;            // wave sub-tile
constexpr int FM = WM / 32, FN = WN / 32;   // 32x32 blocks per wave: 2 x 7
constexpr int kPitch = BK + 8;              // elements per LDS row (144 bytes)
constexpr int kThreads = 256;
constexpr int kXLoads = BM * BK / 8 / kThreads;      // 16-byte X loads per thread per step: 8
constexpr int kWPerThread = 2;                       // 32-code chunks per thread per step
constexpr int kWRows = kThreads * kWPerThread / 2;   // 256 LDS W rows; rows >= BN are never read
constexpr int kStageElems = (BM + kWRows) * kPitch;

template <typename XT>
__device__ __forceinline__ f32x16v mfma32(uint4 a, uint4 b, f32x16v c) {
  if constexpr (std::is_same<XT, bf16_t>::value)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8v, a),
                                                   __builtin_bit_cast(bf16x8v, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8v, a),
                                                  __builtin_bit_cast(f16x8v, b), c, 0, 0, 0);
}

template <typename XT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (std::is_same<XT, bf16_t>::value) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    b2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    half2v v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
}

// 32 dequantized values of one chunk, packed in pairs of the activation type
template <int BITS, typename XT>
__device__ __forceinline__ void dequant_chunk(const uint32_t *w, float s, float b, uint32_t *p) {
  if constexpr (BITS == 4) {
    // bytes of lo hold codes 0,2,4,6 of a word, bytes of hi codes 1,3,5,7
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = w[j] & 0x0F0F0F0Fu, hi = (w[j] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v0 = __builtin_fmaf((float)((lo >> (8 * e)) & 0xFFu), s, b);
        const float v1 = __builtin_fmaf((float)((hi >> (8 * e)) & 0xFFu), s, b);
        p[4 * j + e] = pack2<XT>(v0, v1);
      }
    }
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v0 = __builtin_fmaf((float)(w[j] & 0xFFu), s, b);
      const float v1 = __builtin_fmaf((float)((w[j] >> 8) & 0xFFu), s, b);
      const float v2 = __builtin_fmaf((float)((w[j] >> 16) & 0xFFu), s, b);
      const float v3 = __builtin_fmaf((float)(w[j] >> 24), s, b);
      p[2 * j] = pack2<XT>(v0, v1);
      p[2 * j + 1] = pack2<XT>(v2, v3);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float v0 = __builtin_fmaf((float)chunk_code<BITS>(w, 2 * i), s, b);
      const float v1 = __builtin_fmaf((float)chunk_code<BITS>(w, 2 * i + 1), s, b);
      p[i] = pack2<XT>(v0, v1);
    }
  }
}

// Buffer loads: a resource (base, size in bytes) per operand tile; offsets past
// the size read as zero, so partial tiles need no branches.  0x00020000 is
// the gfx9 descriptor word for untyped 32-bit data.
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
  const int n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (bytes < 0 ? 0 : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, n, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
template <int BITS>
__device__ __forceinline__ void bload_chunk(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t *w) {
  if constexpr (BITS % 4 == 0) {
#pragma unroll
    for (int j = 0; j < BITS / 4; ++j) {
      const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + 16 * j), 0, 0);
      w[4 * j] = v[0]; w[4 * j + 1] = v[1]; w[4 * j + 2] = v[2]; w[4 * j + 3] = v[3];
    }
  } else if constexpr (BITS % 2 == 0) {
#pragma unroll
    for (int j = 0; j < BITS / 2; ++j) {
      const u32x2v v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)(off + 8 * j), 0, 0);
      w[2 * j] = v[0]; w[2 * j + 1] = v[1];
    }
  } else {
#pragma unroll
    for (int j = 0; j < BITS; ++j) w[j] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(off + 4 * j), 0, 0);
  }
}

// Scheduling hint for one segment of 14 MFMAs: NR LDS reads among the first
// slots, NV vector ALU instructions after each MFMA, NW LDS writes among the
// last slots and NG global loads among the first.
template <int NR, int NV, int NW, int NG>
__device__ __forceinline__ void sched_segment() {
#pragma unroll
  for (int i = 0; i < FM * FN; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (NV > 0) __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
    if (i >= FM * FN - NW) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    if (i < NG) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
}
// vector instructions to dequantize one 32-code chunk (approximate)
template <int BITS>
constexpr int kDequantValu = BITS == 4 ? 100 : (BITS == 8 ? 90 : 120);

// registers holding one K step's global data for this thread
struct XRegs {
  uint4 x[kXLoads];  // 8 activation values each
};
template <int BITS>
struct WRegs {
  uint32_t w[kWPerThread][BITS];  // 32-code chunks
  uint32_t s[kWPerThread], b[kWPerThread];
};

template <int BITS, typename XT>
__global__ __launch_bounds__(kThreads) void qmm_kernel(const uint16_t *__restrict__ x, int64_t M,
                                                       const uint32_t *__restrict__ codes,
                                                       const uint16_t *__restrict__ scales,
                                                       const uint16_t *__restrict__ biases,
                                                       int64_t N, int64_t K, int G,
                                                       uint16_t *__restrict__ y, int mtiles,
                                                       int ntiles) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];  // [2][(BM + BN) * kPitch]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave;

  // XCD-aware tile order: block b runs on XCD b % 8; consecutive blocks of one
  // XCD take consecutive tiles of a row-major (m, n) order, so they share m.
  const int tiles = mtiles * ntiles;
  int t = blockIdx.x;
  if ((tiles & 7) == 0) t = (t & 7) * (tiles >> 3) + (t >> 3);
  const int64_t tile_m = (int64_t)(t / ntiles) * BM, tile_n = (int64_t)(t % ntiles) * BN;

  const int nch = (int)(K >> 5), gshift = __builtin_ctz((unsigned)G) - 5;
  const int64_t wpr = (int64_t)nch * BITS, gpr = nch >> gshift;
  const int ksteps = (int)((K + BK - 1) / BK);

  // operand tiles as buffer resources: rows past M or N read as zero
  const int64_t mrows = M - tile_m < BM ? M - tile_m : BM;
  const int64_t nrows = N - tile_n < BN ? N - tile_n : BN;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + tile_m * K, mrows * K * 2);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(codes + tile_n * wpr, nrows * wpr * 4);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(scales + tile_n * gpr, nrows * gpr * 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(biases + tile_n * gpr, nrows * gpr * 2);

  // K steps: when K % 64 == 32 the lone last chunk is processed first (step
  // 0, masked in the prologue), so every step inside the loop is full.
  const bool ktail = (K % BK) != 0;
  auto kbase = [&](int st) -> int {  // first k of step st
    return ktail ? (st == 0 ? (int)K - 32 : (st - 1) * BK) : st * BK;
  };

  auto load_x = [&](int st, XRegs &r) {
    const int k0 = kbase(st);
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
      const int idx = tid + kThreads * i;
      const int row = idx >> 3, c8 = idx & 7;
      r.x[i] = bload16(rx, (uint32_t)(row * K + k0 + c8 * 8) * 2u);
    }
  };
  auto load_w = [&](int st, WRegs<BITS> &r) {
    const int c0 = kbase(st) >> 5;
#pragma unroll
    for (int i = 0; i < kWPerThread; ++i) {
      const int ch = tid + kThreads * i;  // rows >= BN read zeros (outside the resource)
      const int row = ch >> 1;
      int c = c0 + (ch & 1);
      c = c < nch ? c : nch - 1;  // only in the tail step; masked there
      bload_chunk<BITS>(rw, (uint32_t)(row * wpr + c * BITS) * 4u, r.w[i]);
      const uint32_t go = (uint32_t)(row * gpr + (c >> gshift)) * 2u;
      r.s[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)go, 0, 0);
      r.b[i] = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)go, 0, 0);
    }
  };

  // write a step (X as loaded; W dequantized) into LDS buffer `buf`; with
  // `tail` the second 32 k of the step (past K) are zeroed
  auto store_x = [&](const XRegs &rxr, int buf, bool tail) {
    uint16_t *lx = lds + buf * kStageElems;
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
      const int idx = tid + kThreads * i;
      const int row = idx >> 3, c8 = idx & 7;
      const uint4 v = (tail && c8 >= 4) ? make_uint4(0, 0, 0, 0) : rxr.x[i];
      *reinterpret_cast<uint4 *>(lx + row * kPitch + c8 * 8) = v;
    }
  };
  auto store_w_chunk = [&](const WRegs<BITS> &r, int i, int buf) {
    uint16_t *lw = lds + buf * kStageElems + BM * kPitch;
    const int ch = tid + kThreads * i;  // rows >= BN land in pad rows nobody reads
    const int row = ch >> 1, half = ch & 1;
    uint32_t p[16];
    dequant_chunk<BITS, XT>(r.w[i], f16_to_f32((uint16_t)r.s[i]), f16_to_f32((uint16_t)r.b[i]), p);
    uint4 *dst = reinterpret_cast<uint4 *>(lw + row * kPitch + half * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dst[j] = make_uint4(p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]);
  };
  auto store_w = [&](const WRegs<BITS> &r, int buf, bool tail) {
    uint16_t *lw = lds + buf * kStageElems + BM * kPitch;
#pragma unroll
    for (int i = 0; i < kWPerThread; ++i) {
      const int ch = tid + kThreads * i;
      const int row = ch >> 1, half = ch & 1;
      uint32_t p[16];
      dequant_chunk<BITS, XT>(r.w[i], f16_to_f32((uint16_t)r.s[i]), f16_to_f32((uint16_t)r.b[i]), p);
      uint4 *dst = reinterpret_cast<uint4 *>(lw + row * kPitch + half * 32);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dst[j] = (tail && half) ? make_uint4(0, 0, 0, 0)
                                : make_uint4(p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]);
    }
  };

  f32x16v acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // fragment addressing: lane l supplies row (l % 32) of a block, k-group l / 32
  const int frow = lane & 31, fk = (lane >> 5) * 8;
  auto frag = [&](int buf, int kk, uint4(&a)[FM], uint4(&b)[FN]) {
    const uint16_t *lx = lds + buf * kStageElems + (wm * WM + frow) * kPitch + fk + kk * 16;
    const uint16_t *lw = lds + buf * kStageElems + BM * kPitch + frow * kPitch + fk + kk * 16;
#pragma unroll
    for (int i = 0; i < FM; ++i) a[i] = *reinterpret_cast<const uint4 *>(lx + i * 32 * kPitch);
#pragma unroll
    for (int j = 0; j < FN; ++j) b[j] = *reinterpret_cast<const uint4 *>(lw + j * 32 * kPitch);
  };
  auto mfma_kk = [&](const uint4(&a)[FM], const uint4(&b)[FN]) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int i = 0; i < FM; ++i) acc[i][j] = mfma32<XT>(a[i], b[j], acc[i][j]);
  };

  // One K step from LDS buffer cb.  With one wave per SIMD, matrix-core and
  // vector work overlap only through this wave's own instruction order, so
  // the step is cut into four fenced segments, one per 16-k slice: each
  // issues the fragment reads of the next slice, then its 14 MFMAs with a
  // share of the next step's work between them (X stores, dequantization of
  // one W chunk and its stores, the global loads two steps ahead).
  auto step = [&](int cb, XRegs &xn, WRegs<BITS> &wn, bool more, int stw, int stx) {
    uint4 fa[2][FM], fb[2][FN];
    frag(cb, 0, fa[0], fb[0]);
    __builtin_amdgcn_sched_barrier(0);
    frag(cb, 1, fa[1], fb[1]);
    mfma_kk(fa[0], fb[0]);
    if (more) store_x(xn, cb ^ 1, false);
    sched_segment<FM + FN, 0, kXLoads, 0>();
    __builtin_amdgcn_sched_barrier(0);
    frag(cb, 2, fa[0], fb[0]);
    mfma_kk(fa[1], fb[1]);
    if (more) store_w_chunk(wn, 0, cb ^ 1);
    sched_segment<FM + FN, kDequantValu<BITS> / (FM * FN), 4, 0>();
    __builtin_amdgcn_sched_barrier(0);
    frag(cb, 3, fa[1], fb[1]);
    mfma_kk(fa[0], fb[0]);
    if (more) store_w_chunk(wn, 1, cb ^ 1);
    sched_segment<FM + FN, kDequantValu<BITS> / (FM * FN), 4, 0>();
    __builtin_amdgcn_sched_barrier(0);
    mfma_kk(fa[1], fb[1]);
    if (more) {
      load_w(stw, wn);
      load_x(stx, xn);
    }
    sched_segment<0, 0, 0, kXLoads + 6>();
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue: step 0 in buffer 0; X of step 1 and W of steps 1, 2 in flight
  XRegs xr;
  WRegs<BITS> wr[2];
  load_x(0, xr);
  load_w(0, wr[0]);
  store_x(xr, 0, ktail);
  store_w(wr[0], 0, ktail);
  auto last = [&](int st) { return st < ksteps ? st : ksteps - 1; };
  load_x(last(1), xr);
  load_w(last(1), wr[1]);
  load_w(last(2), wr[0]);
  __syncthreads();

  // step st computes from buffer st & 1 while step st + 1 is written to the
  // other buffer; past the last step the loads repeat it (branch-free body)
  int st = 0;
  for (; st + 2 <= ksteps; st += 2) {
    step(0, xr, wr[1], true, last(st + 3), last(st + 2));
    __syncthreads();
    step(1, xr, wr[0], true, last(st + 4), last(st + 3));
    __syncthreads();
  }
  if (st < ksteps) step(st & 1, xr, wr[0], false, 0, 0);  // odd step count: the last step

  // epilogue: accumulator r of lane l in a 32x32 block is row
  // 8*(r/4) + 4*(l/32) + r%4, column l % 32
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = tile_n + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = tile_m + wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < M && n < N) y[m * N + n] = xtraits<XT>::from_f32(acc[i][j][r]);
      }
    }
}

template <int BITS, typename XT>
hipError_t qmm_launch(const void *x, int64_t M, const uint32_t *codes, const uint16_t *scales,
                      const uint16_t *biases, int64_t N, int64_t K, int G, void *y,
                      hipStream_t s) {
  auto kern = qmm_kernel<BITS, XT>;
  const size_t lds = 2 * (size_t)kStageElems * sizeof(uint16_t);
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int64_t mt = (M + BM - 1) / BM, nt = (N + BN - 1) / BN;
  if (mt * nt > 0x7FFFFFFF || mt > 0x7FFFFFFF || nt > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)(mt * nt)), dim3(kThreads), lds, s, (const uint16_t *)x, M,
                     codes, scales, biases, N, K, G, (uint16_t *)y, (int)mt, (int)nt);
  return hipGetLastError();
}

template <typename XT>
hipError_t qmm_bits(const void *x, int64_t M, const uint32_t *codes, const uint16_t *scales,
                    const uint16_t *biases, int64_t N, int64_t K, int G, int bits, void *y,
                    hipStream_t s) {
  switch (bits) {
    case 2: return qmm_launch<2, XT>(x, M, codes, scales, biases, N, K, G, y, s);
    case 3: return qmm_launch<3, XT>(x, M, codes, scales, biases, N, K, G, y, s);
    case 4: return qmm_launch<4, XT>(x, M, codes, scales, biases, N, K, G, y, s);
    case 5: return qmm_launch<5, XT>(x, M, codes, scales, biases, N, K, G, y, s);
    case 6: return qmm_launch<6, XT>(x, M, codes, scales, biases, N, K, G, y, s);
    case 7: return qmm_launch<7, XT>(x, M, codes, scales, biases, N, K, G, y, s);
    case 8: return qmm_launch<8, XT>(x, M, codes, scales, biases, N, K, G, y, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_qmm(const void *x, int x_dtype, int64_t M, const uint32_t *codes,
                      const uint16_t *scales, const uint16_t *biases, int64_t N, int64_t K, int G,
                      int bits, void *y, hipStream_t s) {
  if (x_dtype == X_F16) return qmm_bits<f16_t>(x, M, codes, scales, biases, N, K, G, bits, y, s);
  if (x_dtype == X_BF16) return qmm_bits<bf16_t>(x, M, codes, scales, biases, N, K, G, bits, y, s);
  return hipErrorInvalidValue;
}

}  // namespace aq
