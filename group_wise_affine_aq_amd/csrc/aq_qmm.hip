// aq_qmm.hip -- quantized matrix-matrix product (prefill) on the gfx950 matrix
// cores.
//
// The operation is Y = X @ W^T with W in packed form ("Quantization",
// metalworking MLX notes, QMM: dequantize weight tiles on chip, then a tiled
// GEMM against them), built on v_mfma_f32_32x32x16_{bf16,f16} with binary32
// accumulation (on gfx950 the 32x32x16 form sustains about 1.7x the rate of
// 16x16x32) and on weights dequantized exactly as aq_dequantize returns them
// (q*s + b in binary32, rounded to nearest even into the activation type).
//
// qmm_wr_kernel: one 256-thread workgroup per 256 x 256 tile of Y, one wave
// per SIMD.  Wave w owns the 64 columns 64w .. 64w+63 for all 256 rows
// (8 x 2 blocks, 256 accumulation registers) and dequantizes its own W
// chunks straight into the B operand, so no weight passes through LDS.
// Only the X tile is shared: each K step's 256 x 64 slice is copied to LDS
// by direct global-to-LDS loads into one of four stages, three steps ahead,
// as are the W chunks into register sets.  A step's loads are spread over
// its four 16-k slices, and the one barrier per step waits only for the
// stage it needs.  When the tiles leave a last round at most half full,
// those columns run as 256 x 128 tiles (one 32-column block per wave) in a
// second launch.
//
// The gather variant ("Quantization", metalworking: gather variants of the
// kernels for MoE experts, here at prefill size) computes y[t, j, :] =
// x[t] @ W_{ids[t, j]}^T on the same engine: one workgroup per (256-column
// tile, expert) scans the routing ids on the device, lists the (token, slot)
// pairs routed to its expert in id order, and runs 256-row tiles over that
// list, loading X rows by token and storing Y rows by pair.
#include "aq_device.hpp"
#include "aq_internal.hpp"

namespace aq {
namespace {

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8v __attribute__((ext_vector_type(8)));
typedef float f32x16v __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BK = 64;  // tile rows (full tiles), K step
constexpr int kThreads = 256;

// loads issued for one W chunk (codes, scale, bias)
template <int BITS>
constexpr int kChunkLoads = (BITS % 4 == 0 ? BITS / 4 : (BITS % 2 == 0 ? BITS / 2 : BITS)) + 2;

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their maxima)
constexpr int vmcnt_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }

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

// A register holding v that the optimizer cannot see through (an identity
// DPP move).  ANDing codes with an opaque 0x0F0F0F0F keeps the byte-wise
// conversions below as v_cvt_f32_ubyte{0..3} instead of letting them fold
// into per-code bit-field extracts, while every instruction stays visible to
// the compiler (and to its matrix-core hazard checks).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xE4, 0xF, 0xF, false);
}

// Codes 8u .. 8u+7 of a 32-code chunk dequantized (q*s + b in binary32,
// rounded to nearest even into the activation type) and packed in pairs.
template <int BITS, typename XT, int U>
__device__ __forceinline__ uint4 dequant8(const uint32_t *w, float s, float b, uint32_t nmask) {
  uint32_t p[4];
  if constexpr (BITS == 4) {
    const uint32_t lo = w[U] & nmask, hi = (w[U] >> 4) & nmask;  // codes 0,2,4,6 / 1,3,5,7
#pragma unroll
    for (int e = 0; e < 4; ++e)
      p[e] = pack2<XT>(__builtin_fmaf((float)((lo >> (8 * e)) & 0xFFu), s, b),
                       __builtin_fmaf((float)((hi >> (8 * e)) & 0xFFu), s, b));
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t v = w[2 * U + j];
      p[2 * j] = pack2<XT>(__builtin_fmaf((float)(v & 0xFFu), s, b),
                           __builtin_fmaf((float)((v >> 8) & 0xFFu), s, b));
      p[2 * j + 1] = pack2<XT>(__builtin_fmaf((float)((v >> 16) & 0xFFu), s, b),
                               __builtin_fmaf((float)(v >> 24), s, b));
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      p[e] = pack2<XT>(__builtin_fmaf((float)chunk_code<BITS>(w, 8 * U + 2 * e), s, b),
                       __builtin_fmaf((float)chunk_code<BITS>(w, 8 * U + 2 * e + 1), s, b));
  }
  return make_uint4(p[0], p[1], p[2], p[3]);
}

// Buffer loads: a resource (base, size in bytes) per operand tile; offsets past
// the size read as zero, so partial tiles need no branches.  0x00020000 is
// the gfx9 descriptor word for untyped 32-bit data.  The per-step part of an
// address goes in the scalar offset.
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
  const int n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (bytes < 0 ? 0 : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, n, 0x00020000);
}
template <int BITS>
__device__ __forceinline__ void bload_chunk(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                            uint32_t *w) {
  if constexpr (BITS % 4 == 0) {
#pragma unroll
    for (int j = 0; j < BITS / 4; ++j) {
      const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(voff + 16 * j), (int)soff, 0);
      w[4 * j] = v[0]; w[4 * j + 1] = v[1]; w[4 * j + 2] = v[2]; w[4 * j + 3] = v[3];
    }
  } else if constexpr (BITS % 2 == 0) {
#pragma unroll
    for (int j = 0; j < BITS / 2; ++j) {
      const u32x2v v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)(voff + 8 * j), (int)soff, 0);
      w[2 * j] = v[0]; w[2 * j + 1] = v[1];
    }
  } else {
#pragma unroll
    for (int j = 0; j < BITS; ++j)
      w[j] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(voff + 4 * j), (int)soff, 0);
  }
}

// routing of the gather variant: ids [T, topk] flattened, experts [0, E)
struct Routing {
  const int32_t *ids;
  int64_t pairs;  // T * topk
  int topk;
  int64_t E;
};
// pairs of one expert listed per pass (the rest in later passes)
constexpr int kGList = 4096;

// block-wide exclusive prefix sum of v (256 threads); *total gets the sum
__device__ __forceinline__ int block_exclusive_sum(int v, int *wsum, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(incl, d);
    if (lane >= d) incl += u;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    before += w < wave ? wsum[w] : 0;
    all += wsum[w];
  }
  *total = all;
  return before + incl - v;
}

// ---------------------------------------------------------------------------
// The prefill product with weights dequantized straight into matrix-core
// operands.  One 256-thread workgroup computes a 256 x 256 tile of Y; wave w
// owns the 64 columns 64w .. 64w+63 and all 256 rows: 8 x 2 blocks of
// v_mfma_f32_32x32x16 (256 accumulators per lane, in the accumulation
// registers one wave per SIMD can hold; with NB = 1, a 256 x 128 tile, wave w
// owns the 32 columns 32w .. 32w+31, 8 x 1 blocks).  Each lane loads, for each
// of its NB 32-column blocks, one whole 32-code chunk of its column's W row per K step
// of 64 and dequantizes it (q*s + b in binary32, rounded to nearest even into
// the activation type, the value aq_dequantize returns) directly into the B
// operand: no weight ever passes through LDS, and no other wave needs it.
// Only the X tile is shared: each step's 256 x 64 tile is copied to LDS by
// direct global-to-LDS loads into one of four stages, three steps ahead of
// its use, as are the W chunks (register sets), so one barrier per step
// suffices and HBM latency stays hidden behind three steps of matrix work.
// K order inside a step: the B operand of lane l (column l % 32, half
// h = l / 32) for 16-k slice ks holds codes 8 ks .. 8 ks + 7 of chunk h, i.e.
// k = 32 h + 8 ks + 0..7; the A fragments are read from LDS in that same
// order (a permutation of k applied to both operands leaves the dot products
// unchanged).
constexpr int WBN = 256;                     // tile columns (two 32-column blocks per wave)
constexpr int kWStages = 4;                  // X stages in LDS (32 KB each)

// a tile of 32 FM rows: 16-byte X units per thread per step
template <int FM>
constexpr int kWrXDma = 32 * FM * BK / 8 / kThreads;

// s_waitcnt immediate: at most n vector-memory operations outstanding, and
// no LDS operation (lgkmcnt 0)
constexpr int vm_lgkm0_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4); }

// Workgroup barrier for the X stages: this wave's outstanding loads are
// first cut to `n` (its copies of the stage read next have landed) and its
// LDS reads drained (no copy issued after the barrier can overtake them).
// __syncthreads() would add a release fence, which also waits for every
// global-to-LDS copy still in flight, the later stages' included.  The empty
// asm statements keep the compiler from moving memory accesses across.
template <int n>
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(n));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// one thread's W chunks (one per 32-column block) of one K step
template <int BITS, int NB>
struct WrRegs {
  uint32_t w[NB][BITS];
  uint32_t s[NB], b[NB];
};

// Scheduling hint for one 16-k slice: 2 FM MFMAs, NR LDS reads and NG global
// loads among the first slots, NV vector ALU instructions after each MFMA.
template <int FM, int NB, int NR, int NV, int NG>
__device__ __forceinline__ void sched_kslice() {
#pragma unroll
  for (int i = 0; i < FM * NB; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (i < NG) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    if (NV > 0) __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
  }
}

// FM: 32-row blocks per tile.  NB: 32-column blocks per wave (2: 256 x 256
// tiles; 1: 256 x 128, for a last partial round of tiles).  G1: one group
// per 32-code chunk (G = 32).  y rows are ldy elements apart.  GATHER (MoE prefill, FM = 8): grid y is the
// expert; the workgroup lists the (token, slot) pairs routed to its expert
// (route) and runs 256-row tiles over that list, X rows loaded by token and
// Y rows stored by pair.
template <int BITS, typename XT, int FM, int NB, bool G1, bool GATHER>
__global__ __launch_bounds__(kThreads) void qmm_wr_kernel(const uint16_t *__restrict__ x,
                                                          int64_t M,
                                                          const uint32_t *__restrict__ codes,
                                                          const uint16_t *__restrict__ scales,
                                                          const uint16_t *__restrict__ biases,
                                                          int64_t N, int64_t K, int G,
                                                          uint16_t *__restrict__ y, int64_t ldy,
                                                          Routing route) {
  constexpr int TBM = 32 * FM, TBN = 128 * NB, kXSt = TBM * BK * 2, kXD = kWrXDma<FM>;
  // a thread's loads per step: the X copy, the codes of its NB W chunks,
  // their scales and biases (G > 32: one scale and one bias per lane, for
  // the block of its half, exchanged between the halves afterwards when
  // NB = 2)
  constexpr int kCode = kChunkLoads<BITS> - 2;
  constexpr int kStepLoads = kXD + NB * kCode + (G1 ? 2 * NB : 2);
  // four distinct LDS objects, one per X stage
  __shared__ __attribute__((aligned(16))) char xs0[kXSt], xs1[kXSt], xs2[kXSt], xs3[kXSt];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;

  const int nch = (int)(K >> 5), gshift = __builtin_ctz((unsigned)G) - 5;
  const int64_t wpr = (int64_t)nch * BITS, gpr = nch >> gshift;
  const int ksteps = (int)((K + BK - 1) / BK);

  // Grid x: column tiles, y: row tiles.  Blocks are dealt to the 8 XCDs
  // round-robin in x-fastest order, so the blocks resident on one XCD hold
  // every eighth column tile of the same one or two row tiles and share
  // those X rows in its L2.  (No division: the tile coordinates stay scalar,
  // and with them the operand resources.)
  int64_t tile_m = 0;
  const int64_t tile_n = (int64_t)blockIdx.x * TBN;
  int expert = 0;
  if constexpr (GATHER) {
    expert = blockIdx.y;
    codes += (int64_t)expert * N * wpr;
    scales += (int64_t)expert * N * gpr;
    if (biases) biases += (int64_t)expert * N * gpr;
  } else {
    tile_m = (int64_t)blockIdx.y * TBM;
  }

  // operand tiles as buffer resources: rows past M or N read as zero (the
  // gather addresses all of x by token)
  const int64_t mrows = M - tile_m < TBM ? M - tile_m : TBM;
  const int64_t nrows = N - tile_n < TBN ? N - tile_n : TBN;
  const int xbytes = (int)((GATHER ? M : mrows) * K * 2);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + tile_m * K, xbytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(codes + tile_n * wpr, nrows * wpr * 4);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(scales + tile_n * gpr, nrows * gpr * 2);
  // without a bias array (null) a resource of size 0: its loads return +0
  const __amdgpu_buffer_rsrc_t rb = biases ? make_rsrc(biases + tile_n * gpr, nrows * gpr * 2)
                                           : make_rsrc(scales, 0);

  // K steps: when K % 64 == 32 the lone last chunk is step 0 (its upper half
  // reads zeros), so every later step is full
  const bool ktail = (K % BK) != 0;
  const int koff = ktail ? BK : 0;
  auto kbase = [&](int st) -> int { return ktail && st == 0 ? (int)K - 32 : st * BK - koff; };
  auto kclamp = [&](int st) -> int { return kbase(st < ksteps ? st : ksteps - 1); };

  // X copy: load i of wave w fills rows 8 (8w + i) .. +7; LDS row r holds
  // the row's 16-byte unit u at slot u ^ ((r >> 1) & 7).  Row r of the tile
  // at list position r0 is x row r (plain) or the token of pair
  // glist[r0 + r] (gather; rows >= rows read as zero).
  uint32_t xvoff[kXD], xvoff_tail[kXD];
  __shared__ int glist[GATHER ? kGList : 1];  // pairs of the expert in this pass
  auto set_rows = [&](int r0, int rows) {
#pragma unroll
    for (int i = 0; i < kXD; ++i) {
      const int row = 8 * (wave * kXD + i) + (lane >> 3);
      const int u = (lane & 7) ^ ((row >> 1) & 7);
      uint32_t ro;
      if constexpr (GATHER)
        ro = row < rows ? (uint32_t)((int64_t)(glist[r0 + row] / route.topk) * K * 2)
                        : (uint32_t)xbytes;
      else
        ro = (uint32_t)(row * K * 2);
      xvoff[i] = ro + (uint32_t)u * 16u;
      xvoff_tail[i] = u < 4 ? xvoff[i] : (uint32_t)xbytes;  // k past K: out of range, reads zero
    }
  };
  // loads i0 .. i1-1 of a step's X copy
  auto dma_x = [&](int k0, char *dst, const uint32_t (&vo)[kXD], int i0 = 0, int i1 = kWrXDma<FM>) {
    const uint32_t so = (uint32_t)k0 * 2u;
#pragma unroll
    for (int i = 0; i < kXD; ++i)
      if (i >= i0 && i < i1)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rx, (lds_void *)(dst + (wave * kXD + i) * 1024), 16, (int)vo[i], (int)so, 0, 0);
  };

  // W: block cb of lane l is tile column 64 w + 32 cb + l % 32; the lane
  // reads chunk h of the step (step 0 of a K tail: only h = 0 is inside K).
  // G = 32: the lane reads the scale and bias of its chunk for both blocks;
  // G > 32 (both chunks in one group): only those of block h, which one
  // v_permlane32_swap then gives to both halves.
  uint32_t wvoff[NB], svoff[NB], wvoff0[NB], svoff0[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const int n = 32 * NB * wave + 32 * (G1 ? cb : (NB == 2 ? h : 0)) + (lane & 31);
    wvoff[cb] = (uint32_t)((32 * NB * wave + 32 * cb + (lane & 31)) * wpr + h * BITS) * 4u;
    svoff[cb] = (uint32_t)(n * gpr + (G1 ? h : 0)) * 2u;
    wvoff0[cb] = ktail && h ? 0x80000000u : wvoff[cb];  // past every resource: zeros
    svoff0[cb] = G1 && ktail && h ? 0x80000000u : svoff[cb];
  }
  // part p of a step's W loads: the codes of block p (if any), then (G = 32)
  // the scale and bias of block p, or (G > 32) the scale (p = 0) or the bias
  auto load_w = [&](int k0, WrRegs<BITS, NB> &r, const uint32_t (&wv)[NB], const uint32_t (&sv)[NB],
                    int part) {
    const int c0 = k0 >> 5;
    if (part < NB) bload_chunk<BITS>(rw, wv[part], (uint32_t)(c0 * BITS) * 4u, r.w[part]);
    const uint32_t so = (uint32_t)(c0 >> gshift) * 2u;
    if constexpr (G1) {
      if (part < NB) {
        r.s[part] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)sv[part], (int)so, 0);
        r.b[part] = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)sv[part], (int)so, 0);
      }
    } else if (part == 0) {
      r.s[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)sv[0], (int)so, 0);
    } else {
      r.b[0] = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)sv[0], (int)so, 0);
    }
  };
  // before the first use of a register set (G > 32, NB = 2): lanes l and
  // l + 32 hold the scale (bias) of blocks 0 and 1; afterwards every lane
  // holds both (NB = 1: both halves loaded those of their own column)
  auto share_sb = [&](WrRegs<BITS, NB> &r) {
    if constexpr (!G1 && NB == 2) {
      const auto sp = __builtin_amdgcn_permlane32_swap(r.s[0], r.s[0], false, false);
      const auto bp = __builtin_amdgcn_permlane32_swap(r.b[0], r.b[0], false, false);
      r.s[0] = sp[0];
      r.s[1] = sp[1];
      r.b[0] = bp[0];
      r.b[1] = bp[1];
    }
  };
  const uint32_t nmask = opaque(0x0F0F0F0Fu);
  auto dequant = [&](const WrRegs<BITS, NB> &r, auto kscon, uint4 (&bq)[NB]) {
    constexpr int ks = decltype(kscon)::value;
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
      bq[cb] = dequant8<BITS, XT, ks>(r.w[cb], f16_to_f32((uint16_t)r.s[cb]),
                                      f16_to_f32((uint16_t)r.b[cb]), nmask);
  };

  // A fragments: lane l supplies row (l % 32) of a 32-row block and unit
  // 4 h + ks of the step
  uint32_t xfo[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    xfo[ks] = (uint32_t)((lane & 31) * 128 + (((4 * h + ks) ^ (((lane & 31) >> 1) & 7)) * 16));
  auto frag = [&](const char *st_base, int ks, uint4 (&a)[FM]) {
    const char *p = st_base + xfo[ks];
#pragma unroll
    for (int i = 0; i < FM; ++i) a[i] = *reinterpret_cast<const uint4 *>(p + i * 32 * 128);
  };

  f32x16v acc[FM][NB];
  auto mfma_ks = [&](const uint4 (&a)[FM], const uint4 (&b)[NB]) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < FM; ++i) acc[i][j] = mfma32<XT>(a[i], b[j], acc[i][j]);
  };

  // The pipeline takes the four stages as restrict pointers: every LDS access
  // in it then carries alias scopes, from which the compiler's wait placement
  // can tell a copy into one stage from reads of another (without them it
  // makes each fragment read wait for the latest copy into any stage).
  auto run = [&](char *__restrict__ q0, char *__restrict__ q1, char *__restrict__ q2,
                 char *__restrict__ q3) {
  auto stage = [&](auto jcon) -> char * {
    constexpr int j = decltype(jcon)::value;
    return j == 0 ? q0 : j == 1 ? q1 : j == 2 ? q2 : q3;
  };
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  WrRegs<BITS, NB> wr[kWStages];  // W of step s in wr[s % 4]
  uint4 fa[2][FM], fb[2][NB];
  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;
  using K2 = std::integral_constant<int, 2>;
  using K3 = std::integral_constant<int, 3>;
  constexpr int kNV = 3;  // vector instructions between consecutive MFMAs

  // Step st from stage / register set j = st % 4.  On entry fa[0], fb[0]
  // hold slice 0.  Each slice's MFMAs run while the next slice's fragments
  // are read and its weights dequantized; before the last slice the wave
  // waits for step st + 1's data, meets the others at the barrier (every
  // wave is then done with stage j), and starts step st + 4's X copy into
  // stage j.  A step's loads are spread over four slices (X copy: half after
  // the barrier of step s - 4, half in slice 0 of step s - 3; W: one block in
  // each of slices 1 and 2 of step s - 3): issued in a burst they queue at
  // the memory pipeline and stall the wave's matrix-core issue.  Either way
  // exactly 28 (4-bit) loads follow a step's last one before the barrier
  // that waits for it.
  // The wait counts the loads issued after step st + 1's; in the steps after
  // the main loop (FIN) the compiler drops loads whose registers are never
  // read again, so there the wave waits for all of its loads.
  auto step = [&](auto jcon, auto fincon, int st) {
    constexpr int j = decltype(jcon)::value;
    constexpr bool FIN = decltype(fincon)::value;
    constexpr int jn = (j + 1) & 3;
    using JN = std::integral_constant<int, jn>;
    constexpr int j3 = (j + 3) & 3;  // stage / register set of step st + 3
    using J3 = std::integral_constant<int, j3>;
    char *sb = stage(jcon);
    const int k3 = kclamp(st + 3);
    frag(sb, 1, fa[1]);
    dequant(wr[j], K1{}, fb[1]);
    dma_x(k3, stage(J3{}), xvoff, kXD / 2, kXD);
    mfma_ks(fa[0], fb[0]);
    sched_kslice<FM, NB, FM, kNV, kXD / 2>();
    __builtin_amdgcn_sched_barrier(0);
    frag(sb, 2, fa[0]);
    dequant(wr[j], K2{}, fb[0]);
    load_w(k3, wr[j3], wvoff, svoff, 0);
    mfma_ks(fa[1], fb[1]);
    sched_kslice<FM, NB, FM, kNV, kChunkLoads<BITS>>();
    __builtin_amdgcn_sched_barrier(0);
    frag(sb, 3, fa[1]);
    dequant(wr[j], K3{}, fb[1]);
    load_w(k3, wr[j3], wvoff, svoff, 1);
    mfma_ks(fa[0], fb[0]);
    sched_kslice<FM, NB, FM, kNV, kChunkLoads<BITS>>();
    __builtin_amdgcn_sched_barrier(0);
    // step st + 1's X and W have landed (steps st + 2, st + 3 stay in flight)
    constexpr int kAhead = FIN ? 0 : (2 * kStepLoads < 63 ? 2 * kStepLoads : 63);
    stage_barrier<kAhead>();
    dma_x(kclamp(st + 4), sb, xvoff, 0, kXD / 2);
    frag(stage(JN{}), 0, fa[0]);
    share_sb(wr[jn]);
    dequant(wr[jn], K0{}, fb[0]);
    mfma_ks(fa[1], fb[1]);
    sched_kslice<FM, NB, FM, kNV, kXD / 2>();
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue: steps 0 .. 2 and the first half of step 3's X copy in flight
  // (step 0 masked past K when it is the tail chunk), then slice 0 of step 0
  // (fenced: the counter wait below relies on this issue order)
  dma_x(kbase(0), q0, ktail ? xvoff_tail : xvoff);
  load_w(kbase(0), wr[0], wvoff0, svoff0, 0);
  load_w(kbase(0), wr[0], wvoff0, svoff0, 1);
  __builtin_amdgcn_sched_barrier(0);
  dma_x(kclamp(1), q1, xvoff);
  load_w(kclamp(1), wr[1], wvoff, svoff, 0);
  load_w(kclamp(1), wr[1], wvoff, svoff, 1);
  __builtin_amdgcn_sched_barrier(0);
  dma_x(kclamp(2), q2, xvoff);
  load_w(kclamp(2), wr[2], wvoff, svoff, 0);
  load_w(kclamp(2), wr[2], wvoff, svoff, 1);
  __builtin_amdgcn_sched_barrier(0);
  dma_x(kclamp(3), q3, xvoff, 0, kXD / 2);
  __builtin_amdgcn_sched_barrier(0);
  stage_barrier<(2 * kStepLoads + kXD / 2 < 63 ? 2 * kStepLoads + kXD / 2
                                                          : 63)>();
  frag(q0, 0, fa[0]);
  share_sb(wr[0]);
  if (!G1 && ktail && h) {  // step 0 is the K tail: chunk 1 lies past K, its weights read 0
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) wr[0].s[cb] = wr[0].b[cb] = 0;
  }
  dequant(wr[0], K0{}, fb[0]);

  using LOOP = std::false_type;
  using FIN = std::true_type;
  int st = 0;
  for (; st + 4 <= ksteps; st += 4) {
    step(K0{}, LOOP{}, st);
    step(K1{}, LOOP{}, st + 1);
    step(K2{}, LOOP{}, st + 2);
    step(K3{}, LOOP{}, st + 3);
  }
  if (st < ksteps) step(K0{}, FIN{}, st);
  if (st + 1 < ksteps) step(K1{}, FIN{}, st + 1);
  if (st + 2 < ksteps) step(K2{}, FIN{}, st + 2);
  // the loads issued past the last step (clamped, in range) finish here
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  };
  if constexpr (!GATHER) {
    set_rows(0, TBM);
    run(xs0, xs1, xs2, xs3);
    // epilogue: accumulator r of lane l in a 32x32 block is row
    // 8*(r/4) + 4*(l/32) + r%4, column l % 32
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int64_t n = tile_n + 32 * NB * wave + 32 * j + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = tile_m + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (m < M && n < N) y[m * ldy + n] = xtraits<XT>::from_f32(acc[i][j][r]);
        }
      }
  } else {
    // one 256-row tile of the list from position r0; row lr of the tile is
    // pair glist[r0 + lr], stored to that (token, slot)'s y row
    auto tile = [&](int r0, int rows) {
      set_rows(r0, rows);
      run(xs0, xs1, xs2, xs3);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (lr < rows) {
            uint16_t *yr = y + (int64_t)glist[r0 + lr] * ldy;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
              const int64_t n = tile_n + 32 * NB * wave + 32 * j + (lane & 31);
              if (n < N) yr[n] = xtraits<XT>::from_f32(acc[i][j][r]);
            }
          }
        }
      __syncthreads();  // the stages and the list are reused
    };
    __shared__ int gsum[kThreads / 64 + 2];
    const int64_t total = route.pairs;
    // pairs whose id is outside [0, E): zero rows (written by expert 0)
    if (expert == 0)
      for (int64_t p = tid; p < total; p += kThreads) {
        const int32_t id = route.ids[p];
        if (id < 0 || id >= route.E)
          for (int nn = 0; nn < nrows; ++nn) y[p * ldy + tile_n + nn] = 0;
      }
    // passes over the ids: each lists, in id order, the next kGList pairs
    // routed to this expert (thread t scans a contiguous segment; a block
    // prefix sum of the segment counts gives every match its rank)
    int64_t pos = 0;
    while (pos < total) {
      const int64_t seg = (total - pos + kThreads - 1) / kThreads;
      const int64_t a = pos + tid * seg, b = a + seg < total ? a + seg : total;
      int cnt = 0;
#pragma unroll 8
      for (int64_t p = a; p < b; ++p) cnt += route.ids[p] == expert;
      int found;
      int rank = block_exclusive_sum(cnt, gsum, &found);
      if (tid == 0) gsum[kThreads / 64] = -1;
      __syncthreads();
      if (cnt > 0)
        for (int64_t p = a; p < b; ++p)
          if (route.ids[p] == expert) {
            if (rank < kGList) glist[rank] = (int)p;
            else if (rank == kGList) gsum[kThreads / 64] = (int)p;  // first pair left over
            ++rank;
          }
      __syncthreads();
      const int listed = found < kGList ? found : kGList;
      pos = found > kGList ? (int64_t)gsum[kThreads / 64] : total;
      for (int r0 = 0; r0 < listed; r0 += TBM) tile(r0, listed - r0 < TBM ? listed - r0 : TBM);
    }
  }
}

template <int BITS, typename XT>
hipError_t qmm_wr_launch(const void *x, int64_t M, const uint32_t *codes, const uint16_t *scales,
                         const uint16_t *biases, int64_t N, int64_t K, int G, void *y,
                         hipStream_t s) {
  const int64_t mt = (M + BM - 1) / BM, nt = (N + WBN - 1) / WBN;
  if (nt > 0x7FFFFFFF || 2 * mt > 65535) return hipErrorInvalidValue;  // grid limits
  if ((int64_t)BM * K * 2 > 0x7FFFFFFF) return hipErrorInvalidValue;  // 32-bit tile offsets
  // One block per compute unit at a time: when the tiles leave a last round
  // at most half full, and that remainder is a whole number of column tiles,
  // those columns run as 128-column tiles in a second launch (twice the
  // blocks, half the work each), which fills the chip for that round.  At
  // 2048 x 28672: 896 tiles = 768 (three rounds) + 16 columns of 8, run as
  // 256 half tiles.  Halving the columns rather than the rows keeps each
  // dequantized weight fragment serving 8 row blocks (measured on the MI355X,
  // 4-bit: the tail took 169-193 us as 128 x 256 tiles).
  const int64_t cus = device_cus(), rem = (mt * nt) % cus;
  const int64_t ntail = rem > 0 && 2 * rem <= cus && rem % mt == 0 ? rem / mt : 0;
  const int64_t nmain = nt - ntail, n0 = nmain * WBN;
  const int64_t wpr = (K >> 5) * BITS, gpr = (K >> 5) / (G >> 5);
  uint16_t *yo = (uint16_t *)y;
  auto go = [&](auto nb, auto g1) {
    constexpr int NB = decltype(nb)::value;
    constexpr bool G1 = decltype(g1)::value;
    if (NB == 2)
      hipLaunchKernelGGL((qmm_wr_kernel<BITS, XT, 8, 2, G1, false>),
                         dim3((unsigned)nmain, (unsigned)mt), dim3(kThreads), 0, s,
                         (const uint16_t *)x, M, codes, scales, biases, n0 < N ? n0 : N, K, G, yo,
                         N, Routing{});
    else
      hipLaunchKernelGGL((qmm_wr_kernel<BITS, XT, 8, 1, G1, false>),
                         dim3((unsigned)((N - n0 + 127) / 128), (unsigned)mt), dim3(kThreads), 0,
                         s, (const uint16_t *)x, M, codes + n0 * wpr, scales + n0 * gpr,
                         biases ? biases + n0 * gpr : nullptr, N - n0, K, G, yo + n0, N,
                         Routing{});
  };
  using B2 = std::integral_constant<int, 2>;
  using B1 = std::integral_constant<int, 1>;
  if (nmain > 0) {
    if (G == 32) go(B2{}, std::true_type{});
    else go(B2{}, std::false_type{});
  }
  if (ntail > 0) {
    if (G == 32) go(B1{}, std::true_type{});
    else go(B1{}, std::false_type{});
  }
  return hipGetLastError();
}

template <int BITS, typename XT>
hipError_t gather_qmm_launch(const void *x, int64_t T, const uint32_t *codes,
                             const uint16_t *scales, const uint16_t *biases, int64_t E, int64_t N,
                             int64_t K, const int32_t *ids, int topk, int G, void *y,
                             hipStream_t s) {
  const int64_t nt = (N + WBN - 1) / WBN;
  // all of x is addressed with 32-bit byte offsets; pairs are listed as int
  if (T * K * 2 > 0x7FFFFFFF || T * topk > 0x7FFFFFFF || nt > 0x7FFFFFFF || E > 65535)
    return hipErrorInvalidValue;
  const Routing route{ids, T * topk, topk, E};
  if (G == 32)
    hipLaunchKernelGGL((qmm_wr_kernel<BITS, XT, 8, 2, true, true>), dim3((unsigned)nt, (unsigned)E),
                       dim3(kThreads), 0, s, (const uint16_t *)x, T, codes, scales, biases, N, K,
                       G, (uint16_t *)y, N, route);
  else
    hipLaunchKernelGGL((qmm_wr_kernel<BITS, XT, 8, 2, false, true>), dim3((unsigned)nt, (unsigned)E),
                       dim3(kThreads), 0, s, (const uint16_t *)x, T, codes, scales, biases, N, K,
                       G, (uint16_t *)y, N, route);
  return hipGetLastError();
}

template <typename XT>
hipError_t gather_qmm_bits(const void *x, int64_t T, const uint32_t *codes, const uint16_t *scales,
                           const uint16_t *biases, int64_t E, int64_t N, int64_t K,
                           const int32_t *ids, int topk, int G, int bits, void *y, hipStream_t s) {
  switch (bits) {
#define AQ_GQ(B) case B: return gather_qmm_launch<B, XT>(x, T, codes, scales, biases, E, N, K, ids, topk, G, y, s);
    AQ_GQ(2) AQ_GQ(3) AQ_GQ(4) AQ_GQ(5) AQ_GQ(6) AQ_GQ(7) AQ_GQ(8)
#undef AQ_GQ
  }
  return hipErrorInvalidValue;
}

template <typename XT>
hipError_t qmm_bits(const void *x, int64_t M, const uint32_t *codes, const uint16_t *scales,
                    const uint16_t *biases, int64_t N, int64_t K, int G, int bits, void *y,
                    hipStream_t s) {
#define AQ_QL qmm_wr_launch
  switch (bits) {
    case 2: return AQ_QL<2, XT>(x, M, codes, scales, biases, N, K, G, y, s);
    case 3: return AQ_QL<3, XT>(x, M, codes, scales, biases, N, K, G, y, s);
    case 4: return AQ_QL<4, XT>(x, M, codes, scales, biases, N, K, G, y, s);
    case 5: return AQ_QL<5, XT>(x, M, codes, scales, biases, N, K, G, y, s);
    case 6: return AQ_QL<6, XT>(x, M, codes, scales, biases, N, K, G, y, s);
    case 7: return AQ_QL<7, XT>(x, M, codes, scales, biases, N, K, G, y, s);
    case 8: return AQ_QL<8, XT>(x, M, codes, scales, biases, N, K, G, y, s);
  }
#undef AQ_QL
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

hipError_t launch_gather_qmm(const void *x, int x_dtype, int64_t T, const uint32_t *codes,
                             const uint16_t *scales, const uint16_t *biases, int64_t E, int64_t N,
                             int64_t K, const int32_t *ids, int topk, int G, int bits, void *y,
                             hipStream_t s) {
  if (x_dtype == X_F16)
    return gather_qmm_bits<f16_t>(x, T, codes, scales, biases, E, N, K, ids, topk, G, bits, y, s);
  if (x_dtype == X_BF16)
    return gather_qmm_bits<bf16_t>(x, T, codes, scales, biases, E, N, K, ids, topk, G, bits, y, s);
  return hipErrorInvalidValue;
}

}  // namespace aq
