// aq_qmm.hip -- quantized matrix-matrix product (prefill) on the gfx950 matrix
// cores.
//
// The operation is Y = X @ W^T with W in packed form ("Quantization",
// metalworking MLX notes, QMM: dequantize tiles into on-chip memory, then a
// tiled GEMM against them).  On MI355X:
//  * a 256-thread workgroup computes a BM x BN tile of Y; 4 waves in a 2x2
//    arrangement each own a (BM/2) x (BN/2) sub-tile built from 32x32 blocks
//    of v_mfma_f32_32x32x16_{bf16,f16} (binary32 accumulation);
//  * per K step of 64, the X tile is copied to LDS, and the W tile is read as
//    packed codes, dequantized in registers (q*s + b in binary32, rounded to
//    nearest even into the activation type, i.e. exactly what aq_dequantize
//    produces) and written to LDS; both tiles use a 144-byte row pitch so the
//    16-byte fragment reads of 16 lanes fall in disjoint banks;
//  * the LDS tiles are double-buffered: the global loads for step k+1 are in
//    flight while the matrix cores work on step k.
#include "aq_device.hpp"
#include "aq_internal.hpp"

namespace aq {
namespace {

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8v __attribute__((ext_vector_type(8)));
typedef float f32x16v __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kPitch = BK + 8;  // elements per LDS row (144 bytes)
constexpr int kThreads = 256;

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

// registers holding one K step's global data for this thread
template <int BITS>
struct StepRegs {
  uint4 x[4];       // 4 x 8 activation values
  uint32_t w[BITS]; // one 32-code chunk
  uint32_t sb;      // scale | bias << 16
};

template <int BITS, typename XT>
__global__ __launch_bounds__(kThreads) void qmm_kernel(const uint16_t *__restrict__ x, int64_t M,
                                                       const uint32_t *__restrict__ codes,
                                                       const uint16_t *__restrict__ scales,
                                                       const uint16_t *__restrict__ biases,
                                                       int64_t N, int64_t K, int G,
                                                       uint16_t *__restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][BM * kPitch];  // [buf][X|W]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tile_n = (int64_t)blockIdx.x * BN, tile_m = (int64_t)blockIdx.y * BM;
  const int64_t nchunks = K >> 5, wpr = nchunks * BITS, gpr = K / G;
  const int ksteps = (int)((K + BK - 1) / BK);

  // this thread's W chunk: row wr of the tile, chunk half wh of the K step
  const int wr = tid >> 1, wh = tid & 1;
  int64_t wrow = tile_n + wr;
  const bool wrow_ok = wrow < N;
  if (!wrow_ok) wrow = N - 1;

  auto load_step = [&](int ks, StepRegs<BITS> &r) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + kThreads * i;
      const int row = idx >> 3, c8 = idx & 7;
      const int64_t m = tile_m + row, k = (int64_t)ks * BK + c8 * 8;
      if (m < M && k < K)
        r.x[i] = *reinterpret_cast<const uint4 *>(x + m * K + k);
      else
        r.x[i] = make_uint4(0, 0, 0, 0);
    }
    int64_t c = (int64_t)ks * 2 + wh;
    if (c >= nchunks) c = nchunks - 1;  // zeroed at store time
    load_chunk<BITS>(codes + wrow * wpr + c * BITS, r.w);
    const int64_t g = (c << 5) / G;
    r.sb = (uint32_t)scales[wrow * gpr + g] | ((uint32_t)biases[wrow * gpr + g] << 16);
  };

  auto store_step = [&](int ks, const StepRegs<BITS> &r, int buf) {
    uint16_t *lx = lds[buf][0];
    uint16_t *lw = lds[buf][1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + kThreads * i;
      const int row = idx >> 3, c8 = idx & 7;
      *reinterpret_cast<uint4 *>(lx + row * kPitch + c8 * 8) = r.x[i];
    }
    const bool ok = wrow_ok && ((int64_t)ks * 2 + wh) < nchunks;
    const float s = f16_to_f32((uint16_t)(r.sb & 0xFFFFu));
    const float b = f16_to_f32((uint16_t)(r.sb >> 16));
    uint32_t p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float lo = __builtin_fmaf((float)chunk_code<BITS>(r.w, 2 * i), s, b);
      const float hi = __builtin_fmaf((float)chunk_code<BITS>(r.w, 2 * i + 1), s, b);
      p[i] = ok ? pack2<XT>(lo, hi) : 0u;
    }
    uint4 *dst = reinterpret_cast<uint4 *>(lw + wr * kPitch + wh * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = make_uint4(p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]);
  };

  f32x16v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  StepRegs<BITS> regs;
  load_step(0, regs);
  store_step(0, regs, 0);
  __syncthreads();

  const int frow = lane & 31, fk = (lane >> 5) * 8;
  for (int ks = 0; ks < ksteps; ++ks) {
    const int buf = ks & 1;
    const bool more = ks + 1 < ksteps;
    if (more) load_step(ks + 1, regs);
    const uint16_t *lx = lds[buf][0];
    const uint16_t *lw = lds[buf][1];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      uint4 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const uint4 *>(lx + (wm * 64 + i * 32 + frow) * kPitch + kk * 16 + fk);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const uint4 *>(lw + (wn * 64 + j * 32 + frow) * kPitch + kk * 16 + fk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32<XT>(a[i], b[j], acc[i][j]);
    }
    if (more) store_step(ks + 1, regs, buf ^ 1);
    __syncthreads();
  }

  // epilogue: accumulator r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = tile_n + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = tile_m + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < M && n < N) y[m * N + n] = xtraits<XT>::from_f32(acc[i][j][r]);
      }
    }
}

template <typename XT>
hipError_t qmm_bits(const void *x, int64_t M, const uint32_t *codes, const uint16_t *scales,
                    const uint16_t *biases, int64_t N, int64_t K, int G, int bits, void *y,
                    hipStream_t s) {
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
#define AQ_M(B) case B: hipLaunchKernelGGL((qmm_kernel<B, XT>), grid, dim3(kThreads), 0, s, (const uint16_t *)x, M, codes, scales, biases, N, K, G, (uint16_t *)y); break;
  switch (bits) {
    AQ_M(2) AQ_M(3) AQ_M(4) AQ_M(5) AQ_M(6) AQ_M(7) AQ_M(8)
    default: return hipErrorInvalidValue;
  }
#undef AQ_M
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qmm(const void *x, int x_dtype, int64_t M, const uint32_t *codes,
                      const uint16_t *scales, const uint16_t *biases, int64_t N, int64_t K, int G,
                      int bits, void *y, hipStream_t s) {
  if (M > 65535 * (int64_t)BM) return hipErrorInvalidValue;
  if (x_dtype == X_F16) return qmm_bits<f16_t>(x, M, codes, scales, biases, N, K, G, bits, y, s);
  if (x_dtype == X_BF16) return qmm_bits<bf16_t>(x, M, codes, scales, biases, N, K, G, bits, y, s);
  return hipErrorInvalidValue;
}

}  // namespace aq
