// aq_bench.hip -- measurement helpers declared in include/aq_bench.h: a plain
// streaming-read kernel (the bandwidth a kernel of a given byte count can
// reach on this device) and an MFMA-only loop that records the shader clock.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "aq_bench.h"

namespace {

// grid-stride streaming read, U independent 16-byte loads in flight per thread
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *__restrict__ p, int64_t n16,
                                                          uint32_t *sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + u * stride;
      v[u] = j < n16 ? p[j] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // practically never; keeps the loads alive
}

// one-shot streaming read: workgroup b reads the contiguous block of
// blockDim * U 16-byte units at b * blockDim * U; every thread issues its U
// loads before using any of them
template <int U>
__global__ __launch_bounds__(1024) void read_oneshot_kernel(const uint4 *__restrict__ p, int64_t n16,
                                                            uint32_t *sink) {
  const int64_t base = (int64_t)blockIdx.x * blockDim.x * U + threadIdx.x;
  uint4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t j = base + (int64_t)u * blockDim.x;
    v[u] = j < n16 ? p[j] : make_uint4(0, 0, 0, 0);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  if (acc == 0x9E3779B9u) sink[0] = acc;  // practically never; keeps the loads alive
}

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef float f32x16v __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_clock_kernel(int iters, uint64_t *out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f32x16v acc[14];
#pragma unroll
  for (int j = 0; j < 14; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  // operands: small exact bf16 values derived from the lane (0x3F80 = 1.0)
  const uint32_t w = 0x3F803F80u + (uint32_t)(lane & 7);
  const uint4 a = make_uint4(w, w, w, w), b = make_uint4(w ^ 1u, w, w, w ^ 1u);
  const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 14; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8v, a),
                                                       __builtin_bit_cast(bf16x8v, b), acc[j], 0, 0,
                                                       0);
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 14; ++j) s += acc[j][0];
  if (lane == 0) {
    uint64_t *o = out + ((int64_t)blockIdx.x * 4 + wave) * 2;
    o[0] = c1 - c0 + (s == -1.f ? 1u : 0u);  // the sum keeps the MFMAs alive
    o[1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

aq_status aq_bench_stream_read(const void *buf, int64_t bytes, int blocks, int unroll,
                               uint32_t *sink, void *stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 != 0 || blocks < 1 || blocks > 65535)
    return AQ_ERR_INVALID_ARG;
  if (unroll != 1 && unroll != 4 && unroll != 8) return AQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0) return AQ_ERR_ALIGNMENT;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const uint4 *p = static_cast<const uint4 *>(buf);
  const int64_t n16 = bytes / 16;
  switch (unroll) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, dim3(blocks), dim3(256), 0, s, p, n16, sink); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(blocks), dim3(256), 0, s, p, n16, sink); break;
    default: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(blocks), dim3(256), 0, s, p, n16, sink); break;
  }
  return hipGetLastError() == hipSuccess ? AQ_OK : AQ_ERR_HIP;
}

aq_status aq_bench_read_oneshot(const void *buf, int64_t bytes, int threads, int unroll,
                                uint32_t *sink, void *stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 != 0) return AQ_ERR_INVALID_ARG;
  if (threads != 256 && threads != 512 && threads != 1024) return AQ_ERR_INVALID_ARG;
  if (unroll != 4 && unroll != 8 && unroll != 16) return AQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0) return AQ_ERR_ALIGNMENT;
  const int64_t n16 = bytes / 16, per = (int64_t)threads * unroll;
  const int64_t blocks = (n16 + per - 1) / per;
  if (blocks > 0x7FFFFFFF) return AQ_ERR_UNSUPPORTED;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const uint4 *p = static_cast<const uint4 *>(buf);
  const dim3 grid((unsigned)blocks), block((unsigned)threads);
  switch (unroll) {
    case 4: hipLaunchKernelGGL(read_oneshot_kernel<4>, grid, block, 0, s, p, n16, sink); break;
    case 8: hipLaunchKernelGGL(read_oneshot_kernel<8>, grid, block, 0, s, p, n16, sink); break;
    default: hipLaunchKernelGGL(read_oneshot_kernel<16>, grid, block, 0, s, p, n16, sink); break;
  }
  return hipGetLastError() == hipSuccess ? AQ_OK : AQ_ERR_HIP;
}

aq_status aq_bench_mfma_clock(int blocks, int iters, uint64_t *out, void *stream) {
  if (!out || blocks < 1 || blocks > 65535 || iters < 1 || iters > (1 << 24))
    return AQ_ERR_INVALID_ARG;
  hipLaunchKernelGGL(mfma_clock_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), iters, out);
  return hipGetLastError() == hipSuccess ? AQ_OK : AQ_ERR_HIP;
}

}  // extern "C"
