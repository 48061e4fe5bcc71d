// aq_internal.hpp -- kernel launchers behind the C ABI (arguments already
// validated by aq_api.cpp).  Each returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aq {

enum XType { X_F32 = 0, X_F16 = 1, X_BF16 = 2 };

// compute units of the current device (cached per device)
int device_cus();

hipError_t launch_quantize(const void *w, int w_dtype, int64_t N, int64_t K, int G, int bits,
                           uint32_t *codes, uint16_t *scales, uint16_t *biases, hipStream_t s);

// range-search quantize: steps candidate ranges per group, least squared error
hipError_t launch_quantize_mse(const void *w, int w_dtype, int64_t N, int64_t K, int G, int bits,
                               int steps, uint32_t *codes, uint16_t *scales, uint16_t *biases,
                               hipStream_t s);

// integer zero points: bias = -z*s exactly, z in [0, 2^bits - 1]; zeros may be null
hipError_t launch_quantize_zp(const void *w, int w_dtype, int64_t N, int64_t K, int G, int bits,
                              uint32_t *codes, uint16_t *scales, uint16_t *biases, uint8_t *zeros,
                              hipStream_t s);

hipError_t launch_dequantize(const uint32_t *codes, const uint16_t *scales,
                             const uint16_t *biases, int64_t N, int64_t K, int G, int bits,
                             void *out, int out_dtype, hipStream_t s);

// quantized embedding: out[t, :] = dequantize(table row ids[t]), zero rows for
// ids outside [0, V)
hipError_t launch_embedding(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                            int64_t V, int64_t K, int G, int bits, const int32_t *ids, int64_t T,
                            void *out, int out_dtype, hipStream_t s);

// y[M, N] = x[M, K] @ W^T for 1 <= M <= 8 (matrix-vector kernels)
hipError_t launch_qmv(const void *x, int x_dtype, int M, const uint32_t *codes,
                      const uint16_t *scales, const uint16_t *biases, int64_t N, int64_t K, int G,
                      int bits, void *y, hipStream_t s);

// y[M, N] = x[M, K] @ W^T for a few rows on the matrix cores (4-bit and
// 8-bit codes; more than 16 rows run as slices of 16); qmvm_supported says
// which shapes it takes, qmvm_preferred whether it beats the tiled matmul
// kernel at M > 8
constexpr int kQmvmMaxRows = 256;
bool qmvm_supported(int M, int bits, int64_t N, int64_t K, int G);
bool qmvm_preferred(int64_t M, int bits, int64_t N, int64_t K, int G);
// launch shapes the kernels use (also reported by aq_qmv_describe)
void qmvm_shape(int M, int bits, int64_t N, int64_t K, int G, int &R, int &W, int &XR);
void qmv1_shape(int64_t N, int64_t K, int G, int &cpl, int &ud, int &w, int &sl, int &wpc);
hipError_t launch_qmvm(const void *x, int x_dtype, int M, const uint32_t *codes,
                       const uint16_t *scales, const uint16_t *biases, int64_t N, int64_t K, int G,
                       int bits, void *y, hipStream_t s);

// the mixture-of-experts gather on the matrix cores (4-bit and 8-bit codes;
// gather_qmvm_supported says which shapes it takes)
bool gather_qmvm_supported(int bits, int64_t K, int G);
hipError_t launch_gather_qmvm(const void *x, int x_dtype, int64_t T, const uint32_t *codes,
                              const uint16_t *scales, const uint16_t *biases, int64_t E, int64_t N,
                              int64_t K, const int32_t *ids, int topk, int G, int bits, void *y,
                              hipStream_t s);

// mixture-of-experts gather: y[t, j, :] = x[t] @ W_{ids[t, j]}^T
hipError_t launch_gather_qmv(const void *x, int x_dtype, int64_t T, const uint32_t *codes,
                             const uint16_t *scales, const uint16_t *biases, int64_t E, int64_t N,
                             int64_t K, const int32_t *ids, int topk, int G, int bits, void *y,
                             hipStream_t s);

// y[M, N] = x[M, K] @ W^T for any M (matrix-core kernel)
hipError_t launch_qmm(const void *x, int x_dtype, int64_t M, const uint32_t *codes,
                      const uint16_t *scales, const uint16_t *biases, int64_t N, int64_t K, int G,
                      int bits, void *y, hipStream_t s);

// mixture-of-experts gather at prefill size on the matrix cores: y[t, j, :] =
// x[t] @ W_{ids[t, j]}^T, experts' pairs listed on the device
hipError_t launch_gather_qmm(const void *x, int x_dtype, int64_t T, const uint32_t *codes,
                             const uint16_t *scales, const uint16_t *biases, int64_t E, int64_t N,
                             int64_t K, const int32_t *ids, int topk, int G, int bits, void *y,
                             hipStream_t s);

// block-scaled float modes: mxfp4 (E2M1 codes, exponent byte per 32), nvfp4
// (E2M1 codes, E4M3 scale per 16, tensor scale 2^T), mxfp8 (E4M3 codes,
// exponent byte per 32)
enum FpMode { FP_MXFP4 = 0, FP_NVFP4 = 1, FP_MXFP8 = 2 };
constexpr int64_t kFpMaxK = 49152;  // the decode kernel keeps x (K * 2 bytes) in LDS
hipError_t launch_quantize_fp(const void *w, int w_dtype, int64_t N, int64_t K, int mode, int T,
                              uint32_t *codes, uint8_t *scales, hipStream_t s);
hipError_t launch_dequantize_fp(const uint32_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                                int mode, int T, void *out, int out_dtype, hipStream_t s);
// y[N] = x[K] @ W^T; cpl = 0 is the LDS kernel for K > 16384
void qmv1_fp_shape(int64_t N, int64_t K, int mode, int &cpl, int &ud, int &w, int &wpc);
hipError_t launch_qmv_fp(const void *x, int x_dtype, const uint32_t *codes, const uint8_t *scales,
                         int64_t N, int64_t K, int mode, int T, void *y, hipStream_t s);
// y = x @ W^T for M >= 2 rows of x (slices of 16) and block-scaled W
hipError_t launch_mm_fp_rows(const void *x, int x_dtype, int64_t M, const uint32_t *codes,
                             const uint8_t *scales, int64_t N, int64_t K, int mode, int T, void *y,
                             hipStream_t s);
// y[t, j, :] = x[t] @ W_{ids[t, j]}^T, block-scaled experts W [E, N, K]
hipError_t launch_gather_mm_fp(const void *x, int x_dtype, int64_t Tk, const uint32_t *codes,
                               const uint8_t *scales, int64_t E, int64_t N, int64_t K,
                               const int32_t *ids, int topk, int mode, int T, void *y,
                               hipStream_t s);

}  // namespace aq
