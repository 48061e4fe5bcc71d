// aq_api.cpp -- the extern "C" entry points of libaq (declared in include/aq.h):
// host-side argument validation, shape dispatch and kernel launch.
//
// Validation runs entirely on the host and touches no HIP API, so a bad call
// returns before anything is enqueued (and can be exercised on a machine
// without a GPU).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdio>

#include "aq.h"
#include "aq_internal.hpp"

namespace {

constexpr int64_t kMaxQmvRows = 8;
constexpr int64_t kMaxQmmK = 0x7FFFFFFF / (256 * 2);  // 4194303
// the prefill grid: 256-column tiles in x, 256-row tiles (or twice as many
// 128-row halves for a split last round) in y, at most 65535
constexpr int64_t kMaxQmmM = 65535 / 2 * 256;  // 8388352

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_format(int64_t N, int64_t K, int G, int bits) {
  if (N < 1 || K < 1) return false;
  if (G != 32 && G != 64 && G != 128) return false;
  if (bits < 2 || bits > 8) return false;
  if (K % G != 0) return false;
  return true;
}

bool valid_act_dtype(int d) { return d == AQ_F16 || d == AQ_BF16; }

aq_status from_hip(hipError_t e) { return e == hipSuccess ? AQ_OK : AQ_ERR_HIP; }

// outputs of the quantizers: all three arrays required
aq_status check_weights(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases) {
  if (!codes || !scales || !biases) return AQ_ERR_INVALID_ARG;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(biases)) return AQ_ERR_ALIGNMENT;
  return AQ_OK;
}

// inputs of the consumers: a null bias array means every bias is +0
aq_status check_packed(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases) {
  if (!codes || !scales) return AQ_ERR_INVALID_ARG;
  if (!aligned16(codes) || !aligned16(scales) || (biases && !aligned16(biases)))
    return AQ_ERR_ALIGNMENT;
  return AQ_OK;
}

aq_status check_matmul(const void *x, int x_dtype, int64_t M, const uint32_t *codes,
                       const uint16_t *scales, const uint16_t *biases, int64_t N, int64_t K,
                       int G, int bits, const void *y) {
  if (!valid_format(N, K, G, bits) || M < 1 || !valid_act_dtype(x_dtype))
    return AQ_ERR_INVALID_ARG;
  if (!x || !y) return AQ_ERR_INVALID_ARG;
  aq_status st = check_packed(codes, scales, biases);
  if (st != AQ_OK) return st;
  if (!aligned16(x) || !aligned16(y)) return AQ_ERR_ALIGNMENT;
  return AQ_OK;
}

}  // namespace

namespace aq {

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
      v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

}  // namespace aq

extern "C" {

const char *aq_status_string(aq_status status) {
  switch (status) {
    case AQ_OK: return "AQ_OK";
    case AQ_ERR_INVALID_ARG: return "AQ_ERR_INVALID_ARG: invalid argument";
    case AQ_ERR_UNSUPPORTED: return "AQ_ERR_UNSUPPORTED: not supported by this build";
    case AQ_ERR_ALIGNMENT: return "AQ_ERR_ALIGNMENT: pointer not 16-byte aligned";
    case AQ_ERR_HIP: return "AQ_ERR_HIP: HIP runtime error at launch";
    case AQ_ERR_RANGE: return "AQ_ERR_RANGE: value out of range";
    case AQ_ERR_INDEX: return "AQ_ERR_INDEX: index out of range";
    default: break;
  }
  return "unknown aq_status";
}

const char *aq_version(void) { return "libaq 0.1 (gfx950)"; }

int64_t aq_codes_words(int64_t K, int bits) {
  if (K < 0 || bits < 2 || bits > 8 || (K * bits) % 32 != 0) return -1;
  return K * bits / 32;
}

int64_t aq_qweight_bytes(int64_t N, int64_t K, int group_size, int bits) {
  if (N < 0 || K < 0 || (group_size != 32 && group_size != 64 && group_size != 128) || bits < 2 ||
      bits > 8 || K % group_size != 0)
    return -1;
  return N * K * bits / 8 + N * (K / group_size) * 4;
}

aq_status aq_quantize(const void *w, aq_dtype w_dtype, int64_t N, int64_t K, int group_size,
                      int bits, uint32_t *codes, uint16_t *scales, uint16_t *biases,
                      void *stream) {
  if (!valid_format(N, K, group_size, bits)) return AQ_ERR_INVALID_ARG;
  if (w_dtype != AQ_F32 && w_dtype != AQ_F16 && w_dtype != AQ_BF16) return AQ_ERR_INVALID_ARG;
  if (!w) return AQ_ERR_INVALID_ARG;
  aq_status st = check_weights(codes, scales, biases);
  if (st != AQ_OK) return st;
  if (!aligned16(w)) return AQ_ERR_ALIGNMENT;
  if (N * (K / 8) > (int64_t)0x7FFFFFFF * 256) return AQ_ERR_UNSUPPORTED;
  return from_hip(aq::launch_quantize(w, (int)w_dtype, N, K, group_size, bits, codes, scales,
                                      biases, static_cast<hipStream_t>(stream)));
}

aq_status aq_quantize_mse(const void *w, aq_dtype w_dtype, int64_t N, int64_t K, int group_size,
                          int bits, int steps, uint32_t *codes, uint16_t *scales, uint16_t *biases,
                          void *stream) {
  if (!valid_format(N, K, group_size, bits) || steps < 1 || steps > 50) return AQ_ERR_INVALID_ARG;
  if (w_dtype != AQ_F32 && w_dtype != AQ_F16 && w_dtype != AQ_BF16) return AQ_ERR_INVALID_ARG;
  if (!w) return AQ_ERR_INVALID_ARG;
  aq_status st = check_weights(codes, scales, biases);
  if (st != AQ_OK) return st;
  if (!aligned16(w)) return AQ_ERR_ALIGNMENT;
  if (N * (K / 8) > (int64_t)0x7FFFFFFF * 256) return AQ_ERR_UNSUPPORTED;
  return from_hip(aq::launch_quantize_mse(w, (int)w_dtype, N, K, group_size, bits, steps, codes,
                                          scales, biases, static_cast<hipStream_t>(stream)));
}

aq_status aq_quantize_zp(const void *w, aq_dtype w_dtype, int64_t N, int64_t K, int group_size,
                         int bits, uint32_t *codes, uint16_t *scales, uint16_t *biases,
                         uint8_t *zeros, void *stream) {
  if (!valid_format(N, K, group_size, bits)) return AQ_ERR_INVALID_ARG;
  if (w_dtype != AQ_F32 && w_dtype != AQ_F16 && w_dtype != AQ_BF16) return AQ_ERR_INVALID_ARG;
  if (!w) return AQ_ERR_INVALID_ARG;
  aq_status st = check_weights(codes, scales, biases);
  if (st != AQ_OK) return st;
  if (!aligned16(w) || (zeros && !aligned16(zeros))) return AQ_ERR_ALIGNMENT;
  if (N * (K / 8) > (int64_t)0x7FFFFFFF * 256) return AQ_ERR_UNSUPPORTED;
  return from_hip(aq::launch_quantize_zp(w, (int)w_dtype, N, K, group_size, bits, codes, scales,
                                         biases, zeros, static_cast<hipStream_t>(stream)));
}

aq_status aq_dequantize(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                        int64_t N, int64_t K, int group_size, int bits, void *out,
                        aq_dtype out_dtype, void *stream) {
  if (!valid_format(N, K, group_size, bits)) return AQ_ERR_INVALID_ARG;
  if (out_dtype != AQ_F32 && out_dtype != AQ_F16 && out_dtype != AQ_BF16) return AQ_ERR_INVALID_ARG;
  if (!out) return AQ_ERR_INVALID_ARG;
  aq_status st = check_packed(codes, scales, biases);
  if (st != AQ_OK) return st;
  if (!aligned16(out)) return AQ_ERR_ALIGNMENT;
  if (N * (K / 32) > (int64_t)0x7FFFFFFF * 256) return AQ_ERR_UNSUPPORTED;
  return from_hip(aq::launch_dequantize(codes, scales, biases, N, K, group_size, bits, out,
                                        (int)out_dtype, static_cast<hipStream_t>(stream)));
}

aq_status aq_embedding(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                       int64_t V, int64_t K, int group_size, int bits, const int32_t *ids,
                       int64_t T, void *out, aq_dtype out_dtype, void *stream) {
  if (!valid_format(V, K, group_size, bits) || T < 1) return AQ_ERR_INVALID_ARG;
  if (out_dtype != AQ_F32 && out_dtype != AQ_F16 && out_dtype != AQ_BF16) return AQ_ERR_INVALID_ARG;
  if (!out || !ids) return AQ_ERR_INVALID_ARG;
  aq_status st = check_packed(codes, scales, biases);
  if (st != AQ_OK) return st;
  if (!aligned16(out) || !aligned16(ids)) return AQ_ERR_ALIGNMENT;
  if (T * (K / 32) > (int64_t)0x7FFFFFFF * 256) return AQ_ERR_UNSUPPORTED;
  return from_hip(aq::launch_embedding(codes, scales, biases, V, K, group_size, bits, ids, T, out,
                                       (int)out_dtype, static_cast<hipStream_t>(stream)));
}

aq_status aq_qmv(const void *x, aq_dtype x_dtype, int64_t M, const uint32_t *codes,
                 const uint16_t *scales, const uint16_t *biases, int64_t N, int64_t K,
                 int group_size, int bits, void *y, void *stream) {
  aq_status st = check_matmul(x, x_dtype, M, codes, scales, biases, N, K, group_size, bits, y);
  if (st != AQ_OK) return st;
  if (M > kMaxQmvRows) return AQ_ERR_INVALID_ARG;
  // 2..8 rows of 4-bit or 8-bit codes: dot products on the matrix cores
  if (aq::qmvm_supported((int)M, bits, N, K, group_size))
    return from_hip(aq::launch_qmvm(x, (int)x_dtype, (int)M, codes, scales, biases, N, K,
                                    group_size, bits, y, static_cast<hipStream_t>(stream)));
  return from_hip(aq::launch_qmv(x, (int)x_dtype, (int)M, codes, scales, biases, N, K, group_size,
                                 bits, y, static_cast<hipStream_t>(stream)));
}

int aq_qmv_describe(int64_t M, int64_t N, int64_t K, int group_size, int bits, aq_dtype x_dtype,
                    char *buf, int len) {
  if (!valid_format(N, K, group_size, bits) || M < 1 || M > kMaxQmvRows ||
      !valid_act_dtype(x_dtype) || !buf || len < 1)
    return -1;
  const char *xt = x_dtype == AQ_F16 ? "f16" : "bf16";
  if (M == 1 && K <= 8 * 2048) {
    int cpl, ud, w, sl, wpc;
    aq::qmv1_shape(N, K, group_size, cpl, ud, w, sl, wpc);
    return snprintf(buf, (size_t)len, "qmv1_kernel<BITS=%d, %s, CPL=%d, UD=%d, W=%d, SL=%d>", bits,
                    xt, cpl, ud, w, sl);
  }
  if (aq::qmvm_supported((int)M, bits, N, K, group_size)) {
    int R, W, XR;
    aq::qmvm_shape((int)M, bits, N, K, group_size, R, W, XR);
    return snprintf(buf, (size_t)len, "qmvm_kernel<%s, BITS=%d, W=%d, G=%d, XR=%d, R=%d>", xt,
                    bits, W, group_size, XR, R);
  }
  return snprintf(buf, (size_t)len, "qmv vector kernel<BITS=%d, %s, M=%d>", bits, xt, (int)M);
}

aq_status aq_qmm(const void *x, aq_dtype x_dtype, int64_t M, const uint32_t *codes,
                 const uint16_t *scales, const uint16_t *biases, int64_t N, int64_t K,
                 int group_size, int bits, void *y, void *stream) {
  aq_status st = check_matmul(x, x_dtype, M, codes, scales, biases, N, K, group_size, bits, y);
  if (st != AQ_OK) return st;
  // the kernel addresses a 256-row tile of x with 32-bit byte offsets
  if (K > kMaxQmmK || M > kMaxQmmM || (N + 255) / 256 > 0x7FFFFFFF) return AQ_ERR_UNSUPPORTED;
  return from_hip(aq::launch_qmm(x, (int)x_dtype, M, codes, scales, biases, N, K, group_size,
                                 bits, y, static_cast<hipStream_t>(stream)));
}

aq_status aq_quantized_matmul(const void *x, aq_dtype x_dtype, int64_t M, const uint32_t *codes,
                              const uint16_t *scales, const uint16_t *biases, int64_t N,
                              int64_t K, int group_size, int bits, void *y, void *stream) {
  if (M >= 1 && M <= kMaxQmvRows)
    return aq_qmv(x, x_dtype, M, codes, scales, biases, N, K, group_size, bits, y, stream);
  // a few rows more: the tiled kernel's 256-row tiles would be mostly empty
  // and too few to fill the chip (arguments validated before the shape
  // heuristics look at them)
  if (M > kMaxQmvRows) {
    aq_status st = check_matmul(x, x_dtype, M, codes, scales, biases, N, K, group_size, bits, y);
    if (st != AQ_OK) return st;
    if (aq::qmvm_preferred(M, bits, N, K, group_size))
      return from_hip(aq::launch_qmvm(x, (int)x_dtype, (int)M, codes, scales, biases, N, K,
                                      group_size, bits, y, static_cast<hipStream_t>(stream)));
  }
  return aq_qmm(x, x_dtype, M, codes, scales, biases, N, K, group_size, bits, y, stream);
}

static aq_status check_gather(const void *x, aq_dtype x_dtype, int64_t T, const uint32_t *codes,
                              const uint16_t *scales, const uint16_t *biases, int64_t E,
                              int64_t N, int64_t K, const int32_t *ids, int topk, int group_size,
                              int bits, const void *y) {
  if (!valid_format(N, K, group_size, bits) || T < 1 || E < 1 || topk < 1 ||
      !valid_act_dtype(x_dtype))
    return AQ_ERR_INVALID_ARG;
  if (!x || !y || !ids) return AQ_ERR_INVALID_ARG;
  aq_status st = check_packed(codes, scales, biases);
  if (st != AQ_OK) return st;
  if (!aligned16(x) || !aligned16(y) || !aligned16(ids)) return AQ_ERR_ALIGNMENT;
  if (E > 65535 || T * topk > 0x7FFFFFFF) return AQ_ERR_UNSUPPORTED;
  return AQ_OK;
}

aq_status aq_gather_qmm(const void *x, aq_dtype x_dtype, int64_t T, const uint32_t *codes,
                        const uint16_t *scales, const uint16_t *biases, int64_t E, int64_t N,
                        int64_t K, const int32_t *ids, int topk, int group_size, int bits,
                        void *y, void *stream) {
  aq_status st = check_gather(x, x_dtype, T, codes, scales, biases, E, N, K, ids, topk,
                              group_size, bits, y);
  if (st != AQ_OK) return st;
  if (T * K * 2 > 0x7FFFFFFF) return AQ_ERR_UNSUPPORTED;
  return from_hip(aq::launch_gather_qmm(x, (int)x_dtype, T, codes, scales, biases, E, N, K, ids,
                                        topk, group_size, bits, y,
                                        static_cast<hipStream_t>(stream)));
}

aq_status aq_gather_quantized_matmul(const void *x, aq_dtype x_dtype, int64_t T,
                                     const uint32_t *codes, const uint16_t *scales,
                                     const uint16_t *biases, int64_t E, int64_t N, int64_t K,
                                     const int32_t *ids, int topk, int group_size, int bits,
                                     void *y, void *stream) {
  if (T >= 1 && topk >= 1 && E >= 1 && T * topk >= 32 * E && T * K * 2 <= 0x7FFFFFFF)
    return aq_gather_qmm(x, x_dtype, T, codes, scales, biases, E, N, K, ids, topk, group_size,
                         bits, y, stream);
  return aq_gather_qmv(x, x_dtype, T, codes, scales, biases, E, N, K, ids, topk, group_size, bits,
                       y, stream);
}

aq_status aq_gather_qmv(const void *x, aq_dtype x_dtype, int64_t T, const uint32_t *codes,
                        const uint16_t *scales, const uint16_t *biases, int64_t E, int64_t N,
                        int64_t K, const int32_t *ids, int topk, int group_size, int bits,
                        void *y, void *stream) {
  aq_status st = check_gather(x, x_dtype, T, codes, scales, biases, E, N, K, ids, topk,
                              group_size, bits, y);
  if (st != AQ_OK) return st;
  // 4-bit or 8-bit codes: batches of routed tokens on the matrix cores
  if (aq::gather_qmvm_supported(bits, K, group_size) && T * K * 2 <= 0x7FFFFFFF)
    return from_hip(aq::launch_gather_qmvm(x, (int)x_dtype, T, codes, scales, biases, E, N, K,
                                           ids, topk, group_size, bits, y,
                                           static_cast<hipStream_t>(stream)));
  return from_hip(aq::launch_gather_qmv(x, (int)x_dtype, T, codes, scales, biases, E, N, K, ids,
                                        topk, group_size, bits, y,
                                        static_cast<hipStream_t>(stream)));
}

// ---- block-scaled float modes ---------------------------------------------------------

// group size of a mode; 0 for an unknown mode
static int fp_group(int mode) {
  return mode == AQ_MXFP4 || mode == AQ_MXFP8 ? 32 : (mode == AQ_NVFP4 ? 16 : 0);
}

// shape, mode and tensor exponent (2^T only for nvfp4, |T| <= 100)
static bool valid_fp(int64_t N, int64_t K, int mode, int T) {
  const int g = fp_group(mode);
  if (g == 0 || N < 1 || K < g || K % g != 0) return false;
  return mode == AQ_NVFP4 ? (T >= -100 && T <= 100) : T == 0;
}

aq_status aq_quantize_fp(const void *w, aq_dtype w_dtype, int64_t N, int64_t K, aq_fp_mode mode,
                         int tensor_exp, uint32_t *codes, uint8_t *scales, void *stream) {
  if (!valid_fp(N, K, (int)mode, tensor_exp)) return AQ_ERR_INVALID_ARG;
  if (w_dtype != AQ_F32 && w_dtype != AQ_F16 && w_dtype != AQ_BF16) return AQ_ERR_INVALID_ARG;
  if (!w || !codes || !scales) return AQ_ERR_INVALID_ARG;
  if (!aligned16(w) || !aligned16(codes) || !aligned16(scales)) return AQ_ERR_ALIGNMENT;
  return from_hip(aq::launch_quantize_fp(w, (int)w_dtype, N, K, (int)mode, tensor_exp, codes,
                                         scales, static_cast<hipStream_t>(stream)));
}

aq_status aq_dequantize_fp(const uint32_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                           aq_fp_mode mode, int tensor_exp, void *out, aq_dtype out_dtype,
                           void *stream) {
  if (!valid_fp(N, K, (int)mode, tensor_exp)) return AQ_ERR_INVALID_ARG;
  if (out_dtype != AQ_F32 && out_dtype != AQ_F16 && out_dtype != AQ_BF16) return AQ_ERR_INVALID_ARG;
  if (!codes || !scales || !out) return AQ_ERR_INVALID_ARG;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(out)) return AQ_ERR_ALIGNMENT;
  return from_hip(aq::launch_dequantize_fp(codes, scales, N, K, (int)mode, tensor_exp, out,
                                           (int)out_dtype, static_cast<hipStream_t>(stream)));
}

aq_status aq_qmv_fp(const void *x, aq_dtype x_dtype, const uint32_t *codes,
                    const uint8_t *scales, int64_t N, int64_t K, aq_fp_mode mode, int tensor_exp,
                    void *y, void *stream) {
  if (!valid_fp(N, K, (int)mode, tensor_exp) || !valid_act_dtype(x_dtype))
    return AQ_ERR_INVALID_ARG;
  if (!x || !codes || !scales || !y) return AQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || !aligned16(y))
    return AQ_ERR_ALIGNMENT;
  // the kernels walk rows in 32-code chunks and hold x on chip
  if (K % 32 != 0 || K > aq::kFpMaxK) return AQ_ERR_UNSUPPORTED;
  return from_hip(aq::launch_qmv_fp(x, (int)x_dtype, codes, scales, N, K, (int)mode, tensor_exp,
                                    y, static_cast<hipStream_t>(stream)));
}

aq_status aq_matmul_fp(const void *x, aq_dtype x_dtype, int64_t M, const uint32_t *codes,
                       const uint8_t *scales, int64_t N, int64_t K, aq_fp_mode mode,
                       int tensor_exp, void *y, void *stream) {
  if (M < 1) return AQ_ERR_INVALID_ARG;
  if (M == 1) return aq_qmv_fp(x, x_dtype, codes, scales, N, K, mode, tensor_exp, y, stream);
  if (!valid_fp(N, K, (int)mode, tensor_exp) || !valid_act_dtype(x_dtype))
    return AQ_ERR_INVALID_ARG;
  if (!x || !codes || !scales || !y) return AQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || !aligned16(y))
    return AQ_ERR_ALIGNMENT;
  // 32-code chunks; 16 rows of x per grid slice (at most 65535 slices); the
  // scale array addressed with 32-bit byte offsets
  if (K % 32 != 0 || K > aq::kFpMaxK || M > 16 * 65535) return AQ_ERR_UNSUPPORTED;
  if (N * (K / (mode == AQ_NVFP4 ? 16 : 32)) > 0x7FFFFFF0) return AQ_ERR_UNSUPPORTED;
  return from_hip(aq::launch_mm_fp_rows(x, (int)x_dtype, M, codes, scales, N, K, (int)mode,
                                        tensor_exp, y, static_cast<hipStream_t>(stream)));
}

aq_status aq_gather_matmul_fp(const void *x, aq_dtype x_dtype, int64_t T, const uint32_t *codes,
                              const uint8_t *scales, int64_t E, int64_t N, int64_t K,
                              const int32_t *ids, int topk, aq_fp_mode mode, int tensor_exp,
                              void *y, void *stream) {
  if (!valid_fp(N, K, (int)mode, tensor_exp) || !valid_act_dtype(x_dtype) || T < 1 || E < 1 ||
      topk < 1)
    return AQ_ERR_INVALID_ARG;
  if (!x || !codes || !scales || !ids || !y) return AQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || !aligned16(ids) ||
      !aligned16(y))
    return AQ_ERR_ALIGNMENT;
  // 32-code chunks; x and the scale array addressed with 32-bit byte offsets
  if (K % 32 != 0 || K > aq::kFpMaxK || E > 65535 || T * topk > 0x7FFFFFFF ||
      T * K * 2 > 0x7FFFFFFF || E * N * (K / (mode == AQ_NVFP4 ? 16 : 32)) > 0x7FFFFFF0)
    return AQ_ERR_UNSUPPORTED;
  return from_hip(aq::launch_gather_mm_fp(x, (int)x_dtype, T, codes, scales, E, N, K, ids, topk,
                                          (int)mode, tensor_exp, y,
                                          static_cast<hipStream_t>(stream)));
}

int aq_qmv_fp_describe(int64_t N, int64_t K, aq_fp_mode mode, aq_dtype x_dtype, char *buf,
                       int len) {
  if (!valid_fp(N, K, (int)mode, 0)) return -1;
  if (K % 32 != 0 || K > aq::kFpMaxK || !valid_act_dtype(x_dtype) || !buf || len < 1) return -1;
  const char *xt = x_dtype == AQ_F16 ? "f16" : "bf16";
  const char *mt = mode == AQ_MXFP4 ? "mxfp4" : (mode == AQ_NVFP4 ? "nvfp4" : "mxfp8");
  int cpl, ud, w, wpc;
  aq::qmv1_fp_shape(N, K, (int)mode, cpl, ud, w, wpc);
  if (cpl == 0) return snprintf(buf, (size_t)len, "qmv1_fp_lds_kernel<%s, %s, W=%d>", mt, xt, w);
  return snprintf(buf, (size_t)len, "qmv1_fp_kernel<%s, %s, CPL=%d, UD=%d, W=%d>", mt, xt, cpl, ud,
                  w);
}

}  // extern "C"
