/*
 * aq.h -- C ABI of libaq: group-wise affine weight-only quantization and the
 * matmuls that consume the packed form, for AMD Instinct MI355X (gfx950).
 *
 * The format ("Quantization", metalworking MLX notes, opening paragraph and
 * "Mechanics"; "Quantizing a Model for MLX", "What MLX quantization stores"):
 * a weight matrix W [N, K] (N = out_features, K = in_features) is cut along
 * each row into groups of G = 32, 64 or 128 consecutive weights.  Each group
 * stores one fp16 scale s, one fp16 bias b and G codes q of `bits` = 2..8
 * bits, and w ~= q*s + b.  Layouts (all row-major, contiguous):
 *
 *   codes   uint32 [N, K*bits/32]  one least-significant-bit-first bitstream
 *                                  per row: code k sits at bits
 *                                  [k*bits, k*bits+bits) of the row, bit i
 *                                  of the stream being bit i%32 of word i/32
 *                                  ("Tutorial 10: Quantization", s.3, shift
 *                                  and mask extraction; for bits=3 eight
 *                                  codes fill three bytes)
 *   scales  uint16 [N, K/G]        fp16 bit patterns
 *   biases  uint16 [N, K/G]        fp16 bit patterns ("Tutorial 10", s.4
 *                                  container shapes [out, in/group_size])
 *
 * Conventions shared by every entry point:
 *  - Pointers named as device pointers must point to device memory
 *    (hipMalloc'd or torch CUDA tensors) and be 16-byte aligned, else
 *    AQ_ERR_ALIGNMENT.  The caller allocates and owns every buffer; the
 *    library only borrows them for the asynchronous operation and allocates
 *    nothing.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *    enqueued asynchronously; results are visible after the stream syncs.
 *  - Arguments are checked on the host before anything is enqueued; a bad
 *    argument returns an error and enqueues nothing.  Launch failures return
 *    AQ_ERR_HIP.  Nothing aborts and no exception crosses the ABI.
 *  - group_size in {32, 64, 128}; bits in [2, 8]; K % group_size == 0
 *    (a layer whose width is not a multiple of the group size is left
 *    unquantized: "Quantizing a Model for MLX", "What MLX quantization
 *    stores"); N, K >= 1.  No defaults: both are always explicit.
 *  - The entry points are stateless and re-entrant; calls on different
 *    streams may run concurrently.
 */
#ifndef AQ_H_
#define AQ_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum aq_status {
  AQ_OK = 0,
  AQ_ERR_INVALID_ARG = -1, /* shape, size, null pointer, dtype or enum out of range */
  AQ_ERR_UNSUPPORTED = -2, /* valid request this build does not implement */
  AQ_ERR_ALIGNMENT = -3,   /* a pointer is not 16-byte aligned */
  AQ_ERR_HIP = -4,         /* the HIP runtime reported an error at launch */
  AQ_ERR_RANGE = -5,       /* reserved: value out of the representable range */
  AQ_ERR_INDEX = -6        /* reserved: index out of range */
} aq_status;

typedef enum aq_dtype {
  AQ_F32 = 0,  /* IEEE binary32 */
  AQ_F16 = 1,  /* IEEE binary16 */
  AQ_BF16 = 2  /* bfloat16 */
} aq_dtype;

/* ---- host helpers (no GPU involved) ------------------------------------ */

/* Human-readable name of a status code (static string, never NULL). */
const char *aq_status_string(aq_status status);

/* Library version string. */
const char *aq_version(void);

/* uint32 words per packed row: K*bits/32.  -1 if K*bits is not a multiple
 * of 32 or an argument is out of range. */
int64_t aq_codes_words(int64_t K, int bits);

/* Bytes of one quantized matrix: N*K*bits/8 codes + 2 bytes of scale and
 * 2 bytes of bias per group ("Quantizing a Model for MLX", "What MLX
 * quantization stores": 4.5 bits per weight at G=64, bits=4).  -1 on bad
 * arguments. */
int64_t aq_qweight_bytes(int64_t N, int64_t K, int group_size, int bits);

/* ---- device operations -------------------------------------------------- */

/* Quantize W [N, K] (device; w_dtype AQ_F32, AQ_F16 or AQ_BF16, the latter
 * two widened exactly to binary32) into codes/scales/biases (device,
 * layouts above).  Per group, following "mlx-gptq", "How it works" (the
 * grid spans the group's min-max range) and "Quantizing a Model for MLX"
 * (scale and offset chosen per group):
 *   b = the group minimum rounded down to fp16 (so b <= every member);
 *   s = the smallest fp16 >= 0 with b + (2^bits-1)*s >= the group maximum;
 *   q = the index of the grid point b + q*s nearest to w, ties to even q
 *       (q = 0 when s = 0);
 * hence |w - (q*s + b)| <= s/2 for every weight.
 * Precondition (not checked on the device): weights finite, group minima
 * >= -65504 and the needed scale <= 65504; otherwise the outputs for that
 * group are unspecified. */
aq_status aq_quantize(const void *w, aq_dtype w_dtype, int64_t N, int64_t K, int group_size,
                      int bits, uint32_t *codes, uint16_t *scales, uint16_t *biases,
                      void *stream);

/* Range-search quantize ("mlx-gptq", "How it works": the --mse grid search
 * narrows a group's min-max range where clipping the extremes costs less
 * than the coarser step costs the rest of the group).  Same arguments,
 * outputs, format and preconditions as aq_quantize, plus steps in [1, 50]:
 * candidate i < steps narrows the group's range to [p*min, p*max] with
 * p = (100 - i)/100 (binary64), takes bias, scale and codes from it by the
 * rules of aq_quantize (members outside the narrowed range clip to code 0
 * or 2^bits-1) and scores sum (w - (q*s + b))^2 in binary64; the least
 * score wins, an equal score keeping the wider candidate.  steps = 1 gives
 * exactly aq_quantize.  (The pages fix neither the grid nor the measure;
 * these are this library's choices.)  Scores that differ only in the last
 * bits of their binary64 sums may pick either candidate.
 * AQ_ERR_INVALID_ARG for steps outside [1, 50]. */
aq_status aq_quantize_mse(const void *w, aq_dtype w_dtype, int64_t N, int64_t K, int group_size,
                          int bits, int steps, uint32_t *codes, uint16_t *scales, uint16_t *biases,
                          void *stream);

/* Dequantize ("Tutorial 10: Quantization", s.3 and s.7): out[n, k] =
 * q*s + b evaluated in binary32 (q*s is exact, the add rounds to nearest
 * even), then rounded to nearest even into out_dtype (AQ_F32, AQ_F16 or
 * AQ_BF16).  out is device memory [N, K]. */
aq_status aq_dequantize(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                        int64_t N, int64_t K, int group_size, int bits, void *out,
                        aq_dtype out_dtype, void *stream);

/* Quantized embedding lookup ("Tutorial 10: Quantization", s.6 "Quantized
 * Embeddings"): the packed rows, scales and biases of the token ids are
 * selected and dequantized exactly as aq_dequantize does:
 *   out[t, :] = dequantize(row ids[t] of the V x K table), 0 <= t < T.
 * codes/scales/biases: the table (device, layouts above, V rows).  ids:
 * device int32 [T], T >= 1.  out: device [T, K] in out_dtype (AQ_F32, AQ_F16
 * or AQ_BF16).  An id outside [0, V) reads nothing and gives a zero row. */
aq_status aq_embedding(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                       int64_t V, int64_t K, int group_size, int bits, const int32_t *ids,
                       int64_t T, void *out, aq_dtype out_dtype, void *stream);

/* Quantized matrix-vector product for decode, y = x @ W^T with W given in
 * packed form and dequantized in registers on every use ("Quantization",
 * metalworking, QMV bullet; "Tutorial 10", s.5 Approach 2 with
 * transpose=True).  x: device [M, K] in x_dtype (AQ_F16 or AQ_BF16), 1 <= M
 * <= 8.  y: device [M, N] in x_dtype.  Accumulation in binary32; y is
 * rounded to nearest even.  The kernel variant is chosen per shape (M, K,
 * bits, dtype). */
aq_status aq_qmv(const void *x, aq_dtype x_dtype, int64_t M, const uint32_t *codes,
                 const uint16_t *scales, const uint16_t *biases, int64_t N, int64_t K,
                 int group_size, int bits, void *y, void *stream);

/* Which kernel aq_qmv (and aq_quantized_matmul for M <= 8) launches for this
 * shape, as text: the kernel name and its compile-time shape (for reports and
 * profiles), written to buf (host memory, len bytes, always NUL-terminated).
 * Returns the length of the full text as snprintf does, or -1 for arguments
 * aq_qmv would reject.  For 2 <= M <= 8 it may query the current device's
 * compute-unit count. */
int aq_qmv_describe(int64_t M, int64_t N, int64_t K, int group_size, int bits, aq_dtype x_dtype,
                    char *buf, int len);

/* Quantized matrix-matrix product for prefill ("Quantization", metalworking,
 * QMM bullet): same operation and layouts as aq_qmv for any M >= 1.  Weight
 * tiles are dequantized to x_dtype (rounded to nearest even, the value
 * aq_dequantize returns for that type) and multiplied on the matrix cores
 * with binary32 accumulation.  AQ_ERR_UNSUPPORTED for K > 4194303 (a
 * 256-row tile of x is addressed with 32-bit byte offsets). */
aq_status aq_qmm(const void *x, aq_dtype x_dtype, int64_t M, const uint32_t *codes,
                 const uint16_t *scales, const uint16_t *biases, int64_t N, int64_t K,
                 int group_size, int bits, void *y, void *stream);

/* Shape dispatch for y = x @ W^T ("Quantization", metalworking: host-side
 * dispatch picks the kernel per shape): M <= 8 goes to the matrix-vector
 * kernels of aq_qmv.  For 9 <= M <= 256 with 4-bit or 8-bit codes, while
 * aq_qmm's 256 x 256 output tiles would be mostly empty or too few for the
 * chip (M <= 64, or fewer tiles than an eighth of the compute units), the
 * few-row matrix-core kernel of aq_qmv runs on slices of 16 or 32 rows of x
 * (binary32 accumulation, the same bound).  Otherwise aq_qmm.  Same arguments as aq_qmv
 * with any M >= 1; may query the current device's compute-unit count. */
aq_status aq_quantized_matmul(const void *x, aq_dtype x_dtype, int64_t M, const uint32_t *codes,
                              const uint16_t *scales, const uint16_t *biases, int64_t N,
                              int64_t K, int group_size, int bits, void *y, void *stream);

/* Gather variant for mixture-of-experts layers ("Quantization", metalworking:
 * gather variants for MoE experts): for every token t and slot j,
 *   y[t, j, :] = x[t, :] @ W_e^T   with e = ids[t, j].
 * x: device [T, K] (AQ_F16 or AQ_BF16); codes: device [E, N, K*bits/32];
 * scales, biases: device [E, N, K/G]; ids: device int32 [T, topk];
 * y: device [T, topk, N] in x_dtype.  No routing weights are applied.  Each
 * expert's weights are read once per call however many tokens chose it.
 * An id outside [0, E) is not read from; its output row is set to zero. */
aq_status aq_gather_qmv(const void *x, aq_dtype x_dtype, int64_t T, const uint32_t *codes,
                        const uint16_t *scales, const uint16_t *biases, int64_t E, int64_t N,
                        int64_t K, const int32_t *ids, int topk, int group_size, int bits,
                        void *y, void *stream);

/* The gather product at prefill size, on the matrix cores (the QMM engine
 * of aq_qmm): same operation, arguments and layouts as aq_gather_qmv, for
 * many tokens per expert.  The routing is resolved on the device: one
 * workgroup per (256 columns, expert) lists the (token, slot) pairs routed
 * to its expert and runs 256-row tiles of them, so each expert's weights are
 * read once per 256 routed rows.  Weight tiles are rounded to x_dtype as in
 * aq_qmm.  AQ_ERR_UNSUPPORTED if T*K*2 > 2^31-1 (x addressed with 32-bit
 * byte offsets), E > 65535 or T*topk > 2^31-1. */
aq_status aq_gather_qmm(const void *x, aq_dtype x_dtype, int64_t T, const uint32_t *codes,
                        const uint16_t *scales, const uint16_t *biases, int64_t E, int64_t N,
                        int64_t K, const int32_t *ids, int topk, int group_size, int bits,
                        void *y, void *stream);

/* Shape dispatch for the gather product: aq_gather_qmm when the routed rows
 * average at least 32 per expert (T*topk >= 32*E), else aq_gather_qmv. */
aq_status aq_gather_quantized_matmul(const void *x, aq_dtype x_dtype, int64_t T,
                                     const uint32_t *codes, const uint16_t *scales,
                                     const uint16_t *biases, int64_t E, int64_t N, int64_t K,
                                     const int32_t *ids, int topk, int group_size, int bits,
                                     void *y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* AQ_H_ */
