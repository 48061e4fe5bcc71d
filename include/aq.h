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
 *  - Biases are optional for every consumer (dequantize, embedding and the
 *    matmuls): a NULL biases pointer means every bias is +0, i.e. w = q*s
 *    ("Tutorial 10: Quantization", s.4: biases "Optional ... or None").
 *    The results are then bit for bit those of an all-zero bias array, and
 *    no bias bytes are read.  The quantizers always write biases.
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
  AQ_ERR_INDEX = -6,       /* reserved: index out of range */
  /* range markers, never returned: they make every 32-bit integer a value of
   * the type, so any int a caller passes is well defined in C and C++ */
  AQ_STATUS_RANGE_MIN_ = -0x7FFFFFFF - 1,
  AQ_STATUS_RANGE_MAX_ = 0x7FFFFFFF
} aq_status;

typedef enum aq_dtype {
  AQ_F32 = 0,  /* IEEE binary32 */
  AQ_F16 = 1,  /* IEEE binary16 */
  AQ_BF16 = 2, /* bfloat16 */
  /* range markers, never valid arguments (AQ_ERR_INVALID_ARG): every 32-bit
   * integer is a value of the type, so validating one is well defined */
  AQ_DTYPE_RANGE_MIN_ = -0x7FFFFFFF - 1,
  AQ_DTYPE_RANGE_MAX_ = 0x7FFFFFFF
} aq_dtype;

/* ---- host helpers (no GPU involved) ------------------------------------ */

/* Human-readable name of a status code (static string, never NULL). */
const char *aq_status_string(aq_status status);

/* Library version string. */
const char *aq_version(void);

/* uint32 words per packed row: K*bits/32 (one least-significant-bit-first
 * bitstream per row, several codes to a 32-bit word: "Quantizing a Model for
 * MLX", "What MLX quantization stores"; "Tutorial 10: Quantization", s.3 and
 * s.4, packed weight shape [out, in*bits/32]).  -1 if K*bits is not a
 * multiple of 32 or an argument is out of range. */
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

/* Range-search quantize ("mlx-gptq", "How it works", the --mse option: a
 * group may be quantized over a range narrower than its min-max span,
 * trading error on its outermost members for a finer step on the others).
 * Same arguments, outputs, format and preconditions as aq_quantize, plus
 * steps in [1, 50]: candidate i < steps moves both ends of the group's range
 * inwards by d = (max - min) * (i / 200) (binary64, left to right), i.e.
 * keeps the centred fraction (100 - i)/100 of the width, so every candidate
 * lies inside [min, max]; it takes bias, scale and codes from that range by
 * the rules of aq_quantize (members outside it clip to code 0 or 2^bits-1)
 * and scores sum (w - (q*s + b))^2 in binary64; the least score wins, an
 * equal score keeping the wider candidate.  steps = 1 gives
 * exactly aq_quantize.  (The pages fix neither the grid nor the measure;
 * these are this library's choices.)  Scores that differ only in the last
 * bits of their binary64 sums may pick either candidate.
 * AQ_ERR_INVALID_ARG for steps outside [1, 50]. */
aq_status aq_quantize_mse(const void *w, aq_dtype w_dtype, int64_t N, int64_t K, int group_size,
                          int bits, int steps, uint32_t *codes, uint16_t *scales, uint16_t *biases,
                          void *stream);

/* Quantize with integer zero points ("mlx-gptq", "On NVIDIA: the same recipe
 * in AWQ format", --zero-point int: every group's offset is a whole number of
 * steps, so the result converts without loss to a layout that stores an
 * integer zero point z per group and decodes (q - z)*s).  Same arguments,
 * outputs, format and preconditions as aq_quantize, plus zeros: device uint8
 * [N, K/G] receiving each group's z, or NULL.  Per group:
 *   z is an integer in [0, 2^bits - 1], so the grid -z*s + q*s contains 0;
 *   s = the smallest fp16 >= 0 for which some such z has -z*s <= the group
 *       minimum, (2^bits-1-z)*s >= the group maximum and -z*s exactly an
 *       fp16 value; z = the smallest such integer for that s;
 *   b = -z*s (exact; +0 when z = 0), q as in aq_quantize;
 * hence q*s + b = (q - z)*s exactly and |w - (q*s + b)| <= s/2.  The output
 * is an ordinary (codes, scales, biases) container: every consumer below
 * takes it unchanged. */
aq_status aq_quantize_zp(const void *w, aq_dtype w_dtype, int64_t N, int64_t K, int group_size,
                         int bits, uint32_t *codes, uint16_t *scales, uint16_t *biases,
                         uint8_t *zeros, void *stream);

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
 * 256-row tile of x is addressed with 32-bit byte offsets) or M > 8388352
 * (the launch grid holds at most 65535 row tiles of 128). */
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
 * y: device [T, topk, N] in x_dtype.  No routing weights are applied.  The
 * routing is resolved on the device: each expert's weights are read once
 * for every batch of up to 16 (token, slot) pairs routed to it (8 on the
 * vector path for 2-, 3-, 5-, 6- and 7-bit codes), and experts no token
 * chose are never read.  An id outside [0, E) is not read from; its output
 * row is set to zero. */
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

/* ---- block-scaled float modes ------------------------------------------- */

/* The block-scaled float modes ("Quantization", metalworking MLX notes, the
 * paragraph on the newer modes; "Quantizing a Model for MLX", "Modes, bits
 * and mixed recipes": mxfp4, nvfp4 and mxfp8 with groups of 32, 16 and 32
 * weights and 4, 4 and 8-bit codes, a per-group scale in place of a scale
 * and a bias; ExecuTorch "Quantization": nvfp4 is NVIDIA's FP4 weight-only
 * format at group size 16).  The pages give no bit layout; this library
 * takes the definitions of those names (microscaling for mxfp4 and mxfp8,
 * NVFP4 for nvfp4):
 *
 *   E2M1 code (4 bits): bit 3 sign, bits 2..1 exponent e (bias 1), bit 0
 *     mantissa m; (1 + m/2)*2^(e-1), or m/2 for e = 0 (magnitudes 0, 0.5,
 *     1, 1.5, 2, 3, 4, 6).
 *   E4M3 code (8 bits): bit 7 sign, bits 6..3 exponent e (bias 7), bits
 *     2..0 mantissa m; (1 + m/8)*2^(e-7), or (m/8)*2^-6 for e = 0;
 *     magnitude pattern 0x7F is NaN; largest finite magnitude 448.
 *
 *   mode      group  codes                         scales
 *   AQ_MXFP4   32    uint32 [N, K/8]  E2M1         uint8 [N, K/32]  X + 127 for 2^X
 *   AQ_NVFP4   16    uint32 [N, K/8]  E2M1         uint8 [N, K/16]  E4M3 value s
 *   AQ_MXFP8   32    uint32 [N, K/4]  E4M3         uint8 [N, K/32]  X + 127 for 2^X
 *
 * Codes are packed least significant first into the row's words (code k of
 * a row at bits [b*k, b*k + b) of its bitstream, as above).  A weight's
 * value is code * 2^X (mx modes) or code * s * 2^T (nvfp4, where the whole
 * matrix shares the tensor scale 2^T, the argument tensor_exp = T in
 * [-100, 100]; 0 means no tensor scale; for the mx modes tensor_exp must
 * be 0).  N >= 1, K >= the group size and a multiple of it.  The
 * conventions above (device pointers 16-byte aligned, caller-owned buffers,
 * host-side checks, asynchronous on `stream`) hold. */
typedef enum aq_fp_mode {
  AQ_MXFP4 = 0,
  AQ_NVFP4 = 1,
  AQ_MXFP8 = 2,
  /* range markers, never valid arguments (AQ_ERR_INVALID_ARG) */
  AQ_FP_MODE_RANGE_MIN_ = -0x7FFFFFFF - 1,
  AQ_FP_MODE_RANGE_MAX_ = 0x7FFFFFFF
} aq_fp_mode;

/* Quantize W [N, K] (device; AQ_F32, AQ_F16 or AQ_BF16, widened exactly to
 * binary32) into codes and scales (device) of the given mode.  Per group:
 *   mxfp4, mxfp8: X = floor(log2 max|w|) - E, E the exponent of the
 *     largest code value (2 for E2M1's 6, 8 for E4M3's 448), clamped to
 *     [-127, 127]; -127 for a group of zeros.  The step is 2^X.
 *   nvfp4: s = the E4M3 value nearest to max|w| / (6 * 2^T), ties to the
 *     even code, 448 above it.  The step is s * 2^T.
 *   each weight's code is its own sign bit (so -0 keeps it) with the
 *   magnitude code nearest to |w| / step, ties to the even code, the
 *   largest finite magnitude above it; magnitude 0 when s = 0.
 * A tensor exponent that puts the largest group scale near the top of
 * E4M3's range is T = ceil(log2(max|W| / 2688)) (2688 = 6 * 448).
 * Precondition (not checked on the device): weights finite; otherwise the
 * outputs for that group are unspecified. */
aq_status aq_quantize_fp(const void *w, aq_dtype w_dtype, int64_t N, int64_t K, aq_fp_mode mode,
                         int tensor_exp, uint32_t *codes, uint8_t *scales, void *stream);

/* Dequantize: out[n, k] = the exact value code * step (NaN for NaN code or
 * scale patterns; steps from any scale byte, not only those the quantizer
 * writes), rounded to nearest even into out_dtype (AQ_F32, AQ_F16 or
 * AQ_BF16), +-inf past its range.  out is device memory [N, K]. */
aq_status aq_dequantize_fp(const uint32_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                           aq_fp_mode mode, int tensor_exp, void *out, aq_dtype out_dtype,
                           void *stream);

/* Decode matrix-vector product ("Quantization", metalworking, QMV bullet:
 * the weights are dequantized in registers on every use): y[n] =
 * sum_k x[k] * w^[n, k] for one row x.  x: device [K] in x_dtype (AQ_F16 or
 * AQ_BF16); y: device [N] in x_dtype.  Products are summed in binary32 per
 * group and scaled once per group; y is rounded to nearest even.
 * AQ_ERR_UNSUPPORTED for K not a multiple of 32 (nvfp4) or K > 49152 (x is
 * held on chip). */
aq_status aq_qmv_fp(const void *x, aq_dtype x_dtype, const uint32_t *codes,
                    const uint8_t *scales, int64_t N, int64_t K, aq_fp_mode mode, int tensor_exp,
                    void *y, void *stream);

/* The product for M rows of x ("Quantization", metalworking, QMV bullet and
 * its dispatch section on several rows of x per pass over W, as in
 * speculative decoding): y[m, n] = sum_k x[m, k] * w^[n, k].  x: device
 * [M, K] row-major in x_dtype (AQ_F16 or AQ_BF16); y: device [M, N] in
 * x_dtype.  M = 1 is aq_qmv_fp.  M >= 2 runs on the matrix cores in slices
 * of 16 rows of x, each slice one pass over W: per 32-code chunk the exact
 * code values times x, summed in binary32 per group and scaled once per
 * group (nvfp4: 2^T applied to the sums); y is rounded to nearest even.
 * Arguments as aq_qmv_fp (the same K limits; AQ_ERR_INVALID_ARG for
 * M < 1, AQ_ERR_UNSUPPORTED past M = 16 * 65535 or past 2^31 - 16 scale
 * bytes). */
aq_status aq_matmul_fp(const void *x, aq_dtype x_dtype, int64_t M, const uint32_t *codes,
                       const uint8_t *scales, int64_t N, int64_t K, aq_fp_mode mode,
                       int tensor_exp, void *y, void *stream);

/* Mixture-of-experts gather of the block-scaled product ("Quantization",
 * metalworking: gather variants of the kernels for MoE experts):
 * y[t, j, :] = x[t] @ W_{ids[t, j]}^T for every token t < T and slot
 * j < topk, one output row per (token, slot), no routing weights.  x: device
 * [T, K] in x_dtype (AQ_F16 or AQ_BF16); codes and scales: device, E
 * experts' arrays of aq_quantize_fp back to back ([E, N, ...]); ids: device
 * int32 [T, topk]; y: device [T, topk, N] in x_dtype.  An id outside
 * [0, E) gives a zero row and reads no weights; experts no pair chose are
 * never read.  Each expert's rows are read once per batch of 16 (token,
 * slot) pairs routed to it, on the matrix cores as in aq_matmul_fp (the
 * same sums, the same rounding).  AQ_ERR_INVALID_ARG for T, E or topk
 * below 1 or a bad mode, tensor exponent or pointer; AQ_ERR_UNSUPPORTED for
 * K not a multiple of 32 or past 49152, E > 65535, or x or the scale array
 * past 2^31 bytes. */
aq_status aq_gather_matmul_fp(const void *x, aq_dtype x_dtype, int64_t T, const uint32_t *codes,
                              const uint8_t *scales, int64_t E, int64_t N, int64_t K,
                              const int32_t *ids, int topk, aq_fp_mode mode, int tensor_exp,
                              void *y, void *stream);

/* Which kernel aq_qmv_fp launches for this shape and mode, as text (as
 * aq_qmv_describe does); -1 for arguments aq_qmv_fp would reject. */
int aq_qmv_fp_describe(int64_t N, int64_t K, aq_fp_mode mode, aq_dtype x_dtype, char *buf,
                       int len);

#ifdef __cplusplus
}
#endif

#endif /* AQ_H_ */
