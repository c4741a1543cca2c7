/*
 * aaq.h -- C ABI of the token-wise adaptive activation quantization (AAQ)
 * codec in libtriattn.so, for the pair representation Z on MI355X (gfx950).
 *
 * What is computed (LightNobel article, section 2.2 "adaptive activation
 * quantization"; record layout after section 2.3.2, token-interleaved storage):
 *  - Each token -- one 128-channel vector of Z -- is quantized on its own with
 *    its own scale and zero point (section 2.2.1).
 *  - Groups A and B handle outliers (section 2.2.2): the 5 channels of largest
 *    |x| (equal magnitudes: the lower channel first) are candidates; a
 *    candidate is confirmed when |x - mu| > 3 sigma, mu and sigma being the
 *    mean and the population standard deviation of the token's 128 values,
 *    all in float64 (sigma = sqrt of the two-pass variance).  Confirmed outliers are
 *    stored as INT16 with a scale of their own: s_o = max|x_o| / 32767,
 *    q_o = clamp(rint(x / s_o), -32767, 32767).
 *  - The other values (inliers) are quantized affinely (section 2.2.3: group A
 *    INT8, groups B and C INT4; group C has no outlier handling) over their
 *    range widened to contain 0:  s = (rmax - rmin) / qmax, z = rint(-rmin / s),
 *    q = clamp(rint(x / s) + z, 0, qmax).  A token whose inliers are all zero
 *    gets s = 0, z = 0.  Every step that makes a code is float32: s is a
 *    float32 quotient, 1/s its float32 reciprocal, x / s is evaluated as
 *    x * (1/s), rounding is to nearest even.
 *  - Decoding is s (q - z) for inliers and s_o q_o for outliers, in float32,
 *    then rounded (nearest even) to the output dtype.
 *
 * Record layout (little endian), record t of n at records + t * aaq_record_bytes(group):
 *   group A, 160 B: u8 code[128] (channel c at byte c) | meta (32 B)
 *   group B,  96 B: u4 code[128] (byte j: channel 2j low nibble, 2j+1 high) | meta
 *   group C,  80 B: u4 code[128] | f32 s | u8 z | 11 zero bytes
 *   meta: f32 s | f32 s_o | i16 q_o[5] | u8 channel[5] | u8 z | u8 n | 7 zero bytes
 *   Outlier slots are in ascending channel order; unused slots are zero;
 *   s_o = 0 when n = 0.  An outlier's channel holds the code z.
 *
 * Conventions
 *  - x, y and records are DEVICE pointers, 16-byte aligned; tokens are dense
 *    rows of 128 channels (x: [n][128]), records are back to back.  Any
 *    tensor of shape [..., 128] in C order is n = numel / 128 tokens.
 *  - dtype is TA_BF16 or TA_F32 (include/triattn.h).  Values must be finite.
 *  - The caller owns every buffer.  The library never allocates, frees or
 *    synchronises; it validates every argument on the host (nothing is
 *    enqueued on error, return codes as in include/triattn.h) and enqueues
 *    one kernel on `stream` (a hipStream_t; NULL = the default stream).
 *  - n = 0 is valid and enqueues nothing.
 */
#ifndef AAQ_H
#define AAQ_H

#include <stdint.h>

#include "triattn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Groups (LightNobel article, section 2.2.3). */
enum {
  AAQ_GROUP_A = 0, /* residual-path activations: INT8 inliers + INT16 outliers */
  AAQ_GROUP_B = 1, /* LayerNorm outputs feeding a linear layer: INT4 + INT16 outliers */
  AAQ_GROUP_C = 2  /* all other activations: INT4, no outlier handling */
};

#define AAQ_CHANNELS 128
#define AAQ_TOP_K 5

/* Bytes of one record of `group` (160, 96, 80), or TA_ERR_BAD_GROUP. */
int aaq_record_bytes(int group);

/* Encode n tokens x [n][128] (dtype TA_BF16 / TA_F32) into n records.
 * Errors: TA_ERR_NULL_PTR (x or records NULL with n > 0), TA_ERR_BAD_SHAPE
 * (n < 0 or n > 2^40), TA_ERR_BAD_DTYPE, TA_ERR_BAD_GROUP, TA_ERR_MISALIGNED,
 * TA_ERR_ALIAS (records overlap x), TA_ERR_HIP (launch rejected). */
int aaq_encode(const void* x, int dtype, int64_t n, int group, void* records, void* stream);

/* Decode n records of `group` into y [n][128] (dtype TA_BF16 / TA_F32).
 * Records must be what aaq_encode (or an equivalent encoder) wrote: n above 5
 * is read as 5, a channel above 127 matches no channel.
 * Errors as for aaq_encode (TA_ERR_ALIAS: y overlaps records). */
int aaq_decode(const void* records, int group, int64_t n, void* y, int dtype, void* stream);

/* Stage 1 of triangle attention (as triangle_attn_project, include/triattn.h)
 * reading the pair tensor as token-wise quantized records instead of bf16
 * tokens: the pair tensor is on the residual path, the activations the
 * LightNobel article (section 2.2.3) keeps in group A.  Each token is decoded
 * in registers -- s (q - z), outliers s_o q_o, in fp32 exactly as aaq_decode
 * computes them -- and LayerNorm and the projections run on those fp32 values.
 *   prob     as for triangle_attn_project; dtype must be TA_BF16 (bf16 weights
 *            and workspace)
 *   records  [rows][I] records of `group` (A, B or C), token (i, j) at
 *            records + (i * I + j) * aaq_record_bytes(group); for TA_END the
 *            ending-node lines are the columns of this array, as for z
 *   ws       the workspace of triangle_attn_project; triangle_attn_attend then
 *            runs on it unchanged
 * Errors as for triangle_attn_project, plus TA_ERR_BAD_DTYPE (not bf16) and
 * TA_ERR_BAD_GROUP. */
int triangle_attn_project_aaq(const ta_problem* prob, int variant, const ta_weights* w,
                              const void* records, int group, void* ws, size_t ws_bytes,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AAQ_H */
