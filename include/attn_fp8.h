/*
 * attn_fp8.h - C ABI of the MI355X (gfx950) FP8 exact-attention forward pass.
 *
 * Operation: the exact attention of attn_fwd.h evaluated on 8-bit floating-point
 * inputs, with both products on the FP8 matrix cores (page "Flash Attention"
 * glossary, section "FlashAttention-3 and the FP8 era": FP8 inputs halve the
 * memory traffic again while keeping the accuracy; its hardware section on the
 * H100's FP8 and the B200's low-precision formats).
 *
 * Inputs are OCP e4m3 ("e4m3fn") codes: sign, 4 exponent bits (bias 7), 3
 * mantissa bits, subnormals, S.1111.111 = NaN, no infinities, largest finite
 * magnitude 448. Each input tensor has one fp32 dequantisation scale: the real
 * value of a code x is e4m3(x) * x_scale. For batch b, head h, query row i:
 *
 *     s_ij = scale * sum_c (e4m3(q[b,h,i,c]) q_scale) (e4m3(k[b,h,j,c]) k_scale)
 *     O[b,h,i,:] = sum_{j in J(i)} softmax_j(s_i.) * e4m3(vt[b,h,:,j]) * v_scale
 *     LSE[b,h,i] = ln( sum_{j in J(i)} exp(s_ij) )
 *
 * with J(i) all keys, or keys j <= i when causal.
 *
 * Layout: q and k dense [B][H][N][d] bytes; V is passed TRANSPOSED, vt dense
 * [B][H][d][ldv] bytes with ldv = N rounded up to a multiple of 16 (columns
 * N .. ldv-1 are never used: any byte values, NaN codes included); o dense
 * [B][H][N][d] bf16 (round to nearest even); lse dense [B][H][N] fp32. DEVICE
 * pointers; 64-bit offsets.
 *
 * Precision: the scores are exact products of e4m3 values accumulated by the
 * matrix core; the probabilities are rounded to e4m3 before the second
 * product (their row sum is taken before that rounding); O and LSE as in
 * attn_fwd.h. The achievable accuracy is set by the e4m3 rounding of the
 * probabilities (relative 2^-4), not by bf16.
 *
 * Ownership, asynchrony, errors, thread safety and determinism as in
 * attn_fwd.h: the caller owns every buffer, nothing is allocated, one kernel
 * is enqueued on `stream` (a hipStream_t, NULL = default stream) after host
 * validation, and nothing is written on a validation error.
 */
#ifndef ATTN_FP8_H
#define ATTN_FP8_H

#include "attn_fwd.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * attn_fwd_fp8 - FP8 exact attention forward.
 *   q, k       : e4m3 codes [B][H][N][d], 16-byte aligned.
 *   vt         : e4m3 codes [B][H][d][ldv], ldv = (N + 15) / 16 * 16, 16-byte aligned.
 *   o          : bf16 [B][H][N][d] output, 16-byte aligned.
 *   lse        : fp32 [B][H][N] output, 4-byte aligned.
 *   B, H, N    : >= 0; B*H*N == 0 returns ATTN_OK and launches nothing.
 *   d          : 64 or 128.
 *   causal     : nonzero for the lower-triangular mask (key j visible to query i iff j <= i).
 *   scale      : softmax scale, finite and > 0.
 *   q_scale, k_scale, v_scale : dequantisation scales, finite and > 0; the
 *                product scale * q_scale * k_scale must be a normal fp32 value.
 *   tau        : rescale threshold of the online softmax in log2 units, in
 *                [0, 8] (8 keeps the probabilities inside e4m3's range); any
 *                value gives the same result up to rounding.
 * Returns ATTN_OK; ATTN_ERR_DIM (negative or overflowing sizes),
 * ATTN_ERR_UNSUPPORTED (d, tau), ATTN_ERR_SCALE (a scale not finite or not
 * positive), ATTN_ERR_NULL, ATTN_ERR_MISALIGNED, ATTN_ERR_ALIAS (o or lse
 * overlaps an input or each other), ATTN_ERR_HIP (launch failed).
 */
attn_status_t attn_fwd_fp8(const void* q, const void* k, const void* vt, void* o, float* lse, int B, int H,
                           int N, int d, int causal, float scale, float q_scale, float k_scale,
                           float v_scale, float tau, void* stream);

/* attn_fwd_fp8 with a kernel schedule: ATTN_SCHEDULE_PIPELINED (what attn_fwd_fp8
 * runs) or ATTN_SCHEDULE_REFERENCE, a race check that loads each tile between two
 * block-wide barriers and gives bitwise the same results, several times slower.
 * Another value returns ATTN_ERR_OPTS (after the checks of attn_fwd_fp8). */
attn_status_t attn_fwd_fp8_ex(const void* q, const void* k, const void* vt, void* o, float* lse, int B, int H,
                              int N, int d, int causal, float scale, float q_scale, float k_scale,
                              float v_scale, float tau, int schedule, void* stream);

/* Host-only argument check of attn_fwd_fp8 (never touches the device). */
attn_status_t attn_fwd_fp8_check(const void* q, const void* k, const void* vt, const void* o,
                                 const float* lse, int B, int H, int N, int d, int causal, float scale,
                                 float q_scale, float k_scale, float v_scale, float tau);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FP8_H */
