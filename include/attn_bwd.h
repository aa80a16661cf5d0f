/*
 * attn_bwd.h - C ABI of the MI355X (gfx950) exact-attention backward pass.
 *
 * Operation: the gradients of the exact attention of attn_fwd.h with respect
 * to q, k and v, given dO, the gradient arriving at its output O. The
 * attention probabilities are recomputed on chip from q, k and the forward
 * pass's log-sum-exp instead of being stored (page "Flash Attention" glossary,
 * section "Online softmax and recomputation"); the gradients are formed
 * without atomic additions (page "FlashAttention-4: algorithm-kernel fused
 * pipeline for asymmetric hardware scaling", section 2, on the costs of the
 * backward pass). For batch b, query head h (key/value head g = h / (H/Hkv)),
 * with P_ij = exp(scale * q_i . k_j - LSE_i) over the visible keys (0 otherwise):
 *
 *     dV[g] = sum over h in g of P^T dO          dP = dO V^T
 *     D_i   = dO_i . O_i                          dS = P * (dP - D)
 *     dQ    = scale * dS K                        dK[g] = sum over h in g of scale * dS^T Q
 *
 * Layout as in attn_fwd.h: q, o, dout, dq dense [B][H][N][d] bf16; k, v, dk,
 * dv [B][Hkv][N][d] bf16; lse and delta [B][H][N] fp32. All DEVICE pointers.
 * o and lse are the forward pass's outputs for the same q, k, v, causal flag
 * and scale (any attn_fwd* entry point with bf16 O).
 *
 * Ownership: the caller owns every buffer; the library allocates nothing.
 * delta is an output: D_i per query row (fp32), produced on the way and
 * returned like dq. Every output is written in full (no accumulation into
 * the caller's buffers).
 *
 * Asynchrony and errors as in attn_fwd.h: arguments are validated on the
 * host; on success two kernels are enqueued on `stream` (dq, then dk/dv,
 * which reads delta) and the call returns without synchronising.
 */
#ifndef ATTN_BWD_H
#define ATTN_BWD_H

#include "attn_fwd.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * attn_bwd - exact attention backward.
 *   q, k, v, o, lse, dout : inputs as above (16-byte aligned; lse 4-byte).
 *   dq, dk, dv            : bf16 outputs (16-byte aligned), fp32 accumulation,
 *                           round-to-nearest-even on store.
 *   delta                 : fp32 [B][H][N] output (4-byte aligned).
 *   B, H, Hkv, N, d, causal, scale : as for attn_fwd_gqa (Hkv = H for
 *                           multi-head attention). B*H*N == 0 returns ATTN_OK
 *                           and launches nothing.
 * Returns ATTN_OK; ATTN_ERR_DIM, _UNSUPPORTED, _SCALE, _NULL, _MISALIGNED as
 * for the forward pass; ATTN_ERR_ALIAS if an output overlaps an input or
 * another output; ATTN_ERR_HIP if a launch fails.
 */
attn_status_t attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H,
                       int Hkv, int N, int d, int causal, float scale, void* stream);

/*
 * attn_bwd_ex - attn_bwd with a kernel schedule (ABI 10).
 *   schedule : ATTN_SCHEDULE_PIPELINED (what attn_bwd runs) or
 *              ATTN_SCHEDULE_REFERENCE, a race check for d = 128: dK and dV come
 *              from the one-wavefront dk/dv kernel, which keeps both accumulators
 *              and P in one lane, instead of the wavefront pairs that pass P
 *              through LDS between two wavefronts. Both accumulate every product
 *              in the same order, so dk and dv must be equal bit for bit; dq and
 *              delta come from the same kernel either way. At d = 64 both
 *              schedules run the one-wavefront kernel.
 * Same arguments and error codes as attn_bwd; ATTN_ERR_OPTS for another schedule
 * value.
 */
attn_status_t attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H,
                          int Hkv, int N, int d, int causal, float scale, int schedule, void* stream);

/*
 * attn_bwd_varlen - backward of packed variable-length attention (the layout of
 * attn_fwd_varlen in attn_fwd.h: several sequences folded into the token axis).
 *   q, o, dout, dq : bf16 [H][total][d]; k, v, dk, dv : bf16 [Hkv][total][d];
 *   lse, delta     : fp32 [H][total]; o and lse from attn_fwd_varlen with the same
 *                    cu_seqlens, causal flag and scale.
 *   cu_seqlens     : DEVICE int32 [B+1] cumulative lengths (cu[0] = 0, cu[B] =
 *                    total, non-decreasing), 4-byte aligned. Not validated (that
 *                    would need a synchronisation): the kernels clamp every bound
 *                    into [0, total], so no contents take an access outside the
 *                    tensors; the results of an ill-formed array are undefined.
 *   max_seqlen     : host int >= the longest sequence; it sizes the launch. Rows
 *                    past ceil(max_seqlen / 128) * 128 of a longer sequence are
 *                    not written.
 * Each sequence is the backward pass of attn_bwd on its own rows and keys (the
 * causal mask counts positions from the sequence's first token); dk and dv of a
 * shared key/value head are summed over its query heads. Same error codes as
 * attn_bwd (ATTN_ERR_NULL also for cu_seqlens; ATTN_ERR_DIM for negative
 * max_seqlen or total); B*H*min(max_seqlen, total) == 0 returns ATTN_OK and
 * launches nothing.
 */
attn_status_t attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              float* delta, const int* cu_seqlens, int B, int H, int Hkv, int total,
                              int max_seqlen, int d, int causal, float scale, void* stream);

/* Host-only argument check of attn_bwd_varlen (never touches the device). */
attn_status_t attn_bwd_varlen_check(const void* q, const void* k, const void* v, const void* o,
                                    const float* lse, const void* dout, const void* dq,
                                    const void* dk, const void* dv, const float* delta,
                                    const int* cu_seqlens, int B, int H, int Hkv, int total,
                                    int max_seqlen, int d, int causal, float scale);

/* Host-only argument check of attn_bwd (never touches the device). */
attn_status_t attn_bwd_check(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, const void* dq, const void* dk,
                             const void* dv, const float* delta, int B, int H, int Hkv, int N,
                             int d, int causal, float scale);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_BWD_H */
