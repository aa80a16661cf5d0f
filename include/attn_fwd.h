/*
 * attn_fwd.h - C ABI of the MI355X (gfx950) exact-attention forward library.
 *
 * Operation: exact scaled-dot-product attention. Queries are multiplied with
 * the keys, the scores are normalised by a softmax and the result multiplies
 * the values (page "FlashAttention 4: faster, more memory-efficient attention
 * for LLMs", section "Introduction"). The result equals standard attention up
 * to floating-point rounding; it is not an approximation (page "Flash
 * Attention" glossary, section "Summary of optimisations"). It is computed
 * tile by tile with a running maximum and running sum per query row, so the
 * N x N score matrix never reaches device memory (same glossary page, sections
 * "Tiling with SRAM" and "Online softmax and recomputation").
 *
 * For every batch b, head h and query row i (0-based), with J(i) the visible
 * keys (all keys; or keys j <= i when causal):
 *
 *     s_ij   = scale * sum_c q[b,h,i,c] * k[b,h,j,c]
 *     O[b,h,i,:] = sum_{j in J(i)} softmax_j(s_i.) * v[b,h,j,:]
 *     LSE[b,h,i] = ln( sum_{j in J(i)} exp(s_ij) )          (natural log, fp32)
 *
 * Layout: q, k, v and o are dense row-major [B][H][N][d] tensors (d innermost,
 * no strides, no padding); lse is dense [B][H][N]. All tensor pointers are
 * DEVICE pointers. Offsets are computed in 64-bit.
 *
 * Ownership: the caller allocates and owns every buffer. The library never
 * allocates, frees or keeps device memory, uses no workspace and keeps no
 * state between calls; memory use is linear in N (the O(N) property named on
 * the glossary page, "Summary of optimisations").
 *
 * Asynchrony: every call validates its arguments on the host, then enqueues
 * one kernel on `stream` (a hipStream_t; NULL = the default stream) and
 * returns without synchronising. On a validation error nothing is launched
 * and nothing is written. Device faults surface at the caller's next
 * synchronisation. Calls are reentrant and thread-safe. Results are bitwise
 * reproducible for identical inputs and options.
 */
#ifndef ATTN_FWD_H
#define ATTN_FWD_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 1: attn_fwd, attn_fwd_ex, attn_fwd_check and helpers.
 * 2: adds attn_fwd_gqa and attn_fwd_gqa_check (grouped-query attention).
 * 3: adds attn_fwd_varlen and attn_fwd_varlen_check (packed variable-length batches).
 * 4: adds attn_bwd and attn_bwd_check (backward pass, declared in attn_bwd.h).
 * 5: adds attn_fwd_splitkv and attn_fwd_splitkv_workspace_size (split keys).
 * 6: adds attn_fwd_fp8 and attn_fwd_fp8_check (FP8 e4m3 inputs, declared in attn_fp8.h).
 * 7: adds attn_bwd_varlen and attn_bwd_varlen_check (declared in attn_bwd.h).
 * 8: adds attn_fwd_splitkv_noalloc.
 * 9: adds the schedule option (attn_fwd_opts.schedule) and attn_fwd_fp8_ex.
 * 10: adds attn_bwd_ex (the backward pass with a schedule, declared in attn_bwd.h). */
#define ATTN_ABI_VERSION 10

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL (with B*H*N > 0) */
  ATTN_ERR_DIM = 2,         /* B, H or N negative, Hkv not a divisor of H, or sizes overflow */
  ATTN_ERR_UNSUPPORTED = 3, /* d not in {64, 128}, or an unknown option value */
  ATTN_ERR_MISALIGNED = 4,  /* q, k, v, o not 16-byte aligned, or lse not 4-byte aligned */
  ATTN_ERR_SCALE = 5,       /* scale is not finite */
  ATTN_ERR_ALIAS = 6,       /* o or lse overlaps an input, or o overlaps lse */
  ATTN_ERR_HIP = 7,         /* the kernel launch failed; details in attn_last_error() */
  ATTN_ERR_OPTS = 8         /* opts->struct_size too small, tau out of [0, 64], or an unknown schedule */
} attn_status_t;

/* Output element type of o. */
enum { ATTN_O_BF16 = 0, ATTN_O_F32 = 1 };

/* Kernel schedule: the production ping-pong pipeline, or a reference schedule
 * that computes the same tiles in the same arithmetic order with every load
 * fenced by a block-wide barrier before its first use (no tile is in flight
 * while another is read). The two give bitwise-identical results; a difference
 * shows a synchronisation error in the pipeline. */
enum { ATTN_SCHEDULE_PIPELINED = 0, ATTN_SCHEDULE_REFERENCE = 1 };

/*
 * Options for attn_fwd_ex. Initialise with attn_fwd_opts_init, then set fields.
 *
 * rescale_tau_log2: threshold of the adaptive online rescale (page "FlashAttention
 *   4: faster, more memory-efficient attention for LLMs", section "Smarter online
 *   softmax rescaling (new in FA4)"): the stored row maximum and the partial
 *   results are only rescaled when a tile's maximum exceeds the maximum in use by
 *   more than tau, measured in log2 units of the scaled scores. 0 = classic
 *   policy (rescale on every increase). Default 8. Range [0, 64]. Any value gives
 *   the same result up to rounding.
 * exp2_poly_eighths: how many of every 8 score columns take 2^x from a cubic
 *   polynomial on the vector ALU instead of the hardware exp2 instruction (page
 *   "FlashAttention 4: faster, more memory-efficient attention for LLMs", section
 *   "Software exponential on CUDA cores"). 0..8; supported values are 0, 4 and 8
 *   (others return ATTN_ERR_UNSUPPORTED). Default 0.
 * o_dtype: ATTN_O_BF16 (default; fp32 accumulate, round-to-nearest-even on
 *   store) or ATTN_O_F32.
 * rescale_count: optional DEVICE pointer to int32 [B][H][N]; when not NULL the
 *   kernel stores, per query row, the number of rescales after the row's first
 *   tile (instrumentation; not part of the result). Must not overlap any tensor.
 * schedule: ATTN_SCHEDULE_PIPELINED (default) or ATTN_SCHEDULE_REFERENCE (a race
 *   check, several times slower; needs exp2_poly_eighths 0 and scale >= 0, else
 *   ATTN_ERR_UNSUPPORTED; other values: ATTN_ERR_OPTS). Callers built against
 *   ABI 8, whose struct ends before this field, pass the shorter struct_size and
 *   get the default.
 */
typedef struct attn_fwd_opts {
  size_t struct_size; /* sizeof(attn_fwd_opts) */
  float rescale_tau_log2;
  int exp2_poly_eighths;
  int o_dtype;
  int* rescale_count;
  int schedule;
} attn_fwd_opts;

/* Fill *opts with the defaults (struct_size set, tau 8, no polynomial, bf16 O,
 * pipelined schedule). */
void attn_fwd_opts_init(attn_fwd_opts* opts);

/*
 * attn_fwd - exact attention forward with default options.
 *   q, k, v : const bf16 [B][H][N][d], device, 16-byte aligned, read only.
 *   o       : bf16 [B][H][N][d], device, 16-byte aligned, written.
 *   lse     : float [B][H][N], device, 4-byte aligned, written (natural-log LSE).
 *   B, H, N : >= 0; if any is 0 the call returns ATTN_OK and does nothing
 *             (pointers may then be NULL). B*H*ceil(N/128) must fit in int32 and
 *             (N + 256) * d * 2 must be below 2^31 (one head is addressed with
 *             32-bit byte offsets), else ATTN_ERR_DIM.
 *   d       : 64 or 128.
 *   causal  : 0 = all keys visible; nonzero = key j visible to query i iff j <= i.
 *   scale   : any finite float (0 gives uniform weights; negative is allowed).
 *   stream  : hipStream_t to enqueue on (NULL = default stream).
 * Returns ATTN_OK or an error code; on error nothing is launched.
 */
attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int N, int d, int causal, float scale, void* stream);

/* attn_fwd with options (NULL opts = defaults). Same argument contract. */
attn_status_t attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int N, int d, int causal, float scale,
                          const attn_fwd_opts* opts, void* stream);

/* Host-only argument check used by both entry points: returns the status that
 * attn_fwd_ex would return before launching (never touches the device). */
attn_status_t attn_fwd_check(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, int B, int H, int N, int d, int causal,
                             float scale, const attn_fwd_opts* opts);

/*
 * attn_fwd_gqa - grouped-query (and multi-query) attention forward: several
 * query heads share one key/value head (page "FlashAttention 4: faster, more
 * memory-efficient attention for LLMs", sections "Key points" and
 * "Compatibility and current status", which list GQA/MQA among the
 * configurations of earlier FlashAttention versions).
 *   q       : const bf16 [B][H][N][d], device, 16-byte aligned.
 *   k, v    : const bf16 [B][Hkv][N][d], device, 16-byte aligned.
 *   o, lse  : as for attn_fwd ([B][H][N][d] and [B][H][N]).
 *   Hkv     : key/value heads, 1 <= Hkv <= H and H % Hkv == 0 (0 when H == 0),
 *             else ATTN_ERR_DIM. Query head h reads key/value head
 *             h / (H / Hkv) (consecutive groups of H / Hkv query heads):
 *
 *     s_ij = scale * sum_c q[b,h,i,c] * k[b, h/(H/Hkv), j, c]   (v likewise)
 *
 *             Hkv = 1 is multi-query attention; Hkv = H is attn_fwd_ex,
 *             bit for bit.
 * Every other argument, the error behaviour and the asynchrony are those of
 * attn_fwd_ex. The kernel and the tile walk are the same; the query heads of
 * one group run next to each other, so their shared K and V tiles are
 * fetched from HBM about once per group.
 */
attn_status_t attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Hkv, int N, int d, int causal, float scale,
                           const attn_fwd_opts* opts, void* stream);

/* Host-only argument check of attn_fwd_gqa (never touches the device). */
attn_status_t attn_fwd_gqa_check(const void* q, const void* k, const void* v, const void* o,
                                 const float* lse, int B, int H, int Hkv, int N, int d,
                                 int causal, float scale, const attn_fwd_opts* opts);

/*
 * attn_fwd_varlen - attention over a packed batch of sequences of different
 * lengths (page "FlashAttention 4: faster, more memory-efficient attention for
 * LLMs", section "Key points", which lists variable-length batches among the
 * features earlier FlashAttention versions had and FA4 lacked). Each sequence
 * attends only to itself; query and key/value sequences share the same bounds
 * (self-attention), and the causal mask counts positions from the sequence's
 * first token. Grouped-query heads as for attn_fwd_gqa.
 *   q, o       : bf16 [H][total][d] (o: float [H][total][d] with ATTN_O_F32),
 *                device, 16-byte aligned: the dense layout with the batch
 *                folded into the token axis.
 *   k, v       : const bf16 [Hkv][total][d], device, 16-byte aligned.
 *   lse        : float [H][total], device, 4-byte aligned.
 *   cu_seqlens : const int32 [B + 1], DEVICE, 4-byte aligned: cumulative
 *                lengths, cu[0] = 0, non-decreasing, cu[B] = total; sequence b
 *                is tokens cu[b] .. cu[b+1]-1 of every head. Empty sequences
 *                are allowed. The host cannot read it without synchronising,
 *                so its contents are not validated: the kernel clamps every
 *                bound into [0, total] (no access leaves the tensors whatever
 *                it holds), but rows of an ill-formed array are not defined.
 *   B          : number of sequences (>= 0).
 *   total      : tokens per head (>= 0); (total + 256) * d * 2 < 2^31.
 *   max_seqlen : >= the longest sequence (values above total are treated as
 *                total); it sizes the launch. Rows of a sequence longer than
 *                max_seqlen rounded up to a multiple of 256 are not written.
 *   rescale_count option: int32 [H][total].
 * B, H, total or max_seqlen of 0 return ATTN_OK and launch nothing. Other
 * arguments, errors (cu_seqlens NULL: ATTN_ERR_NULL; outputs overlapping
 * cu_seqlens: ATTN_ERR_ALIAS) and asynchrony as for attn_fwd_ex.
 */
attn_status_t attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                              const int* cu_seqlens, int B, int H, int Hkv, int total,
                              int max_seqlen, int d, int causal, float scale,
                              const attn_fwd_opts* opts, void* stream);

/* Host-only argument check of attn_fwd_varlen (never touches the device, so it
 * does not read cu_seqlens). */
attn_status_t attn_fwd_varlen_check(const void* q, const void* k, const void* v, const void* o,
                                    const float* lse, const int* cu_seqlens, int B, int H,
                                    int Hkv, int total, int max_seqlen, int d, int causal,
                                    float scale, const attn_fwd_opts* opts);

/*
 * attn_fwd_splitkv - attn_fwd_gqa with the keys of every query tile split into
 * n_splits ranges computed by separate workgroups, for shapes with too few
 * query tiles to occupy the GPU and for very long sequences (page "Flash
 * Attention" glossary, overview section and its list of benefits, on contexts of
 * 128k and 1M tokens; page "FlashAttention 4: faster, more memory-efficient
 * attention for LLMs", section "Conclusion", on forward throughput at long
 * sequence lengths). Unit s of a query tile
 * computes O_s and LSE_s over its key range into the workspace (fp32); a second
 * kernel merges them per row: LSE = log sum_s exp(LSE_s), O = sum_s
 * exp(LSE_s - LSE) O_s. The result equals attn_fwd_gqa's up to rounding.
 *   n_splits        : 1 .. 1024, or 0 to pick enough units to give every compute
 *                     unit one; clamped to the number of 64-key tiles (and
 *                     reduced so that no unit is empty).
 *   workspace       : DEVICE buffer, 256-byte aligned, of at least
 *                     attn_fwd_splitkv_workspace_size(B, H, N, d, n_splits)
 *                     bytes, owned by the caller; must not overlap any tensor.
 *                     Its contents on entry are ignored; on return they are
 *                     unspecified. Calls that share a workspace must not overlap.
 *                     With one unit per query tile the plain kernel runs and
 *                     the workspace is not touched (same bits either way).
 *   opts            : tau and o_dtype as for attn_fwd_ex; exp2_poly_eighths must
 *                     be 0 and rescale_count NULL (else ATTN_ERR_UNSUPPORTED).
 * Other arguments and errors as for attn_fwd_gqa; also ATTN_ERR_NULL (no
 * workspace), ATTN_ERR_MISALIGNED, ATTN_ERR_DIM (workspace too small, n_splits
 * out of range, B*H*N + 4 above 2^31 - 1), ATTN_ERR_ALIAS (workspace overlaps).
 * Two kernels are enqueued on `stream`.
 */
attn_status_t attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int Hkv, int N, int d, int causal, float scale,
                               int n_splits, void* workspace, size_t workspace_bytes,
                               const attn_fwd_opts* opts, void* stream);

/* Workspace bytes attn_fwd_splitkv needs for these sizes (0 for invalid or
 * empty sizes). Host only. */
size_t attn_fwd_splitkv_workspace_size(int B, int H, int N, int d, int n_splits);

/* Size of the device scratch array attn_fwd_splitkv_noalloc uses (64 MiB). */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * attn_fwd_splitkv_noalloc - attn_fwd_splitkv for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation. The split-key partial results go to
 * a scratch array of ATTN_NOALLOC_SCRATCH_BYTES bytes that the library holds on
 * every GPU it runs on, for the life of the process (its address is looked up
 * once per device, on the first call there). The call allocates nothing and
 * frees nothing; the caller still passes q, k, v, o and lse.
 *   Sizes whose workspace (attn_fwd_splitkv_workspace_size) exceeds the scratch
 *   array return ATTN_ERR_DIM with the sizes in attn_last_error(); nothing is
 *   launched. The scratch contents on entry do not matter (every partial result
 *   the merge reads is written by the same call).
 *   Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 *   (other streams, other host threads) race and give undefined results.
 * Arguments, results and other errors as for attn_fwd_splitkv; ATTN_ERR_HIP if
 * the scratch address cannot be obtained.
 */
attn_status_t attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                       int B, int H, int Hkv, int N, int d, int causal, float scale,
                                       int n_splits, const attn_fwd_opts* opts, void* stream);

/* Tile shape the kernel uses for head dim d: query rows per workgroup and keys
 * per KV tile (the granularity of the online softmax and of the rescale
 * decisions, which the optional rescale counter reports). Returns ATTN_OK, or
 * ATTN_ERR_UNSUPPORTED for a head dim other than 64 or 128, or ATTN_ERR_NULL. */
attn_status_t attn_fwd_tile_shape(int d, int* query_rows, int* key_cols);

/* Static text for a status code. Takes any int (an attn_status_t converts
 * implicitly); a value that is not a status gives "unknown status". */
const char* attn_status_str(int status);

/* Text of the last error raised on the calling thread ("" if none). */
const char* attn_last_error(void);

/* ATTN_ABI_VERSION of the loaded library. */
int attn_abi_version(void);

/*
 * Host evaluation of the kernel's polynomial 2^x (the same inline routine the
 * device code uses), for checking its error bound on the CPU. Writes
 * y[i] = 2^x[i] for i < n. Inputs below -127 are clamped to -127.
 */
void attn_exp2_poly_host(const float* x, float* y, size_t n);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_H */
