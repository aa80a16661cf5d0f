// attn_bwd.hip - C ABI, argument checks and launches of the gfx950 attention
// backward kernels (attn_bwd_kernel.h). The contract of every entry point is
// documented in include/attn_bwd.h.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "attn_bwd.h"
#include "attn_bwd_kernel.h"
#include "attn_host.h"

namespace {

using attn_host::fail;
using attn_host::overlaps;

attn_status_t validate(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                       const void* dq, const void* dk, const void* dv, const float* delta, int B, int H, int Hkv,
                       int N, int d, float scale, bool* work) {
  attn_host::clear_error();
  *work = false;
  if (B < 0 || H < 0 || N < 0) return fail(ATTN_ERR_DIM, "negative size B=%d H=%d N=%d", B, H, N);
  if (H > 0 ? (Hkv < 1 || Hkv > H || H % Hkv != 0) : Hkv != 0)
    return fail(ATTN_ERR_DIM, "key/value heads Hkv=%d must divide query heads H=%d", Hkv, H);
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dim d=%d (supported: 64, 128)", d);
  if (!isfinite(scale)) return fail(ATTN_ERR_SCALE, "scale is not finite");
  if ((int64_t)B * H * N == 0) return ATTN_OK;
  const int64_t rows = (int64_t)B * H * N;
  const int64_t tiles = (int64_t)B * H * ((N + attn_grad::kRows - 1) / attn_grad::kRows);
  if (rows > (int64_t)1 << 40 || tiles > INT32_MAX)
    return fail(ATTN_ERR_DIM, "problem too large: B*H*N=%lld", (long long)rows);
  if ((int64_t)(N + 256) * d * 2 > INT32_MAX) return fail(ATTN_ERR_DIM, "N=%d too long for one head", N);
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta)
    return fail(ATTN_ERR_NULL, "NULL tensor pointer");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout | (uintptr_t)dq | (uintptr_t)dk |
       (uintptr_t)dv) & 15)
    return fail(ATTN_ERR_MISALIGNED, "q, k, v, o, dout, dq, dk and dv must be 16-byte aligned");
  if (((uintptr_t)lse | (uintptr_t)delta) & 3) return fail(ATTN_ERR_MISALIGNED, "lse and delta must be 4-byte aligned");
  const size_t qb = (size_t)rows * d * 2, kvb = (size_t)B * Hkv * N * d * 2, lb = (size_t)rows * 4;
  const void* ins[6] = {q, k, v, o, lse, dout};
  const size_t in_b[6] = {qb, kvb, kvb, qb, lb, qb};
  const void* outs[4] = {dq, dk, dv, delta};
  const size_t out_b[4] = {qb, kvb, kvb, lb};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], out_b[i], ins[j], in_b[j])) return fail(ATTN_ERR_ALIAS, "an output overlaps an input");
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], out_b[i], outs[j], out_b[j])) return fail(ATTN_ERR_ALIAS, "two outputs overlap");
  }
  *work = true;
  return ATTN_OK;
}

// Packed batches: q, o, dout, dq [H][total][d]; k, v, dk, dv [Hkv][total][d]; lse, delta
// [H][total]; cu_seqlens B + 1 device int32 (contents not validated: the kernels clamp
// every bound into [0, total]).
attn_status_t validate_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, const void* dq, const void* dk, const void* dv, const float* delta,
                              const int* cu, int B, int H, int Hkv, int total, int max_seqlen, int d, float scale,
                              bool* work) {
  attn_host::clear_error();
  *work = false;
  if (B < 0 || H < 0 || total < 0 || max_seqlen < 0)
    return fail(ATTN_ERR_DIM, "negative size B=%d H=%d total=%d max_seqlen=%d", B, H, total, max_seqlen);
  if (H > 0 ? (Hkv < 1 || Hkv > H || H % Hkv != 0) : Hkv != 0)
    return fail(ATTN_ERR_DIM, "key/value heads Hkv=%d must divide query heads H=%d", Hkv, H);
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dim d=%d (supported: 64, 128)", d);
  if (!isfinite(scale)) return fail(ATTN_ERR_SCALE, "scale is not finite");
  const int64_t seq = max_seqlen < total ? max_seqlen : total;
  if ((int64_t)B * H * seq == 0) return ATTN_OK;
  const int64_t rows = (int64_t)H * total;
  const int64_t tiles = (int64_t)B * H * ((seq + attn_grad::kRows - 1) / attn_grad::kRows);
  if (rows > (int64_t)1 << 40 || tiles > INT32_MAX)
    return fail(ATTN_ERR_DIM, "problem too large: H*total=%lld", (long long)rows);
  if ((int64_t)(total + 256) * d * 2 > INT32_MAX) return fail(ATTN_ERR_DIM, "total=%d too long", total);
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta || !cu)
    return fail(ATTN_ERR_NULL, "NULL tensor pointer");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout | (uintptr_t)dq | (uintptr_t)dk |
       (uintptr_t)dv) & 15)
    return fail(ATTN_ERR_MISALIGNED, "q, k, v, o, dout, dq, dk and dv must be 16-byte aligned");
  if (((uintptr_t)lse | (uintptr_t)delta | (uintptr_t)cu) & 3)
    return fail(ATTN_ERR_MISALIGNED, "lse, delta and cu_seqlens must be 4-byte aligned");
  const size_t qb = (size_t)rows * d * 2, kvb = (size_t)Hkv * total * d * 2, lb = (size_t)rows * 4;
  const void* ins[7] = {q, k, v, o, lse, dout, cu};
  const size_t in_b[7] = {qb, kvb, kvb, qb, lb, qb, (size_t)(B + 1) * 4};
  const void* outs[4] = {dq, dk, dv, delta};
  const size_t out_b[4] = {qb, kvb, kvb, lb};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 7; ++j)
      if (overlaps(outs[i], out_b[i], ins[j], in_b[j])) return fail(ATTN_ERR_ALIAS, "an output overlaps an input");
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], out_b[i], outs[j], out_b[j])) return fail(ATTN_ERR_ALIAS, "two outputs overlap");
  }
  *work = true;
  return ATTN_OK;
}

// nb: batch (dense) or number of sequences (packed); grids (dense) B*H*n_tiles and
// B*Hkv*n_tiles, (packed) H*nseq*n_tiles and Hkv*nseq*n_tiles.
template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch(const attn_grad::BwdParams& p, int nb, int Hkv, hipStream_t stream, bool reference = false) {
  void* args[] = {const_cast<attn_grad::BwdParams*>(&p)};
  const dim3 block(64 * attn_grad::kWaves);
  // dq first: it stores D, which the dkdv kernel reads (same stream, in order)
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&attn_grad::attn_bwd_dq_kernel<D, CAUSAL, VARLEN>),
                                 dim3(nb * p.H * p.n_tiles), block, args, 0, stream);
  if (e != hipSuccess) return e;
  // D = 128: wavefront pairs (two wavefronts per key block, eight per workgroup); the
  // reference schedule (dense layout only) runs the one-wavefront kernel instead
  if constexpr (D == 128 && !VARLEN) {
    if (reference)
      return hipLaunchKernel(reinterpret_cast<const void*>(&attn_grad::attn_bwd_dkdv_kernel<D, CAUSAL, false>),
                             dim3(nb * Hkv * p.n_tiles), block, args, 0, stream);
  }
  if constexpr (D == 128)
    return hipLaunchKernel(reinterpret_cast<const void*>(&attn_grad::attn_bwd_dkdv_pair_kernel<D, CAUSAL, VARLEN>),
                           dim3(nb * Hkv * p.n_tiles), dim3(2 * 64 * attn_grad::kWaves), args, 0, stream);
  else
    return hipLaunchKernel(reinterpret_cast<const void*>(&attn_grad::attn_bwd_dkdv_kernel<D, CAUSAL, VARLEN>),
                           dim3(nb * Hkv * p.n_tiles), block, args, 0, stream);
}

template <bool VARLEN>
hipError_t launch_any(const attn_grad::BwdParams& p, int d, bool causal, int nb, int Hkv, hipStream_t s,
                      bool reference = false) {
  if (d == 128)
    return causal ? launch<128, true, VARLEN>(p, nb, Hkv, s, reference)
                  : launch<128, false, VARLEN>(p, nb, Hkv, s, reference);
  return causal ? launch<64, true, VARLEN>(p, nb, Hkv, s) : launch<64, false, VARLEN>(p, nb, Hkv, s);
}

attn_grad::BwdParams make_params(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                 const void* dout, void* dq, void* dk, void* dv, float* delta, int H, int Hkv,
                                 float scale) {
  attn_grad::BwdParams p;
  p.q = (const __bf16*)q;
  p.k = (const __bf16*)k;
  p.v = (const __bf16*)v;
  p.o = (const __bf16*)o;
  p.lse = lse;
  p.dout = (const __bf16*)dout;
  p.dq = (__bf16*)dq;
  p.dk = (__bf16*)dk;
  p.dv = (__bf16*)dv;
  p.delta = delta;
  p.cu_seqlens = nullptr;
  p.nseq = 0;
  p.H = H;
  p.G = H / Hkv;
  p.scale = scale;
  p.c = scale * 1.44269504088896341f;
  const attn_host::DeviceShape ds = attn_host::device_shape();
  p.n_xcd = ds.xcds;
  p.cus_per_xcd = ds.cus / ds.xcds;
  return p;
}

}  // namespace

extern "C" {

attn_status_t attn_bwd_check(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, const void* dq, const void* dk, const void* dv, const float* delta,
                             int B, int H, int Hkv, int N, int d, int causal, float scale) {
  (void)causal;
  bool work;
  return validate(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Hkv, N, d, scale, &work);
}

attn_status_t attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H, int Hkv, int N,
                          int d, int causal, float scale, int schedule, void* stream) {
  bool work = false;
  attn_status_t st = validate(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Hkv, N, d, scale, &work);
  if (st == ATTN_OK && schedule != ATTN_SCHEDULE_PIPELINED && schedule != ATTN_SCHEDULE_REFERENCE)
    return fail(ATTN_ERR_OPTS, "unknown schedule %d", schedule);
  if (st != ATTN_OK || !work) return st;
  attn_grad::BwdParams p = make_params(q, k, v, o, lse, dout, dq, dk, dv, delta, H, Hkv, scale);
  p.N = N;
  p.n_tiles = (N + attn_grad::kRows - 1) / attn_grad::kRows;
  const hipError_t e =
      launch_any<false>(p, d, causal != 0, B, Hkv, (hipStream_t)stream, schedule == ATTN_SCHEDULE_REFERENCE);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ATTN_OK;
}

attn_status_t attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H, int Hkv, int N,
                       int d, int causal, float scale, void* stream) {
  return attn_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Hkv, N, d, causal, scale,
                     ATTN_SCHEDULE_PIPELINED, stream);
}

attn_status_t attn_bwd_varlen_check(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                    const void* dout, const void* dq, const void* dk, const void* dv,
                                    const float* delta, const int* cu_seqlens, int B, int H, int Hkv, int total,
                                    int max_seqlen, int d, int causal, float scale) {
  (void)causal;
  bool work;
  return validate_varlen(q, k, v, o, lse, dout, dq, dk, dv, delta, cu_seqlens, B, H, Hkv, total, max_seqlen, d, scale,
                         &work);
}

attn_status_t attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, void* dq, void* dk, void* dv, float* delta, const int* cu_seqlens,
                              int B, int H, int Hkv, int total, int max_seqlen, int d, int causal, float scale,
                              void* stream) {
  bool work = false;
  const attn_status_t st = validate_varlen(q, k, v, o, lse, dout, dq, dk, dv, delta, cu_seqlens, B, H, Hkv, total,
                                           max_seqlen, d, scale, &work);
  if (st != ATTN_OK || !work) return st;
  attn_grad::BwdParams p = make_params(q, k, v, o, lse, dout, dq, dk, dv, delta, H, Hkv, scale);
  p.cu_seqlens = cu_seqlens;
  p.nseq = B;
  p.N = total;
  const int seq = max_seqlen < total ? max_seqlen : total;
  p.n_tiles = (seq + attn_grad::kRows - 1) / attn_grad::kRows;
  const hipError_t e = launch_any<true>(p, d, causal != 0, B, Hkv, (hipStream_t)stream);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ATTN_OK;
}

}  // extern "C"
