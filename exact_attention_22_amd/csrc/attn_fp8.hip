// attn_fp8.hip - C ABI, argument checks and launch of the gfx950 FP8 attention
// forward kernel (attn_fp8_kernel.h). The contract is documented in
// include/attn_fp8.h.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "attn_fp8.h"
#include "attn_fp8_kernel.h"
#include "attn_host.h"

namespace {

using attn_host::fail;
using attn_host::overlaps;

attn_status_t validate(const void* q, const void* k, const void* vt, const void* o, const float* lse, int B, int H,
                       int N, int d, float scale, float qs, float ks, float vs, float tau, bool* work) {
  attn_host::clear_error();
  *work = false;
  if (B < 0 || H < 0 || N < 0) return fail(ATTN_ERR_DIM, "negative size B=%d H=%d N=%d", B, H, N);
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dim d=%d (supported: 64, 128)", d);
  if (!(tau >= 0.f && tau <= 8.f)) return fail(ATTN_ERR_UNSUPPORTED, "tau=%g outside [0, 8]", (double)tau);
  const float sc[4] = {scale, qs, ks, vs};
  for (float x : sc)
    if (!isfinite(x) || !(x > 0.f)) return fail(ATTN_ERR_SCALE, "scales must be finite and positive");
  const float c = scale * qs * ks * 1.44269504088896341f;
  if (!isnormal(c)) return fail(ATTN_ERR_SCALE, "scale * q_scale * k_scale is not a normal fp32 value");
  if ((int64_t)B * H * N == 0) return ATTN_OK;
  const int64_t rows = (int64_t)B * H * N;
  const int64_t ldv = ((int64_t)N + 15) / 16 * 16;
  const int64_t tiles = (int64_t)B * H * ((N + attn_fp8::kMinRows - 1) / attn_fp8::kMinRows);
  if (rows > (int64_t)1 << 40 || tiles > INT32_MAX / 2 || ldv > INT32_MAX)
    return fail(ATTN_ERR_DIM, "problem too large: B*H*N=%lld", (long long)rows);
  // within one head the kernel forms byte offsets such as (N - j0) * d and
  // d * ldv - j0 in 32 bits, and its buffer resources count bytes in 32 bits
  if ((ldv + 64) * d > INT32_MAX)
    return fail(ATTN_ERR_DIM, "N=%d too large: one head's %lld x %d bytes exceed 32-bit offsets", N,
                (long long)ldv, d);
  if (!q || !k || !vt || !o || !lse) return fail(ATTN_ERR_NULL, "NULL tensor pointer");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)vt | (uintptr_t)o) & 15)
    return fail(ATTN_ERR_MISALIGNED, "q, k, vt and o must be 16-byte aligned");
  if ((uintptr_t)lse & 3) return fail(ATTN_ERR_MISALIGNED, "lse must be 4-byte aligned");
  const size_t qb = (size_t)rows * d, vb = (size_t)B * H * d * ldv, ob = (size_t)rows * d * 2, lb = (size_t)rows * 4;
  const void* ins[3] = {q, k, vt};
  const size_t in_b[3] = {qb, qb, vb};
  for (int j = 0; j < 3; ++j)
    if (overlaps(o, ob, ins[j], in_b[j]) || overlaps(lse, lb, ins[j], in_b[j]))
      return fail(ATTN_ERR_ALIAS, "an output overlaps an input");
  if (overlaps(o, ob, lse, lb)) return fail(ATTN_ERR_ALIAS, "o overlaps lse");
  *work = true;
  return ATTN_OK;
}

template <int D, bool CAUSAL>
hipError_t launch(const attn_fp8::Fp8Params& p, bool ref, hipStream_t stream) {
  void* args[] = {const_cast<attn_fp8::Fp8Params*>(&p)};
  const void* fn = ref ? reinterpret_cast<const void*>(&attn_fp8::attn_fwd_fp8_kernel<D, CAUSAL, true>)
                       : reinterpret_cast<const void*>(&attn_fp8::attn_fwd_fp8_kernel<D, CAUSAL, false>);
  return hipLaunchKernel(fn, dim3(p.n_xcd * p.per_xcd), dim3(64 * attn_fp8::Shape<D>::NW), args, 0, stream);
}

}  // namespace

extern "C" {

attn_status_t attn_fwd_fp8_check(const void* q, const void* k, const void* vt, const void* o, const float* lse, int B,
                                 int H, int N, int d, int causal, float scale, float q_scale, float k_scale,
                                 float v_scale, float tau) {
  (void)causal;
  bool work;
  return validate(q, k, vt, o, lse, B, H, N, d, scale, q_scale, k_scale, v_scale, tau, &work);
}

attn_status_t attn_fwd_fp8_ex(const void* q, const void* k, const void* vt, void* o, float* lse, int B, int H,
                              int N, int d, int causal, float scale, float q_scale, float k_scale, float v_scale,
                              float tau, int schedule, void* stream) {
  bool work = false;
  attn_status_t st = validate(q, k, vt, o, lse, B, H, N, d, scale, q_scale, k_scale, v_scale, tau, &work);
  if (st == ATTN_OK && schedule != ATTN_SCHEDULE_PIPELINED && schedule != ATTN_SCHEDULE_REFERENCE)
    st = fail(ATTN_ERR_OPTS, "schedule %d", schedule);
  if (st != ATTN_OK || !work) return st;
  const bool ref = schedule == ATTN_SCHEDULE_REFERENCE;
  attn_fp8::Fp8Params p;
  p.q = (const uint8_t*)q;
  p.k = (const uint8_t*)k;
  p.vt = (const uint8_t*)vt;
  p.o = (__bf16*)o;
  p.lse = lse;
  p.N = N;
  p.ldv = (N + 15) / 16 * 16;
  const int rows = d == 128 ? attn_fp8::Shape<128>::ROWS : attn_fp8::Shape<64>::ROWS;
  p.nq_tiles = (N + rows - 1) / rows;
  p.total_tiles = B * H * p.nq_tiles;
  const attn_host::DeviceShape ds = attn_host::device_shape();
  p.n_xcd = ds.xcds;
  p.per_xcd = (p.total_tiles + p.n_xcd - 1) / p.n_xcd;
  p.cus_per_xcd = ds.cus / ds.xcds;
  p.c = scale * q_scale * k_scale * 1.44269504088896341f;
  p.ov = v_scale;
  p.tau = tau;
  p.psum_thr = (1.f - 0x1p-10f) * exp2f(tau);  // P above 2^tau puts a partial sum above this
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (d == 128)
    e = causal ? launch<128, true>(p, ref, s) : launch<128, false>(p, ref, s);
  else
    e = causal ? launch<64, true>(p, ref, s) : launch<64, false>(p, ref, s);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ATTN_OK;
}

attn_status_t attn_fwd_fp8(const void* q, const void* k, const void* vt, void* o, float* lse, int B, int H, int N,
                           int d, int causal, float scale, float q_scale, float k_scale, float v_scale, float tau,
                           void* stream) {
  return attn_fwd_fp8_ex(q, k, vt, o, lse, B, H, N, d, causal, scale, q_scale, k_scale, v_scale, tau,
                         ATTN_SCHEDULE_PIPELINED, stream);
}

}  // extern "C"
