// attn_fwd.hip - C ABI, argument checks and launch of the gfx950 attention forward kernel.
//
// The operation is exact scaled-dot-product attention (page "FlashAttention 4:
// faster, more memory-efficient attention for LLMs", section "Introduction"),
// computed by the tiled kernel in attn_fwd_kernel.h. The contract of every
// entry point is documented in include/attn_fwd.h.
#include <hip/hip_runtime.h>

#include <math.h>

#include <atomic>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "attn_fwd.h"
#include "attn_fwd_kernel.h"
#include "exp2_poly.h"

namespace {

thread_local char g_last_error[256] = "";

attn_status_t fail(attn_status_t s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
attn_status_t fail(attn_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Tile configuration: 8 wavefronts (256 query rows) per workgroup, BC keys per KV tile.
constexpr int kWaves = 8;
constexpr int kRows = 32 * kWaves;  // query rows per workgroup
template <int D> struct Cfg;
template <> struct Cfg<128> { static constexpr int BC = 64; };
template <> struct Cfg<64> { static constexpr int BC = 64; };

// Compute units per XCD of the current device (8 XCDs per MI355X), cached per
// device; 0 if the runtime cannot tell (then every tile gets its own workgroup).
int cus_per_xcd() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8) return 0;
    v = cus / 8;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

template <int D, bool CAUSAL, bool OF32, int POLY8>
hipError_t launch(const attn::Params& p, bool neg, hipStream_t stream) {
  // hipLaunchKernel reports this launch's own error (no sticky state from other calls).
  // A negative scale flips the row maximum of s*c into c * min(s): separate instantiation.
  // One workgroup per compute unit walks its XCD's tile range, so the next tile's
  // loads overlap the current tile's epilogue (causal: in a length-balanced order).
  int per_wg_xcd = p.per_xcd;
  const int slots = cus_per_xcd();
  if (slots > 0 && slots < per_wg_xcd) per_wg_xcd = slots;
  const dim3 grid(per_wg_xcd * 8), block(64 * kWaves);
  void* args[] = {const_cast<attn::Params*>(&p)};
  const void* fn = neg ? reinterpret_cast<const void*>(&attn::attn_fwd_kernel<D, Cfg<D>::BC, CAUSAL, OF32, POLY8, true>)
                       : reinterpret_cast<const void*>(&attn::attn_fwd_kernel<D, Cfg<D>::BC, CAUSAL, OF32, POLY8, false>);
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

template <int D, bool CAUSAL, bool OF32>
hipError_t launch_poly(const attn::Params& p, int poly8, bool neg, hipStream_t s) {
  switch (poly8) {
    case 0: return launch<D, CAUSAL, OF32, 0>(p, neg, s);
    case 4: return launch<D, CAUSAL, OF32, 4>(p, neg, s);
    default: return launch<D, CAUSAL, OF32, 8>(p, neg, s);
  }
}

template <int D>
hipError_t launch_d(const attn::Params& p, bool causal, bool of32, int poly8, bool neg, hipStream_t s) {
  if (causal)
    return of32 ? launch_poly<D, true, true>(p, poly8, neg, s) : launch_poly<D, true, false>(p, poly8, neg, s);
  return of32 ? launch_poly<D, false, true>(p, poly8, neg, s) : launch_poly<D, false, false>(p, poly8, neg, s);
}

attn_status_t check_impl(const void* q, const void* k, const void* v, const void* o, const float* lse, int B,
                         int H, int Hkv, int N, int d, float scale, const attn_fwd_opts* opts) {
  g_last_error[0] = '\0';
  attn_fwd_opts def;
  attn_fwd_opts_init(&def);
  if (opts) {
    if (opts->struct_size < sizeof(attn_fwd_opts))
      return fail(ATTN_ERR_OPTS, "opts->struct_size %zu < %zu", opts->struct_size, sizeof(attn_fwd_opts));
    def = *opts;
  }
  if (B < 0 || H < 0 || N < 0) return fail(ATTN_ERR_DIM, "negative size B=%d H=%d N=%d", B, H, N);
  if (H > 0 ? (Hkv < 1 || Hkv > H || H % Hkv != 0) : Hkv != 0)
    return fail(ATTN_ERR_DIM, "key/value heads Hkv=%d must divide query heads H=%d", Hkv, H);
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dim d=%d (supported: 64, 128)", d);
  if (!isfinite(scale)) return fail(ATTN_ERR_SCALE, "scale is not finite");
  if (!(def.rescale_tau_log2 >= 0.f && def.rescale_tau_log2 <= 64.f))
    return fail(ATTN_ERR_OPTS, "rescale_tau_log2 %g outside [0, 64]", (double)def.rescale_tau_log2);
  if (def.exp2_poly_eighths != 0 && def.exp2_poly_eighths != 4 && def.exp2_poly_eighths != 8)
    return fail(ATTN_ERR_UNSUPPORTED, "exp2_poly_eighths %d (supported: 0, 4, 8)", def.exp2_poly_eighths);
  if (def.o_dtype != ATTN_O_BF16 && def.o_dtype != ATTN_O_F32)
    return fail(ATTN_ERR_UNSUPPORTED, "o_dtype %d", def.o_dtype);
  if ((int64_t)B * H * N == 0) return ATTN_OK;  // empty: nothing to do

  const int64_t rows = (int64_t)B * H * N;
  const int64_t tiles = (int64_t)B * H * ((N + kRows - 1) / kRows);
  if (rows > (int64_t)1 << 40 || tiles + 8 > INT32_MAX)
    return fail(ATTN_ERR_DIM, "problem too large: B*H*N=%lld", (long long)rows);
  // one head's tensor (plus one tile of padding rows) is addressed with 32-bit byte offsets
  if ((int64_t)(N + 256) * d * 2 > INT32_MAX) return fail(ATTN_ERR_DIM, "N=%d too long for one head", N);
  if (!q || !k || !v || !o || !lse) return fail(ATTN_ERR_NULL, "NULL tensor pointer");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15)
    return fail(ATTN_ERR_MISALIGNED, "q, k, v and o must be 16-byte aligned");
  if ((uintptr_t)lse & 3) return fail(ATTN_ERR_MISALIGNED, "lse must be 4-byte aligned");
  if (def.rescale_count && ((uintptr_t)def.rescale_count & 3))
    return fail(ATTN_ERR_MISALIGNED, "rescale_count must be 4-byte aligned");

  const size_t q_bytes = (size_t)rows * d * 2;
  const size_t kv_bytes = (size_t)B * Hkv * N * d * 2;
  const size_t o_bytes = (size_t)rows * d * (def.o_dtype == ATTN_O_F32 ? 4 : 2);
  const size_t l_bytes = (size_t)rows * 4;
  const void* ins[3] = {q, k, v};
  const size_t in_bytes[3] = {q_bytes, kv_bytes, kv_bytes};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(o, o_bytes, ins[i], in_bytes[i])) return fail(ATTN_ERR_ALIAS, "o overlaps an input");
    if (overlaps(lse, l_bytes, ins[i], in_bytes[i])) return fail(ATTN_ERR_ALIAS, "lse overlaps an input");
    if (def.rescale_count && overlaps(def.rescale_count, l_bytes, ins[i], in_bytes[i]))
      return fail(ATTN_ERR_ALIAS, "rescale_count overlaps an input");
  }
  if (overlaps(o, o_bytes, lse, l_bytes)) return fail(ATTN_ERR_ALIAS, "o overlaps lse");
  if (def.rescale_count &&
      (overlaps(def.rescale_count, l_bytes, o, o_bytes) || overlaps(def.rescale_count, l_bytes, lse, l_bytes)))
    return fail(ATTN_ERR_ALIAS, "rescale_count overlaps an output");
  return ATTN_OK;
}

attn_status_t run(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N,
                  int d, int causal, float scale, const attn_fwd_opts* opts, void* stream) {
  const attn_status_t st = check_impl(q, k, v, o, lse, B, H, Hkv, N, d, scale, opts);
  if (st != ATTN_OK) return st;
  if ((int64_t)B * H * N == 0) return ATTN_OK;
  attn_fwd_opts o2;
  attn_fwd_opts_init(&o2);
  if (opts) o2 = *opts;

  attn::Params p;
  p.q = (const __bf16*)q;
  p.k = (const __bf16*)k;
  p.v = (const __bf16*)v;
  p.o = o;
  p.lse = lse;
  p.rescale_count = o2.rescale_count;
  p.N = N;
  p.H = H;
  p.G = H / Hkv;
  p.nq_tiles = (N + kRows - 1) / kRows;
  p.total_tiles = B * H * p.nq_tiles;
  p.per_xcd = (p.total_tiles + 7) / 8;
  // c = scale * log2(e) in fp32. Masked scores are set to -inf (+inf for a negative
  // scale) and rely on s*c - m = -inf; for scale == 0 that product would be NaN, so
  // 0 is replaced by 2^-100: |s| <= 2^17 for bf16 inputs with d <= 128, hence
  // |s*c| < 2^-82 and 2^(s*c - m) rounds to exactly 1.0f, as with c = 0.
  p.c = scale * 1.44269504088896341f;
  if (p.c == 0.f) p.c = 0x1p-100f;
  p.tau = o2.rescale_tau_log2;

  const bool of32 = o2.o_dtype == ATTN_O_F32;
  const bool neg = scale < 0.f;
  const hipError_t err =
      d == 128 ? launch_d<128>(p, causal != 0, of32, o2.exp2_poly_eighths, neg, (hipStream_t)stream)
               : launch_d<64>(p, causal != 0, of32, o2.exp2_poly_eighths, neg, (hipStream_t)stream);
  if (err != hipSuccess) return fail(ATTN_ERR_HIP, "kernel launch: %s", hipGetErrorString(err));
  return ATTN_OK;
}

}  // namespace

extern "C" {

void attn_fwd_opts_init(attn_fwd_opts* opts) {
  if (!opts) return;
  memset(opts, 0, sizeof *opts);
  opts->struct_size = sizeof *opts;
  opts->rescale_tau_log2 = 8.0f;
  opts->exp2_poly_eighths = 0;
  opts->o_dtype = ATTN_O_BF16;
  opts->rescale_count = nullptr;
}

attn_status_t attn_fwd_check(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, int B, int H, int N, int d, int causal,
                             float scale, const attn_fwd_opts* opts) {
  (void)causal;
  return check_impl(q, k, v, o, lse, B, H, H, N, d, scale, opts);
}

attn_status_t attn_fwd_gqa_check(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                 int B, int H, int Hkv, int N, int d, int causal, float scale,
                                 const attn_fwd_opts* opts) {
  (void)causal;
  return check_impl(q, k, v, o, lse, B, H, Hkv, N, d, scale, opts);
}

attn_status_t attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                          int N, int d, int causal, float scale, const attn_fwd_opts* opts, void* stream) {
  return run(q, k, v, o, lse, B, H, H, N, d, causal, scale, opts, stream);
}

attn_status_t attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                           int Hkv, int N, int d, int causal, float scale, const attn_fwd_opts* opts,
                           void* stream) {
  return run(q, k, v, o, lse, B, H, Hkv, N, d, causal, scale, opts, stream);
}

attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                       int d, int causal, float scale, void* stream) {
  return attn_fwd_ex(q, k, v, o, lse, B, H, N, d, causal, scale, nullptr, stream);
}

const char* attn_status_str(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer";
    case ATTN_ERR_DIM: return "bad dimensions";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head dim or option";
    case ATTN_ERR_MISALIGNED: return "misaligned pointer";
    case ATTN_ERR_SCALE: return "scale not finite";
    case ATTN_ERR_ALIAS: return "output overlaps another tensor";
    case ATTN_ERR_HIP: return "HIP launch error";
    case ATTN_ERR_OPTS: return "bad options";
  }
  return "unknown status";
}

const char* attn_last_error(void) { return g_last_error; }

attn_status_t attn_fwd_tile_shape(int d, int* query_rows, int* key_cols) {
  if (!query_rows || !key_cols) return fail(ATTN_ERR_NULL, "NULL output pointer");
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dim d=%d (supported: 64, 128)", d);
  *query_rows = kRows;
  *key_cols = d == 128 ? Cfg<128>::BC : Cfg<64>::BC;
  return ATTN_OK;
}

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

void attn_exp2_poly_host(const float* x, float* y, size_t n) {
  for (size_t i = 0; i < n; ++i) y[i] = attn_exp2_poly(x[i]);
}

}  // extern "C"
