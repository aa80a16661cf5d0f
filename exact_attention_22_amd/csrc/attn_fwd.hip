// attn_fwd.hip - C ABI, argument checks and launch of the gfx950 attention forward kernel.
//
// The operation is exact scaled-dot-product attention (page "FlashAttention 4:
// faster, more memory-efficient attention for LLMs", section "Introduction"),
// computed by the tiled kernel in attn_fwd_kernel.h. The contract of every
// entry point is documented in include/attn_fwd.h.
#include <hip/hip_runtime.h>

#include <math.h>

#include <atomic>
#include <mutex>
#include <stdarg.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "attn_fwd.h"
#include "attn_host.h"
#include "attn_fwd_launch.h"
#include "exp2_poly.h"

namespace attn_host {

thread_local char g_last_error[256] = "";

void clear_error() { g_last_error[0] = '\0'; }

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

}  // namespace attn_host

namespace attn_host {

DeviceShape device_shape() {
  static std::atomic<int> cache[64];  // per device: xcds << 16 | cus, 0 = not yet read
  const DeviceShape fallback{8, 256};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fallback;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0, xcds = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1 ||
        cus > 0xFFFF)
      return fallback;
    if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcds < 1 || xcds > cus)
      xcds = cus % 8 == 0 ? 8 : 1;
    v = xcds << 16 | cus;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return DeviceShape{v >> 16, v & 0xFFFF};
}

}  // namespace attn_host

namespace attn_launch {

int cus_per_xcd() {
  const attn_host::DeviceShape ds = attn_host::device_shape();
  return ds.cus / ds.xcds;
}

}  // namespace attn_launch

namespace {

using attn_host::fail;
using attn_host::g_last_error;
using attn_host::overlaps;

using attn_launch::Cfg;
using attn_launch::kRows;

hipError_t launch_any(const attn::Params& p, int d, bool causal, bool of32, int poly8, bool neg, bool varlen,
                      bool ref, hipStream_t s) {
  using attn_launch::launch_dense;
  if (d == 128)
    return causal ? launch_dense<128, true>(p, of32, poly8, neg, varlen, ref, s)
                  : launch_dense<128, false>(p, of32, poly8, neg, varlen, ref, s);
  return causal ? launch_dense<64, true>(p, of32, poly8, neg, varlen, ref, s)
                : launch_dense<64, false>(p, of32, poly8, neg, varlen, ref, s);
}

// One call, dense ([B][H][N][d]) or packed (varlen: [H][total][d] with cu_seqlens).
struct Problem {
  const void *q, *k, *v;
  void* o;
  float* lse;
  const int* cu;   // packed only
  bool varlen;
  int B, H, Hkv;   // B: batch (dense) or number of sequences (packed)
  int N;           // dense: sequence length; packed: total tokens per head
  int max_seqlen;  // packed only
  int d;
  float scale;
};

// Host-side validation shared by every entry point (never touches the device).
// On success *def holds the options in effect and *work whether anything is to be done.
attn_status_t validate(const Problem& P, const attn_fwd_opts* opts, attn_fwd_opts* def, bool* work) {
  g_last_error[0] = '\0';
  *work = false;
  attn_fwd_opts_init(def);
  if (opts) {
    // callers built against a header without `schedule` pass the shorter struct
    // and get the default schedule
    const size_t base = offsetof(attn_fwd_opts, schedule);
    if (opts->struct_size < base)
      return fail(ATTN_ERR_OPTS, "opts->struct_size %zu < %zu", opts->struct_size, base);
    memcpy(def, opts, opts->struct_size < sizeof(attn_fwd_opts) ? opts->struct_size : sizeof(attn_fwd_opts));
    def->struct_size = sizeof(attn_fwd_opts);
  }
  const int B = P.B, H = P.H, Hkv = P.Hkv, N = P.N, d = P.d;
  if (B < 0 || H < 0 || N < 0) return fail(ATTN_ERR_DIM, "negative size B=%d H=%d N=%d", B, H, N);
  if (P.varlen && P.max_seqlen < 0) return fail(ATTN_ERR_DIM, "negative max_seqlen %d", P.max_seqlen);
  if (H > 0 ? (Hkv < 1 || Hkv > H || H % Hkv != 0) : Hkv != 0)
    return fail(ATTN_ERR_DIM, "key/value heads Hkv=%d must divide query heads H=%d", Hkv, H);
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dim d=%d (supported: 64, 128)", d);
  if (!isfinite(P.scale)) return fail(ATTN_ERR_SCALE, "scale is not finite");
  if (!(def->rescale_tau_log2 >= 0.f && def->rescale_tau_log2 <= 64.f))
    return fail(ATTN_ERR_OPTS, "rescale_tau_log2 %g outside [0, 64]", (double)def->rescale_tau_log2);
  if (def->exp2_poly_eighths != 0 && def->exp2_poly_eighths != 4 && def->exp2_poly_eighths != 8)
    return fail(ATTN_ERR_UNSUPPORTED, "exp2_poly_eighths %d (supported: 0, 4, 8)", def->exp2_poly_eighths);
  if (def->o_dtype != ATTN_O_BF16 && def->o_dtype != ATTN_O_F32)
    return fail(ATTN_ERR_UNSUPPORTED, "o_dtype %d", def->o_dtype);
  if (def->schedule != ATTN_SCHEDULE_PIPELINED && def->schedule != ATTN_SCHEDULE_REFERENCE)
    return fail(ATTN_ERR_OPTS, "schedule %d", def->schedule);
  if (def->schedule == ATTN_SCHEDULE_REFERENCE && (def->exp2_poly_eighths != 0 || P.scale < 0.f))
    return fail(ATTN_ERR_UNSUPPORTED, "the reference schedule needs exp2_poly_eighths 0 and scale >= 0");
  // longest sequence a query tile walk has to cover
  const int64_t seq = P.varlen ? (P.max_seqlen < N ? P.max_seqlen : N) : N;
  if ((int64_t)B * H * seq == 0) return ATTN_OK;  // empty: nothing to do

  // output rows: B*H*N (dense) or H*total (packed)
  const int64_t rows = P.varlen ? (int64_t)H * N : (int64_t)B * H * N;
  const int64_t tiles = (int64_t)B * H * ((seq + kRows - 1) / kRows);
  if (rows > (int64_t)1 << 40 || tiles + 8 > INT32_MAX)
    return fail(ATTN_ERR_DIM, "problem too large: %lld rows, %lld tiles", (long long)rows, (long long)tiles);
  // one head's rows (plus one tile of padding rows) are addressed with 32-bit byte
  // offsets; packed: the whole token axis, so that no contents of cu_seqlens can
  // take an offset past that range
  if ((int64_t)(N + 256) * d * 2 > INT32_MAX)
    return fail(ATTN_ERR_DIM, "%s=%d too long for 32-bit row offsets", P.varlen ? "total" : "N", N);
  if (!P.q || !P.k || !P.v || !P.o || !P.lse || (P.varlen && !P.cu))
    return fail(ATTN_ERR_NULL, "NULL tensor pointer");
  if (((uintptr_t)P.q | (uintptr_t)P.k | (uintptr_t)P.v | (uintptr_t)P.o) & 15)
    return fail(ATTN_ERR_MISALIGNED, "q, k, v and o must be 16-byte aligned");
  if ((uintptr_t)P.lse & 3) return fail(ATTN_ERR_MISALIGNED, "lse must be 4-byte aligned");
  if (P.varlen && ((uintptr_t)P.cu & 3)) return fail(ATTN_ERR_MISALIGNED, "cu_seqlens must be 4-byte aligned");
  if (def->rescale_count && ((uintptr_t)def->rescale_count & 3))
    return fail(ATTN_ERR_MISALIGNED, "rescale_count must be 4-byte aligned");

  const size_t q_bytes = (size_t)rows * d * 2;
  const size_t kv_bytes = (size_t)rows / H * Hkv * d * 2;
  const size_t o_bytes = (size_t)rows * d * (def->o_dtype == ATTN_O_F32 ? 4 : 2);
  const size_t l_bytes = (size_t)rows * 4;
  const void* ins[4] = {P.q, P.k, P.v, P.cu};
  const size_t in_bytes[4] = {q_bytes, kv_bytes, kv_bytes, P.varlen ? (size_t)(B + 1) * 4 : 0};
  for (int i = 0; i < 4; ++i) {
    if (overlaps(P.o, o_bytes, ins[i], in_bytes[i])) return fail(ATTN_ERR_ALIAS, "o overlaps an input");
    if (overlaps(P.lse, l_bytes, ins[i], in_bytes[i])) return fail(ATTN_ERR_ALIAS, "lse overlaps an input");
    if (def->rescale_count && overlaps(def->rescale_count, l_bytes, ins[i], in_bytes[i]))
      return fail(ATTN_ERR_ALIAS, "rescale_count overlaps an input");
  }
  if (overlaps(P.o, o_bytes, P.lse, l_bytes)) return fail(ATTN_ERR_ALIAS, "o overlaps lse");
  if (def->rescale_count &&
      (overlaps(def->rescale_count, l_bytes, P.o, o_bytes) || overlaps(def->rescale_count, l_bytes, P.lse, l_bytes)))
    return fail(ATTN_ERR_ALIAS, "rescale_count overlaps an output");
  *work = true;
  return ATTN_OK;
}

attn_status_t run(const Problem& P, int causal, const attn_fwd_opts* opts, void* stream) {
  attn_fwd_opts o2;
  bool work = false;
  const attn_status_t st = validate(P, opts, &o2, &work);
  if (st != ATTN_OK || !work) return st;

  attn::Params p;
  p.q = (const __bf16*)P.q;
  p.k = (const __bf16*)P.k;
  p.v = (const __bf16*)P.v;
  p.o = P.o;
  p.lse = P.lse;
  p.rescale_count = o2.rescale_count;
  p.cu_seqlens = P.varlen ? P.cu : nullptr;
  p.nseq = P.varlen ? P.B : 0;
  p.N = P.N;
  p.H = P.H;
  p.G = P.H / P.Hkv;
  const int seq = P.varlen ? (P.max_seqlen < P.N ? P.max_seqlen : P.N) : P.N;
  p.nq_tiles = (seq + kRows - 1) / kRows;
  p.total_tiles = P.B * P.H * p.nq_tiles;
  p.n_xcd = attn_host::device_shape().xcds;
  p.per_xcd = (p.total_tiles + p.n_xcd - 1) / p.n_xcd;
  // c = scale * log2(e) in fp32. Masked scores are set to -inf (+inf for a negative
  // scale) and rely on s*c - m = -inf; for scale == 0 that product would be NaN, so
  // 0 is replaced by 2^-100. For inputs with |q|, |k| < 2^33 (at d <= 128,
  // |s| < 2^73), every x = s*c - m then has |x| < 2^-26 and 2^x rounds to exactly
  // 1.0f, as with c = 0 (uniform weights over the visible keys).
  p.c = P.scale * 1.44269504088896341f;
  if (p.c == 0.f) p.c = 0x1p-100f;
  p.tau = o2.rescale_tau_log2;
  p.psum_thr = (1.f - 0x1p-10f) * exp2f(o2.rescale_tau_log2);  // P above 2^tau puts a partial sum above this
  p.n_splits = 1;
  p.split_tiles = 0;
  p.ws_o = nullptr;
  p.ws_lse = nullptr;
  p.split_stride = 0;

  const bool ref = o2.schedule == ATTN_SCHEDULE_REFERENCE;
  const bool of32 = o2.o_dtype == ATTN_O_F32;
  const bool neg = P.scale < 0.f;
  const hipError_t err =
      launch_any(p, P.d, causal != 0, of32, o2.exp2_poly_eighths, neg, P.varlen, ref, (hipStream_t)stream);
  if (err != hipSuccess) return fail(ATTN_ERR_HIP, "kernel launch: %s", hipGetErrorString(err));
  return ATTN_OK;
}

// Split keys into n_splits units per query tile (0: enough units to give every
// compute unit one). Returns the unit count through *splits and the key tiles per
// unit through *split_tiles.
void split_shape(int B, int H, int N, int d, int n_splits, int* splits, int* split_tiles) {
  const int bc = d == 128 ? Cfg<128>::BC : Cfg<64>::BC;
  const int key_tiles = (N + bc - 1) / bc;
  int s = n_splits;
  if (s <= 0) {
    const int64_t units = (int64_t)B * H * ((N + kRows - 1) / kRows);
    const int cus = attn_host::device_shape().cus;
    s = units >= cus ? 1 : (int)((cus + units - 1) / units);
  }
  s = s < 1 ? 1 : (s > key_tiles ? key_tiles : s);
  const int st = (key_tiles + s - 1) / s;
  *split_tiles = st;
  *splits = (key_tiles + st - 1) / st;  // no unit without key tiles
}

size_t split_workspace_bytes(int B, int H, int N, int d, int splits) {
  const size_t rows = (size_t)B * H * N;
  const size_t o_bytes = (splits * rows * d * 4 + 255) / 256 * 256;
  return o_bytes + splits * rows * 4;
}

attn_status_t run_split(const Problem& P, int causal, int n_splits, void* ws, size_t ws_bytes,
                        const attn_fwd_opts* opts, void* stream) {
  attn_fwd_opts o2;
  bool work = false;
  attn_status_t st = validate(P, opts, &o2, &work);
  if (st != ATTN_OK || !work) return st;
  if (n_splits < 0 || n_splits > 1024) return fail(ATTN_ERR_DIM, "n_splits %d outside [0, 1024]", n_splits);
  if (o2.exp2_poly_eighths != 0) return fail(ATTN_ERR_UNSUPPORTED, "split keys: exp2_poly_eighths must be 0");
  if (o2.rescale_count) return fail(ATTN_ERR_UNSUPPORTED, "split keys: no rescale counter");
  int splits, split_tiles;
  split_shape(P.B, P.H, P.N, P.d, n_splits, &splits, &split_tiles);
  const size_t need = split_workspace_bytes(P.B, P.H, P.N, P.d, splits);
  if (!ws) return fail(ATTN_ERR_NULL, "NULL workspace");
  // one unit per query tile: the merge would multiply by exp(0) = 1, so the plain
  // kernel gives the same bits without the workspace round trip
  if (splits == 1) return run(P, causal, opts, stream);
  if ((uintptr_t)ws & 255) return fail(ATTN_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(ATTN_ERR_DIM, "workspace of %zu bytes, %zu needed", ws_bytes, need);
  const int64_t rows = (int64_t)P.B * P.H * P.N;
  const int64_t units = (int64_t)P.B * P.H * ((P.N + kRows - 1) / kRows) * splits;
  if (units + 8 > INT32_MAX || rows + 4 > INT32_MAX) return fail(ATTN_ERR_DIM, "too many split units or rows");
  const size_t q_bytes = (size_t)rows * P.d * 2, kv_bytes = (size_t)rows / P.H * P.Hkv * P.d * 2;
  const size_t o_bytes = (size_t)rows * P.d * (o2.o_dtype == ATTN_O_F32 ? 4 : 2);
  const void* others[5] = {P.q, P.k, P.v, P.o, P.lse};
  const size_t other_bytes[5] = {q_bytes, kv_bytes, kv_bytes, o_bytes, (size_t)rows * 4};
  for (int i = 0; i < 5; ++i)
    if (overlaps(ws, need, others[i], other_bytes[i])) return fail(ATTN_ERR_ALIAS, "workspace overlaps a tensor");

  attn::Params p;
  p.q = (const __bf16*)P.q;
  p.k = (const __bf16*)P.k;
  p.v = (const __bf16*)P.v;
  p.o = P.o;
  p.lse = P.lse;
  p.rescale_count = nullptr;
  p.cu_seqlens = nullptr;
  p.nseq = 0;
  p.N = P.N;
  p.H = P.H;
  p.G = P.H / P.Hkv;
  p.nq_tiles = (P.N + kRows - 1) / kRows;
  p.total_tiles = (int)units;
  p.n_xcd = attn_host::device_shape().xcds;
  p.per_xcd = (p.total_tiles + p.n_xcd - 1) / p.n_xcd;
  p.c = P.scale * 1.44269504088896341f;
  if (p.c == 0.f) p.c = 0x1p-100f;
  p.tau = o2.rescale_tau_log2;
  p.psum_thr = (1.f - 0x1p-10f) * exp2f(o2.rescale_tau_log2);  // P above 2^tau puts a partial sum above this
  p.n_splits = splits;
  p.split_tiles = split_tiles;
  p.ws_o = (float*)ws;
  p.ws_lse = (float*)((char*)ws + (splits * (size_t)rows * P.d * 4 + 255) / 256 * 256);
  p.split_stride = (size_t)rows;
  const bool ref = o2.schedule == ATTN_SCHEDULE_REFERENCE;
  const bool of32 = o2.o_dtype == ATTN_O_F32;
  const bool neg = P.scale < 0.f;
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (P.d == 128)
    e = causal ? attn_launch::launch_split<128, true>(p, neg, of32, (int)rows, ref, s)
               : attn_launch::launch_split<128, false>(p, neg, of32, (int)rows, ref, s);
  else
    e = causal ? attn_launch::launch_split<64, true>(p, neg, of32, (int)rows, ref, s)
               : attn_launch::launch_split<64, false>(p, neg, of32, (int)rows, ref, s);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ATTN_OK;
}

Problem dense(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H, int Hkv,
              int N, int d, float scale) {
  return Problem{q, k, v, const_cast<void*>(o), const_cast<float*>(lse), nullptr, false, B, H, Hkv, N, 0, d, scale};
}

Problem packed(const void* q, const void* k, const void* v, const void* o, const float* lse, const int* cu, int B,
               int H, int Hkv, int total, int max_seqlen, int d, float scale) {
  return Problem{q, k, v, const_cast<void*>(o), const_cast<float*>(lse), cu, true, B, H, Hkv, total, max_seqlen, d, scale};
}

// Scratch of attn_fwd_splitkv_noalloc: a file-scope device array that every GPU
// the library runs on holds until the process ends. In host code its name is a
// host-side stand-in, not a device address; host code only ever uses the address
// hipGetSymbolAddress returns on the device that is current, kept per device.
static __device__ __align__(256) char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

// Device address of this device's scratch array (nullptr and a message on error),
// looked up once per device on its first use.
void* scratch_address() {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    fail(ATTN_ERR_HIP, "no current device for the scratch array");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      fail(ATTN_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      return nullptr;
    }
    addr[dev] = ptr;
  }
  return addr[dev];
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
  attn_fwd_opts def;
  bool work;
  return validate(dense(q, k, v, o, lse, B, H, H, N, d, scale), opts, &def, &work);
}

attn_status_t attn_fwd_gqa_check(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                 int B, int H, int Hkv, int N, int d, int causal, float scale,
                                 const attn_fwd_opts* opts) {
  (void)causal;
  attn_fwd_opts def;
  bool work;
  return validate(dense(q, k, v, o, lse, B, H, Hkv, N, d, scale), opts, &def, &work);
}

attn_status_t attn_fwd_varlen_check(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                    const int* cu_seqlens, int B, int H, int Hkv, int total, int max_seqlen, int d,
                                    int causal, float scale, const attn_fwd_opts* opts) {
  (void)causal;
  attn_fwd_opts def;
  bool work;
  return validate(packed(q, k, v, o, lse, cu_seqlens, B, H, Hkv, total, max_seqlen, d, scale), opts, &def, &work);
}

attn_status_t attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                          int N, int d, int causal, float scale, const attn_fwd_opts* opts, void* stream) {
  return run(dense(q, k, v, o, lse, B, H, H, N, d, scale), causal, opts, stream);
}

attn_status_t attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                           int Hkv, int N, int d, int causal, float scale, const attn_fwd_opts* opts,
                           void* stream) {
  return run(dense(q, k, v, o, lse, B, H, Hkv, N, d, scale), causal, opts, stream);
}

size_t attn_fwd_splitkv_workspace_size(int B, int H, int N, int d, int n_splits) {
  if (B <= 0 || H <= 0 || N <= 0 || (d != 64 && d != 128) || n_splits < 0 || n_splits > 1024) return 0;
  int splits, split_tiles;
  split_shape(B, H, N, d, n_splits, &splits, &split_tiles);
  return split_workspace_bytes(B, H, N, d, splits);
}

attn_status_t attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                       int H, int Hkv, int N, int d, int causal, float scale, int n_splits,
                                       const attn_fwd_opts* opts, void* stream) {
  const Problem P = dense(q, k, v, o, lse, B, H, Hkv, N, d, scale);
  // sizes the check in run_split rejects get no scratch lookup either
  const size_t need = attn_fwd_splitkv_workspace_size(B, H, N, d, n_splits);
  if (need > ATTN_NOALLOC_SCRATCH_BYTES)
    return fail(ATTN_ERR_DIM, "split-key partials need %zu bytes; the library's scratch holds %zu", need,
                (size_t)ATTN_NOALLOC_SCRATCH_BYTES);
  // need == 0 only for invalid or empty sizes: run_split then reports the
  // argument error (or does nothing) before it would look at the workspace
  void* ws = need ? scratch_address() : nullptr;
  if (need && !ws) return ATTN_ERR_HIP;
  return run_split(P, causal, n_splits, ws, ATTN_NOALLOC_SCRATCH_BYTES, opts, stream);
}
attn_status_t attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                               int Hkv, int N, int d, int causal, float scale, int n_splits, void* workspace,
                               size_t workspace_bytes, const attn_fwd_opts* opts, void* stream) {
  return run_split(dense(q, k, v, o, lse, B, H, Hkv, N, d, scale), causal, n_splits, workspace, workspace_bytes,
                   opts, stream);
}

attn_status_t attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                              const int* cu_seqlens, int B, int H, int Hkv, int total, int max_seqlen, int d,
                              int causal, float scale, const attn_fwd_opts* opts, void* stream) {
  return run(packed(q, k, v, o, lse, cu_seqlens, B, H, Hkv, total, max_seqlen, d, scale), causal, opts, stream);
}

attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                       int d, int causal, float scale, void* stream) {
  return attn_fwd_ex(q, k, v, o, lse, B, H, N, d, causal, scale, nullptr, stream);
}

const char* attn_status_str(int s) {
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
