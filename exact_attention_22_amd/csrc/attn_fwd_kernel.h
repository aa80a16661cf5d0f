// attn_fwd_kernel.h - tiled exact-attention forward kernel for gfx950 (MI355X).
//
// One workgroup computes 256 query rows of one (batch, head); each of its 8
// wavefronts owns 32 rows. With grouped-query attention the head's keys and
// values are those of the key/value head its group of query heads shares. The keys and values stream through LDS in
// tiles of BC rows, the queries stay in registers, and per query row the kernel
// keeps a running maximum and running sum, so the N x N score matrix never
// leaves the chip (page "Flash Attention" glossary, sections "Tiling with SRAM"
// and "Online softmax and recomputation"; page "FlashAttention 4: faster, more
// memory-efficient attention for LLMs", sections "Why attention kernels still
// dominate LLM cost" and "What's new in FlashAttention 4").
//
// Both products run on the bf16 matrix cores, v_mfma_f32_32x32x16_bf16, in a
// transposed form chosen for the CDNA register layout:
//   S^T = K . Q^T   (M = 32 keys, N = 32 queries, K = head dim)
//   O^T += V^T . P^T (M = 32 value features, N = 32 queries, K = keys)
// In the 32x32 accumulator layout lane l holds column n = l % 32 and rows
// 8*(r/4) + 4*(l/32) + r%4 of register r. With queries on the columns, every
// lane owns ONE query row: the row maximum and row sum are in-lane reductions
// plus one exchange with lane l^32 (v_permlane32_swap), and the rescale of the
// output accumulator is a per-lane scalar multiply. The probabilities P^T come
// out of the first product already in the B-operand layout of the second one
// (lane l: column l%32, eight consecutive k-slots); the eight keys a lane holds
// for one k-step are {16h + 8*(j/4) + 4*(l/32) + j%4 : j = 0..7}. The matching
// A operand (value feature l%32, those eight keys) is a column read of the
// row-major V tile: gfx950's LDS transpose read ds_read_b64_tr_b16 gives it in
// two instructions. Within each group of 16 lanes, output lane i, element e is
// the 16-bit word at (address supplied by lane 4e + i/4) + (i%4) words, so lane
// i supplies the address of key row i/4 and value-feature quad i%4 and receives
// four consecutive keys of one value feature.
//
// Data movement: K and V tiles go from HBM/L2 straight into LDS with buffer
// loads that write LDS (each wave instruction fills 1 KiB: lane l's 16 bytes
// land at base + 16*l), double-buffered (V as a head and a tail, see VSplit).
// Rows are stored unpadded with an XOR swizzle of their 16-byte chunks, chosen
// so that both the 16-byte K reads and the V transpose reads are free of bank
// conflicts. Keys past N read as zeros (buffer range check) and are masked.
// Every LDS read is issued by the wavefront in its matrix phase, under its own
// products: on gfx950 an LDS read occupies the issuing wavefront for about
// (bytes / 64) cycles but does not slow a matrix-core wavefront on the same
// SIMD, so reads in the softmax phase would lengthen the critical path.
//
// Schedule: a workgroup holds two groups of four wavefronts (one of each per
// SIMD) that alternate, one phase apart, between the softmax of tile t on the
// VALU and the matrix work (O += P_t V_t, S_{t+1} = K_{t+1} Q^T), so every SIMD
// keeps one wavefront feeding the matrix core while the other computes
// exponentials (see the ping-pong section below). This is the CDNA form of the
// overlap the pages obtain with warp specialisation and asynchronous MMA (page
// "FlashAttention 4: faster, more memory-efficient attention for LLMs",
// section "What's new in FlashAttention 4"; page "FlashAttention-4:
// algorithm-kernel fused pipeline for asymmetric hardware scaling", section 2).
//
// Online softmax with the adaptive rescale of page "FlashAttention 4: faster,
// more memory-efficient attention for LLMs", section "Smarter online softmax
// rescaling (new in FA4)": scores are taken in base 2, x = s * c with
// c = scale * log2(e) in fp32 (the scale is never folded into bf16 Q); the
// maximum in use m only moves when a tile's maximum exceeds it by more than
// tau, and then the partial sum and the output accumulator are rescaled by
// 2^(m_old - m_new). Otherwise P = 2^(x - m) may exceed 1 (by at most 2^tau),
// which fp32 accumulation and bf16 P hold without loss of range. The final
// O = acc / l and LSE = ln 2 * (m + log2 l) are written once.
#ifndef ATTN_FWD_KERNEL_H
#define ATTN_FWD_KERNEL_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "exp2_poly.h"


namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct Params {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  void* o;
  float* lse;
  int* rescale_count;  // optional, one int32 per output row
  const int* cu_seqlens;  // packed batches: nseq + 1 cumulative sequence lengths (device)
  int nseq;            // packed batches: number of sequences
  int N;               // rows of one head in memory: the sequence length, or the packed total
  int H;               // query heads
  int G;               // query heads per key/value head (H / Hkv; 1 = multi-head)
  int nq_tiles;        // ceil(N / BR); packed batches: ceil(longest sequence / BR)
  int total_tiles;     // B * H * nq_tiles; packed batches: H * nseq * nq_tiles
  int n_xcd;           // XCDs of the device (workgroup slot v runs on XCD v % n_xcd)
  int per_xcd;         // ceil(total_tiles / n_xcd): tiles per XCD slice
  float c;             // scale * log2(e) in fp32; +-2^-100 stands in for 0 (see the launcher)
  float tau;           // rescale threshold, log2 units
  float psum_thr;      // 2^tau * (1 - 2^-10): partial tile sums above it take the exact-maximum path
  // split keys: tile (bh, qt) is n_splits units, unit s covering key tiles
  // [s * split_tiles, (s + 1) * split_tiles); each writes its normalised O and LSE
  // over those keys to ws_o [n_splits][B*H*N][D] and ws_lse [n_splits][B*H*N]
  int n_splits;
  int split_tiles;
  float* ws_o;
  float* ws_lse;
  size_t split_stride;  // B * H * N rows
};

// Buffer resource over `bytes` bytes at `base`: raw loads at byte offsets >= bytes
// return zeros, which zero-fills the rows past N with no branch. The third
// descriptor word selects 32-bit data format (DATA_FORMAT = 4 in bits 15..18),
// which raw untyped loads require on gfx9-family parts.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// LDS layout of a K or V tile: BC rows of D bf16 (2*D bytes), no padding; the
// 16-byte chunk c of row r is stored at chunk position c ^ swizzle(r).
// K is read 16 bytes per lane with 16 consecutive rows in each 16-lane phase:
// the swizzle gives those rows 16 distinct bank groups. V is read with the
// transpose read: each 32-lane phase touches rows r0..r0+3 (r0 % 4 == 0) and
// four consecutive chunks; the swizzle spreads them over all 64 banks.
template <int D>
__device__ __forceinline__ int kswz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int vswz(int r) {
  return D == 128 ? (4 * (r & 3)) : (4 * ((r >> 1) & 1));
}

// Loads of one BC-row tile of K or V into an LDS tile buffer by NW wavefronts.
// Each wave instruction fills 1 KiB (RPL consecutive rows); wave-load i of
// wavefront w covers rows RPL*(NW*i + w) .. +RPL-1. With that assignment the
// row's swizzle does not depend on i, so wave-load i reads at the per-lane byte
// offset of load 0 plus i*STEP (load_offsets, fixed for the whole kernel). One
// buffer resource per tile ends at row N, so rows past N read as zeros with no
// per-load arithmetic. (Free functions: a device member function calling these
// builtins breaks the kernel's host-side stub.)
template <int D, int BC, int NW>
struct LoadShape {
  static constexpr int CH = D / 8;            // 16-byte chunks per row
  static constexpr int RPL = 64 / CH;         // rows per wave-load
  static constexpr int LPW = BC / RPL / NW;   // wave-loads per wave
  static constexpr int STEP = RPL * NW * D * 2;  // bytes between a wavefront's loads
  static_assert(BC % (RPL * NW) == 0, "load split");
};

template <int D, int BC, int NW, bool ISK>
__device__ __forceinline__ void load_offsets(uint32_t* off, int wave, int lane) {  // off: LoadShape::LPW entries
  using S = LoadShape<D, BC, NW>;
  const int r = wave * S::RPL + lane / S::CH;  // row of load 0; load i adds RPL*NW*i rows
  const int c = (lane % S::CH) ^ (ISK ? kswz<D>(r) : vswz<D>(r));
#pragma unroll
  for (int i = 0; i < S::LPW; ++i) off[i] = (uint32_t)(r * D + 8 * c) * 2 + (uint32_t)(i * S::STEP);
}

// A tile that is not `live` (past the last tile, or starting at or past row N)
// gets a zero-size resource: its loads fill the buffer with zeros without
// touching memory, so every step issues the same loads and the load/wait
// sequence has no branches.
template <int D, int BC, int NW>
__device__ __forceinline__ void load_tile(const uint32_t* off, const __bf16* head, int N, int j0, char* buf, int wave,
                                          bool live) {  // off: LoadShape::LPW per-load offsets
  using S = LoadShape<D, BC, NW>;
  live = live && j0 < N;
  const char* base = (const char*)(head + (size_t)(live ? j0 : 0) * D);
  // readfirstlane keeps the (uniform) record count in a scalar register: a
  // resource in vector registers would need a loop over lanes.
  const uint32_t rec = __builtin_amdgcn_readfirstlane(live ? (uint32_t)(N - j0) * D * 2 : 0u);
  const __amdgpu_buffer_rsrc_t rsrc = buffer_rsrc(base, rec);
#pragma unroll
  for (int i = 0; i < S::LPW; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(buf + (NW * i + wave) * 1024), 16, off[i], 0, 0, 0);
}

// K fragment (A operand of S^T = K Q^T): row R, 16-byte chunk c.
template <int D>
__device__ __forceinline__ bf16x8 k_frag(const char* kb, int R, int c) {
  return *(const bf16x8*)(kb + R * (2 * D) + ((c ^ kswz<D>(R)) << 4));
}
// Per-lane byte offsets of the K fragments of k-step kk for key row l32 of a
// 32-row chunk (the chunk's 32*cc rows add a compile-time offset, which keeps
// the swizzle since 32*cc does not change the row modulo 16); computed once per
// kernel so that each fragment read is one instruction with an immediate offset.
template <int D>
__device__ __forceinline__ void k_offsets(int (&koffs)[D / 16], int lane) {
  const int l32 = lane & 31, hl = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) koffs[kk] = l32 * (2 * D) + (((2 * kk + hl) ^ kswz<D>(l32)) << 4);
}
template <int D>
__device__ __forceinline__ bf16x8 k_frag_at(const char* kb, int off, int cc) {
  return *(const bf16x8*)(kb + off + cc * 32 * (2 * D));
}

// Transpose-read addressing of the swizzled V tile. For value-feature block mt,
// lane l (16-lane group g, index i) reads key rows row0 + i/4 with
// row0 = 32*cc + 16*h + 4*(g/2) (+ 8 for the second read) and value features
// 32*mt + 16*(g%2) + 4*(i%4) .. +3. The swizzle only depends on the row modulo 4
// (D = 128) or 4 (D = 64: (row/2)%2), which cc, h and the +8 do not change, so
// the byte offset is a per-lane part (v_offsets, once per kernel) plus a
// compile-time row offset folded into the instruction.
template <int D>
__device__ __forceinline__ void v_offsets(int (&voffs)[D / 32], int lane) {
  const int i = lane & 15, g = lane >> 4;
  const int r = 4 * (g >> 1) + (i >> 2);  // row within a 16-row block
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) {
    const int dv = 32 * mt + 16 * (g & 1) + 4 * (i & 3);
    voffs[mt] = r * (2 * D) + (((dv >> 3) ^ vswz<D>(r)) << 4) + ((dv & 7) << 1);
  }
}
// Four consecutive keys of one value feature (see v_offsets); `rows` is the
// compile-time row offset 32*cc + 16*h (+8).
template <int D>
__device__ __forceinline__ s16x4 v_col4(const char* vrow, int rows) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(lds_void*)(vrow + rows * (2 * D)));
}

// Max / min / sum of a value with its copy in lane l^32 (the other half of the same query row).
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_min(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Part of S^T = K Q^T for the K tile in `kb`: the MFMAs with flat index
// cc * (D/16) + kk in [F0, F1) (chunk cc of 32 keys, k-step kk); a chunk's chain
// starts from zero at kk = 0.
template <int D, int NC, int F0, int F1>
__device__ __forceinline__ void qk_part(const char* kb, const bf16x8 (&qreg)[D / 16], f32x16 (&s)[NC],
                                        const int (&koffs)[D / 16]) {
  constexpr int KK = D / 16;
#pragma unroll
  for (int f = F0; f < F1; ++f) {
    const int cc = f / KK, kk = f % KK;
    if (kk == 0) s[cc] = f32x16{};
    s[cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag_at<D>(kb, koffs[kk], cc), qreg[kk], s[cc], 0, 0, 0);
  }
}

// PV operands (V^T fragments) of k-steps [G0, G1): k-step g = 2*cc + h covers
// keys 32*cc + 16*h .. +15; one fragment per value-feature block mt.
template <int D, int BC, int G0, int G1>
__device__ __forceinline__ void v_read(bf16x8 (&va)[BC / 32][2][D / 32], const char* vb, const int (&voffs)[D / 32]) {
#pragma unroll
  for (int g = G0; g < G1; ++g)
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) {
      const int cc = g / 2, h = g % 2;
      const s16x4 lo = v_col4<D>(vb + voffs[mt], 32 * cc + 16 * h);
      const s16x4 hi = v_col4<D>(vb + voffs[mt], 32 * cc + 16 * h + 8);
      va[cc][h][mt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
}

// Running softmax state of the 32 query rows of a wavefront (one row per lane pair).
template <int D>
struct RowState {
  f32x16 oacc[D / 32];  // O^T accumulator (unnormalised)
  float m_used;          // maximum in use, log2 units
  float thr;             // m_used + tau: a tile maximum above it triggers a rescale
  float psum_thr;        // 2^tau less a margin: a tile's partial sum above it may need a rescale
  float l_sum;           // this lane's partial row sum
  int n_rescale;
};

// ============================================================================
// Ping-pong schedule: one workgroup of 8 wavefronts (two per SIMD, 256 query
// rows). Group A (wavefronts 0-3) and group B (4-7) run the same per-tile
// sequence - a VALU phase (softmax of tile t: S_t -> P_t) and a matrix phase
// (O += P_t V_t, then S_{t+1} = K_{t+1} Q^T) - offset by one phase, with a
// workgroup barrier between phases. Wavefronts are dealt to the SIMDs
// round-robin, so every SIMD holds one wavefront of each group and always has
// one of them feeding the matrix core while the other runs the softmax.
//
// Global step 2k:   A: softmax(k)                 B: matrix(k-1)
// Global step 2k+1: A: loads tiles; matrix(k)     B: softmax(k)
// Each group runs pairs (softmax(k), matrix(k)), so the PV operands and P of a
// tile live within one pair; group B starts with an empty step and group A ends
// with one. All LDS reads are issued in the matrix phases. Group A issues the
// tile loads in its matrix phase and waits for them at the end of its next
// softmax phase, before the barrier ending that step.
//
// Which steps end at a barrier depends on the head dim. Only the barriers after
// even steps are needed for the LDS buffers (see the main loop); at d = 128 the
// kernel has just those, and each wavefront's own order (A: matrix then
// softmax, B: softmax then matrix) keeps the two groups of a SIMD in opposite
// phases between them, give or take the difference of the phase lengths, while
// no wavefront waits for the slowest SIMD halfway. At d = 64 the matrix phase
// is much shorter than the softmax phase, and without a barrier after every
// step the two softmax phases of a SIMD drift into each other; there every
// step ends at a barrier.
// ============================================================================

// Barrier between phases. It waits for this wavefront's LDS reads and writes
// (lgkmcnt(0)), not for its global->LDS loads in flight: a workgroup release
// fence would also wait for those (they write LDS), which would serialise the
// loads with the phase that issued them. The loading wavefronts instead wait
// for their previous step's loads explicitly before this barrier. The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void phase_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Per-phase clock instrumentation, compiled in only with -DATTN_PHASE_CLOCKS (the
// micro/phase_clocks.py tool builds such a library). Each wavefront sums, over its
// tiles, the shader-clock cycles of its softmax phase, of the wait at the barrier
// that ends it, of its matrix phase and of the wait at the barrier after that,
// and stores the sums (with its tile count, total cycles and group) in place of
// the rescale counts: 8 int32 per wavefront at (blockIdx.x * 8 + wave) * 8.
struct PhaseClock {
#ifdef ATTN_PHASE_CLOCKS
  uint64_t acc[4] = {0, 0, 0, 0};
  uint64_t prev = 0, begin = 0;
  int tiles = 0;
#endif
  __device__ __forceinline__ void start() {
#ifdef ATTN_PHASE_CLOCKS
    begin = prev = __builtin_amdgcn_s_memtime();
#endif
  }
  __device__ __forceinline__ void restart() {
#ifdef ATTN_PHASE_CLOCKS
    prev = __builtin_amdgcn_s_memtime();
#endif
  }
  // The phase since the last mark ends here; f waits at the barrier that follows it.
  template <int I, class F>
  __device__ __forceinline__ void phase_then(F&& f) {
#ifdef ATTN_PHASE_CLOCKS
    const uint64_t a = __builtin_amdgcn_s_memtime();
    f();
    const uint64_t b = __builtin_amdgcn_s_memtime();
    acc[I] += a - prev;
    acc[I + 1] += b - a;
    prev = b;
    tiles += I == 2;
#else
    f();
#endif
  }
  __device__ __forceinline__ void store(int* out, int slot, int wave, int lane, int grp) {
#ifdef ATTN_PHASE_CLOCKS
    if (out && lane == 0) {
      int* o = out + (slot * 8 + wave) * 8;
      for (int i = 0; i < 4; ++i) o[i] = (int)acc[i];
      o[4] = tiles;
      o[5] = (int)(__builtin_amdgcn_s_memtime() - begin);
      o[6] = grp;
      o[7] = 0;
    }
#endif
  }
};

// Score halves U0 .. U1-1 of a tile (half u = 2 cc + h: registers 8h .. 8h+7 of
// score block cc, one k-step of the PV product): mask keys >= N and (causal) keys
// after the query (on boundary tiles), and P = 2^(s*c - m) with m the maximum in
// use, packed to bf16 in the PV operand order; returns this lane's partial sum of
// those halves. Two partial sums keep the additions off one dependency chain.
template <int BC, bool CAUSAL, bool NEG, int U0, int U1>
__device__ __forceinline__ void mask_blocks(f32x16 (&s)[BC / 32], bool masked, int j0, int N, int my_q, int lane) {
  constexpr float mask_val = NEG ? INFINITY : -INFINITY;
  const int hl = lane >> 5;
  if (masked) {
#pragma unroll
    for (int u = U0; u < U1; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int cc = u / 2, r = 8 * (u % 2) + j;
        const int key = j0 + 32 * cc + 8 * (r / 4) + 4 * hl + (r % 4);
        const bool hide = key >= N || (CAUSAL && key > my_q);
        s[cc][r] = hide ? mask_val : s[cc][r];
      }
  }
}
template <int BC, int POLY8, int U0, int U1>
__device__ __forceinline__ float exp_blocks(const f32x16 (&s)[BC / 32], bf16x8 (&pb)[BC / 32][2], float c, float mc) {
  float part[2] = {0.f, 0.f};
#pragma unroll
  for (int u = U0; u < U1; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int cc = u / 2, h = u % 2, r = 8 * h + j;
        const float x = fmaf(s[cc][r], c, mc);
        float e;
        if (POLY8 == 8 || (POLY8 == 4 && (r & 4)))
          e = attn_exp2_poly(x);
        else
          e = __builtin_amdgcn_exp2f(x);
        part[j & 1] += e;
        pb[cc][h][j] = (__bf16)e;
      }
  // pack here: otherwise the packing sinks past the rescale check and keeps every
  // fp32 exponential live until then
#pragma unroll
  for (int u = U0; u < U1; ++u) asm volatile("" : "+v"(pb[u / 2][u % 2]));
  return part[0] + part[1];
}

// At d = 64 the matrix phase (16 products) is much shorter than the softmax phase,
// so the exponentials of a tile's first score half are taken at the end of the
// matrix phase that computes the scores (PRE = 1 of the 2 NC halves), which
// balances the two wavefronts of a SIMD; at d = 128 the softmax phase takes the
// whole tile.
template <int D>
struct ExpSplit {
  static constexpr int PRE = D == 64 ? 1 : 0;
};

// VALU phase: mask (boundary tiles), adaptive rescale, P = 2^(s*c - m) with the
// fp32 row sum, packed to bf16 in the PV operand order. Score halves below PRE were
// masked and exponentiated with the same maximum at the end of the previous
// matrix phase; t_pre is their partial sum. The phase issues no LDS
// reads: an LDS read holds its own wavefront's issue for about (bytes / 64)
// cycles, which the matrix phase hides under its products and this phase cannot.
template <int D, int BC, bool CAUSAL, int POLY8, bool NEG>
__device__ __forceinline__ void softmax_phase(RowState<D>& st, f32x16 (&s)[BC / 32], bf16x8 (&pb)[BC / 32][2],
                                              bool masked, int j0, int N, int my_q, int lane, float c, float tau,
                                              float t_pre) {
  constexpr int NC = BC / 32;
  constexpr int MT = D / 32;
  constexpr int PRE = ExpSplit<D>::PRE;
  mask_blocks<BC, CAUSAL, NEG, PRE, 2 * NC>(s, masked, j0, N, my_q, lane);
  // The tile maximum is needed only when a rescale may be due: a row whose
  // tile maximum exceeds m + tau has a P above 2^tau, so the partial sum of the
  // lane holding that key exceeds 2^tau (the sum of non-negative terms is at
  // least each term). The exponentials are therefore taken with the maximum in
  // use first, and only a wavefront with such a sum (or with m still -inf,
  // which gives +inf or NaN) computes the exact tile maximum, applies the
  // threshold rule per row and takes the exponentials again. The rescale policy
  // is unchanged; its maximum reduction leaves the common path.
  float tsum = exp_blocks<BC, POLY8, PRE, 2 * NC>(s, pb, c, -st.m_used);
  if (PRE > 0) tsum = t_pre + tsum;
  if (__any(!(tsum <= st.psum_thr))) {
    float red = s[0][0];
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
#pragma unroll
      for (int r = 0; r < 16; ++r) red = NEG ? fminf(red, s[cc][r]) : fmaxf(red, s[cc][r]);
    red = NEG ? pair_min(red) : pair_max(red);
    const float m_tile = red * c;  // -inf when every key of the row is masked (c is never 0)
    const bool need = m_tile > st.thr;
    if (__any(need)) {  // otherwise the exponentials above stand
      const float alpha = need ? __builtin_amdgcn_exp2f(st.m_used - m_tile) : 1.f;
      st.n_rescale += (need && st.m_used != -INFINITY) ? 1 : 0;
      st.m_used = need ? m_tile : st.m_used;
      st.thr = st.m_used + tau;
      st.l_sum *= alpha;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.oacc[mt][r] *= alpha;
      tsum = exp_blocks<BC, POLY8, 0, 2 * NC>(s, pb, c, -st.m_used);
    }
  }
  st.l_sum += tsum;
  // P is consumed only after the phase barrier and the row sum only at the next
  // rescale; these empty asm uses keep both computed in this phase instead of
  // letting them sink past the barrier (which would keep the fp32 exponentials
  // live through the matrix phase).
#pragma unroll
  for (int cc = 0; cc < NC; ++cc)
#pragma unroll
    for (int h = 0; h < 2; ++h) asm volatile("" ::"v"(pb[cc][h]));
  asm volatile("" : "+v"(st.l_sum));
}

// V tiles are stored as a head (the first VHK k-steps of 16 keys: 4 PV operands
// per lane) and a tail (the other keys), each in its own double buffer. The head
// of a tile is read one matrix phase ahead and carried in registers, so the
// first PV products of a matrix phase never wait for LDS; the tail is read
// during the same phase's products, one k-step ahead of its use.
template <int D>
struct VSplit {
  static constexpr int MT = D / 32;
  static constexpr int HKS = 4 / MT;       // head k-steps (4 operands per lane)
  static constexpr int HROWS = 16 * HKS;   // head keys
  static_assert(4 % MT == 0, "head of whole k-steps");
};

// PV operand of value-feature block mt for k-step ks of a V head or tail buffer:
// two transpose reads (see v_offsets).
template <int D>
__device__ __forceinline__ bf16x8 v_operand(const char* buf, int ks, int mt, const int (&voffs)[D / 32]) {
  const s16x4 lo = v_col4<D>(buf + voffs[mt], 16 * ks);
  const s16x4 hi = v_col4<D>(buf + voffs[mt], 16 * ks + 8);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Number of LDS reads issued after PV product (g, mt) of matrix_phase.
template <int D, int BC, int KA>
__host__ __device__ constexpr int pv_reads(int g, int mt) {
  constexpr int NKS = BC / 16, HKS = VSplit<D>::HKS;
  return 2 * (g + 1 >= HKS && g + 1 < NKS) + 2 * (g >= NKS - HKS) + (g == NKS - 1 && mt < KA);
}
template <int D, int BC, int KA, int I>
__device__ __forceinline__ void pv_sched() {
  constexpr int MT = D / 32, NPV = (BC / 16) * MT;
  if constexpr (I < NPV) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, pv_reads<D, BC, KA>(I / MT, I % MT), 0);
    pv_sched<D, BC, KA, I + 1>();
  }
}

// Matrix phase: O^T += V_t^T P_t^T, then S_{t+1} = K_{t+1} Q^T. V_t's head
// operands come in `va`; the LDS reads of this phase ride under the products:
// after PV product (g, mt), the transpose reads of V_t's tail operand (g+1, mt)
// (from `vtl`) or, in the last VHK k-steps, of V_{t+1}'s head operand (from
// `vhd_next`, into `va` for the next matrix phase), and the first KA K_{t+1}
// fragments after the last k-step's products; each QK product is followed by
// the K fragment KA ahead. `loads` issues this wavefront's tile loads (if any),
// one per product in the second half of the QK products. After a wavefront's
// last tile the buffers hold stale data; that S and those operands are never
// used.
template <int D, int BC, int NLOADS, typename Loads, typename AfterQK>
__device__ __forceinline__ void matrix_phase(RowState<D>& st, f32x16 (&s)[BC / 32], const bf16x8 (&pb)[BC / 32][2],
                                             bf16x8 (&va)[VSplit<D>::HKS][D / 32], const bf16x8 (&qreg)[D / 16],
                                             const char* kb, const char* vtl, const char* vhd_next,
                                             const int (&voffs)[D / 32], const int (&koffs)[D / 16], int lane,
                                             Loads&& loads, AfterQK&& after_qk) {
  constexpr int NC = BC / 32;
  constexpr int MT = D / 32;
  constexpr int KK = D / 16;
  constexpr int NKS = BC / 16;      // k-steps of 16 keys
  constexpr int HKS = VSplit<D>::HKS;
  constexpr int NQK = NC * KK;      // QK products
  constexpr int KA = MT < 4 ? MT : 4;  // K fragments read ahead of the QK products
  static_assert(NLOADS <= NQK - KA, "one tile load per late QK product");
  // Issue priority up while this wavefront feeds the matrix core, so the
  // softmax wavefront on the same SIMD does not delay its MFMA issue.
  __builtin_amdgcn_s_setprio(1);
  bf16x8 kf[NQK];
  bf16x8 vf[NKS][MT];
  auto vfrag = [&](const char* buf, int ks, int mt) { return v_operand<D>(buf, ks, mt, voffs); };
  auto kread = [&](int f) { kf[f] = k_frag_at<D>(kb, koffs[f % KK], f / KK); };
#pragma unroll
  for (int g = 0; g < HKS; ++g)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) vf[g][mt] = va[g][mt];
#pragma unroll
  for (int g = 0; g < NKS; ++g)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      st.oacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[g][mt], pb[g / 2][g % 2], st.oacc[mt], 0, 0, 0);
      if (g + 1 >= HKS && g + 1 < NKS) vf[g + 1][mt] = vfrag(vtl, g + 1 - HKS, mt);
      if (g >= NKS - HKS) va[g - (NKS - HKS)][mt] = vfrag(vhd_next, g - (NKS - HKS), mt);
      if (g == NKS - 1 && mt < KA) kread(mt);
    }
#pragma unroll
  for (int f = 0; f < NQK; ++f) {
    const int cc = f / KK, kk = f % KK;
    if (f + KA < NQK) kread(f + KA);
    s[cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[f], qreg[kk], kk == 0 ? f32x16{} : s[cc], 0, 0, 0);
  }
  loads();
  // Instruction order as described above.
  pv_sched<D, BC, KA, 0>();
#pragma unroll
  for (int f = 0; f < NQK - KA - NLOADS; ++f) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
#pragma unroll
  for (int f = 0; f < NLOADS; ++f) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, KA, 0);
  __builtin_amdgcn_s_setprio(0);
  // vector work on the new scores (the first block's exponentials at d = 64)
  after_qk();
}

// O^T += V^T P^T of the reference schedule: the PV products of matrix_phase in
// the same order (k-step by k-step, value-feature block mt within), with every
// operand read from the head and tail buffers beforehand.
template <int D, int BC>
__device__ __forceinline__ void pv_reference(RowState<D>& st, const bf16x8 (&pb)[BC / 32][2], const char* vhd,
                                             const char* vtl, const int (&voffs)[D / 32]) {
  constexpr int NKS = BC / 16, HKS = VSplit<D>::HKS, MT = D / 32;
  bf16x8 vf[NKS][MT];
#pragma unroll
  for (int g = 0; g < NKS; ++g)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) vf[g][mt] = v_operand<D>(g < HKS ? vhd : vtl, g < HKS ? g : g - HKS, mt, voffs);
#pragma unroll
  for (int g = 0; g < NKS; ++g)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      st.oacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[g][mt], pb[g / 2][g % 2], st.oacc[mt], 0, 0, 0);
}

// VARLEN: packed variable-length batches. q and o are [H][total][D], k and v
// [Hkv][total][D], lse [H][total]; sequence b owns tokens cu[b] .. cu[b+1]-1 of
// every head and attends only to itself (causal positions counted from its
// first token). Each tile reads its sequence's bounds; the buffer resources end
// at the sequence's last row, so no load crosses into the next sequence.
// SPLIT: split keys (see Params); requires OF32 (the partial results are fp32).
// REF: the reference schedule, for race checking: the same arithmetic in the
// same order (each wavefront's QK, softmax and PV products of every tile), with
// one buffer per tensor, every tile load issued after a barrier that follows
// all reads of the previous tile and waited for (vmcnt(0) and a barrier) before
// any read, and no phase offset between the wavefront groups. Its results must
// equal the pipelined schedule's bit for bit.
template <int D, int BC, bool CAUSAL, bool OF32, int POLY8, bool NEG, bool VARLEN, bool SPLIT = false,
          bool REF = false>
__global__ void __launch_bounds__(512, 1) attn_fwd_kernel(const Params p) {
  constexpr int NW = 8;            // wavefronts per workgroup (2 per SIMD)
  constexpr int BR = 32 * NW;      // query rows per workgroup
  constexpr int NC = BC / 32;
  constexpr int KK = D / 16;
  constexpr int MT = D / 32;
  constexpr int TILEB = BC * D * 2;
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(!SPLIT || (OF32 && !VARLEN), "split keys: fp32 partials, dense layout");

  // K tiles double-buffered; V tiles as head and tail, each double-buffered (they
  // are read at different steps, see below)
  constexpr int VHR = VSplit<D>::HROWS;  // head keys
  constexpr int VTR = BC - VHR;          // tail keys
  __shared__ __attribute__((aligned(1024))) char kbuf0[TILEB];
  __shared__ __attribute__((aligned(1024))) char kbuf1[TILEB];
  __shared__ __attribute__((aligned(1024))) char vhd0[VHR * D * 2];
  __shared__ __attribute__((aligned(1024))) char vhd1[VHR * D * 2];
  __shared__ __attribute__((aligned(1024))) char vtl0[VTR * D * 2];
  __shared__ __attribute__((aligned(1024))) char vtl1[VTR * D * 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: group A, 1: group B
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  const int N = p.N;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  uint32_t koff[LoadShape<D, BC, 4>::LPW], vhoff[LoadShape<D, VHR, 4>::LPW], vtoff[LoadShape<D, VTR, 4>::LPW];
  load_offsets<D, BC, 4, true>(koff, wave & 3, lane);
  load_offsets<D, VHR, 4, false>(vhoff, wave & 3, lane);
  load_offsets<D, VTR, 4, false>(vtoff, wave & 3, lane);
  int voffs[MT];
  v_offsets<D>(voffs, lane);
  int koffs[KK];
  k_offsets<D>(koffs, lane);
  const float c = p.c;
  const float tau = p.tau;

  // Tile v of the launch's virtual sequence: workgroup slot v runs logical tile
  // (v % X) * per_xcd + v / X with X = n_xcd, so each XCD (slots are dealt
  // round-robin to the X XCDs) works through a contiguous range of tiles and the
  // query tiles of one head share that XCD's L2. A launch with fewer workgroups
  // than slots walks the slots v, v + gridDim.x, ... (gridDim.x is a multiple of
  // X, so a workgroup stays on its XCD's range); the next tile's Q, K_0, V_0 and
  // K_1 loads are then issued before the current tile's epilogue.
  struct Tile {
    int bh, kvh, i0, n_tiles, t_full;  // kvh: the (batch, key/value head) that bh reads
    int n, start;  // packed batches: the sequence's length and first token (bh, kvh: heads)
    int kb, sp;    // split keys: first key tile of the unit, and its split index
  };
  // Causal: a persistent workgroup's successive tiles alternate direction
  // through its XCD's range (round r of S slots takes position i or S-1-i). The
  // range is ordered head by head with the longest query tiles first, so this
  // pairs long tiles with short ones and every workgroup gets about the same
  // work, while the tiles running at the same time stay within few heads (their
  // K and V share the XCD's L2).
  const int X = p.n_xcd;
  const int S = (int)gridDim.x / X;  // workgroups per XCD
  // Packed batches: logical tile (h * nseq + b) * nq_tiles + qt, so an XCD's range
  // holds whole heads with all their sequences (equal work per XCD when X divides
  // H). Slots past a sequence's last query tile are empty (-1) and skipped.
  // Returns 1 for a tile, -1 for an empty slot, 0 past the end of the range.
  auto tile_of = [&](int v, Tile& t) -> int {
    int j = v / X;
    const int x = v - j * X;
    if (CAUSAL) {
      const int r = j / S, i = j - r * S;
      j = r * S + ((r & 1) ? S - 1 - i : i);
    }
    const int logical = x * p.per_xcd + j;
    if (j >= p.per_xcd || logical >= p.total_tiles) return 0;
    int unit = logical;
    if (SPLIT) {  // logical = (bh * nq_tiles + qt) * n_splits + sp
      unit = logical / p.n_splits;
      t.sp = logical - unit * p.n_splits;
    }
    t.bh = unit / p.nq_tiles;
    int qt = unit - t.bh * p.nq_tiles;
    int n = N;
    if (VARLEN) {
      const int h = t.bh / p.nseq, b = t.bh - h * p.nseq;
      // bounds clamped into [0, total]: any contents of cu keep every access in range
      const int a = min(max(p.cu_seqlens[b], 0), N);
      const int e = min(max(p.cu_seqlens[b + 1], a), N);
      t.start = a;
      t.n = n = e - a;
      // a sequence longer than nq_tiles query tiles has its later rows left unwritten
      const int nq = min((n + BR - 1) / BR, p.nq_tiles);
      if (qt >= nq) return -1;
      if (CAUSAL) qt = nq - 1 - qt;  // longest rows first
      t.bh = h;
      t.kvh = h / p.G;
    } else {
      // consecutive groups of G query heads share a key/value head: b*H + h -> b*(H/G) + h/G
      const int b = t.bh / p.H, h = t.bh - b * p.H;
      t.kvh = b * (p.H / p.G) + h / p.G;
      if (CAUSAL) qt = p.nq_tiles - 1 - qt;  // longest rows first
    }
    t.i0 = qt * BR;
    const int kv_end = CAUSAL ? min(n, t.i0 + BR) : n;
    t.n_tiles = (kv_end + BC - 1) / BC;
    t.t_full = n / BC;
    if (CAUSAL) t.t_full = min(t.t_full, (t.i0 + 1) / BC);
    if (SPLIT) {  // key tiles of this unit; units past the tile's last key tile are empty
      t.kb = t.sp * p.split_tiles;
      if (t.kb >= t.n_tiles) return -1;
      t.n_tiles = min(p.split_tiles, t.n_tiles - t.kb);
      t.t_full -= t.kb;
    }
    return 1;
  };
  // The first tile at or after slot v (advancing v past empty slots).
  auto find_tile = [&](int& v, Tile& t) -> bool {
    for (;;) {
      const int r = tile_of(v, t);
      if (!(VARLEN || SPLIT) || r >= 0) return r > 0;
      v += (int)gridDim.x;
    }
  };
  bf16x8 qreg[KK];
  auto issue_loads = [&](const Tile& t) {
    const size_t head = VARLEN ? ((size_t)t.bh * N + t.start) * D : (size_t)t.bh * (size_t)N * D;
    const size_t kvhead = VARLEN ? ((size_t)t.kvh * N + t.start) * D : (size_t)t.kvh * (size_t)N * D;
    const int n = VARLEN ? t.n : N;
    // split keys: K and V start at the unit's first key tile
    const size_t kvoff = kvhead + (SPLIT ? (size_t)t.kb * BC * D : 0);
    const int nkv = n - (SPLIT ? t.kb * BC : 0);
    // K_0, K_1 (group A) and V_0, V_1's head (group B); n_tiles >= 1
    if (REF) {
    } else if (grp == 0) {
      load_tile<D, BC, 4>(koff, p.k + kvoff, nkv, 0, kbuf0, wave & 3, true);
      load_tile<D, BC, 4>(koff, p.k + kvoff, nkv, BC, kbuf1, wave & 3, t.n_tiles > 1);
    } else {
      load_tile<D, VHR, 4>(vhoff, p.v + kvoff, nkv, 0, vhd0, wave & 3, true);
      load_tile<D, VTR, 4>(vtoff, p.v + kvoff, nkv, VHR, vtl0, wave & 3, true);
      load_tile<D, VHR, 4>(vhoff, p.v + kvoff, nkv, BC, vhd1, wave & 3, t.n_tiles > 1);
    }
    const __amdgpu_buffer_rsrc_t qrsrc =
        buffer_rsrc(p.q + head, VARLEN ? (uint32_t)n * D * 2 : head_bytes);
    const int q_row = t.i0 + wave * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qreg[kk] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrsrc, (uint32_t)(q_row * D + 16 * kk + 8 * hl) * 2, 0, 0));
  };

  int slot = blockIdx.x;
  Tile tile;
  if (!find_tile(slot, tile)) return;
  PhaseClock clk;
  clk.start();
  issue_loads(tile);
  for (;;) {
  const int bh = tile.bh;
  const int i0 = tile.i0;
  const int n_tiles = tile.n_tiles;
  const int t_full = tile.t_full;
  // first output row of this (head, sequence) and the rows it has
  const size_t row0 = VARLEN ? (size_t)bh * p.N + tile.start : (size_t)bh * p.N;
  const int N = VARLEN ? tile.n : p.N;
  const int wq0 = i0 + wave * 32;
  const int my_q = wq0 + l32;
  const size_t kvhead = VARLEN ? ((size_t)tile.kvh * p.N + tile.start) * D : (size_t)tile.kvh * (size_t)N * D;
  // split keys: K/V pointers and row count from the unit's first key tile kt0; the
  // masks use absolute key positions ((k + kt0) * BC against N and the query row)
  const int kt0 = SPLIT ? tile.kb : 0;
  const int Nkv = N - kt0 * BC;
  const __bf16* const kh = p.k + kvhead + (size_t)kt0 * BC * D;
  const __bf16* const vh = p.v + kvhead + (size_t)kt0 * BC * D;

  RowState<D> st;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) st.oacc[mt] = f32x16{};
  st.m_used = -INFINITY;
  st.thr = -INFINITY;
  st.psum_thr = p.psum_thr;
  st.l_sum = 0.f;
  st.n_rescale = 0;

  f32x16 s[NC];
  bf16x8 va[VSplit<D>::HKS][MT];  // PV operands of the head of the V tile the next matrix phase multiplies
  bf16x8 pb[NC][2];                // P of the tile in flight, in the PV operand order
  float t_pre = 0.f;               // partial row sum of its first ExpSplit<D>::PRE blocks
  constexpr int PRE = ExpSplit<D>::PRE;
  // the first PRE blocks of tile k's scores: masked and exponentiated right after the
  // products that form them (the previous matrix phase, or the prologue)
  auto pre_blocks = [&](int k) {
    if (PRE > 0) {
      mask_blocks<BC, CAUSAL, NEG, 0, PRE>(s, k >= t_full, (k + kt0) * BC, N, my_q, lane);
      t_pre = exp_blocks<BC, POLY8, 0, PRE>(s, pb, c, -st.m_used);
    }
  };
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wavefront's tile and Q loads landed
  if (REF) {
    // reference schedule: one buffer per tensor, full waits, no phase offset
    for (int k = 0; k < n_tiles; ++k) {
      __syncthreads();  // every wavefront's reads of the previous tile are complete
      if (grp == 0) {
        load_tile<D, BC, 4>(koff, kh, Nkv, k * BC, kbuf0, wave & 3, true);
      } else {
        load_tile<D, VHR, 4>(vhoff, vh, Nkv, k * BC, vhd0, wave & 3, true);
        load_tile<D, VTR, 4>(vtoff, vh, Nkv, k * BC + VHR, vtl0, wave & 3, true);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      qk_part<D, NC, 0, NC * KK>(kbuf0, qreg, s, koffs);
      pre_blocks(k);
      softmax_phase<D, BC, CAUSAL, POLY8, NEG>(st, s, pb, k >= t_full, (k + kt0) * BC, N, my_q, lane, c, tau,
                                               t_pre);
      pv_reference<D, BC>(st, pb, vhd0, vtl0, voffs);
    }
    __syncthreads();
  } else {
  __syncthreads();                      // K_0, K_1, V_0, V_1's head resident for every wavefront
#pragma unroll
  for (int g = 0; g < VSplit<D>::HKS; ++g)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const s16x4 lo = v_col4<D>(vhd0 + voffs[mt], 16 * g);
      const s16x4 hi = v_col4<D>(vhd0 + voffs[mt], 16 * g + 8);
      va[g][mt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  qk_part<D, NC, 0, NC * KK>(kbuf0, qreg, s, koffs);
  pre_blocks(0);
  clk.restart();

  // Every wavefront runs all n_tiles tiles of its workgroup: a tile past a causal
  // row's last visible key is fully masked (P = 0) and leaves m, l and O as they
  // are, so no wavefront takes a separate code path. Tile k's buffers are
  // kbuf[k % 2], vhd[k % 2] and vtl[k % 2]. Both groups pass n_tiles + 1
  // barriers at d = 128 (those ending the even steps) and 2 * n_tiles + 1 at
  // d = 64 (every step).
  //
  // LDS reads: matrix(k) (group A at step 2k+1, group B at step 2k+2) reads
  // V_k's tail, K_{k+1} and V_{k+1}'s head; the softmax phase reads none.
  // Tile loads: group A issues, during matrix(k) (step 2k+1), K_{k+2} into
  // kbuf[k % 2] and V_{k+2}'s head into vhd[k % 2] (K_k and V_k's head were last
  // read by matrix(k-1), steps 2k-1 and 2k), and V_{k+1}'s tail into
  // vtl[(k+1) % 2] (V_{k-1}'s tail was last read by matrix(k-1)). It waits for
  // them at the end of softmax(k+1), before the barrier ending step 2k+2; all
  // three are first read at step 2k+3. Every barrier waits for the wavefront's
  // own LDS reads, so no buffer is overwritten under a read.
  //
  // The barriers ending the even steps suffice for this. Between the barrier
  // ending step 2k and the one ending step 2k+2, the reads are those of
  // matrix(k) in both groups (V_k's tail, K_{k+1}, V_{k+1}'s head), the writes
  // those group A issues in matrix(k) (K_{k+2}, V_{k+2}'s head, V_{k+1}'s tail):
  // different buffers. The buffers written were last read by matrix(k-1), which
  // both groups finish before the barrier ending step 2k; the loads are waited
  // for before the barrier ending step 2k+2, and first read after it.
  constexpr bool EVERY_STEP = D == 64;  // also a barrier after the odd steps
  auto wait_loads = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };  // vmcnt(0)
  // without a barrier: only keep the compiler from moving memory accesses across
  auto odd_step_end = [] {
    if (EVERY_STEP)
      phase_barrier();
    else
      asm volatile("" ::: "memory");
  };
  constexpr int NLD =
      LoadShape<D, BC, 4>::LPW + LoadShape<D, VHR, 4>::LPW + LoadShape<D, VTR, 4>::LPW;  // group A's loads per step
  if (grp == 0) {
    auto pair = [&](int k, char* kb0, char* kb1, char* vh0, char* vh1, char* vt0, char* vt1) {
      softmax_phase<D, BC, CAUSAL, POLY8, NEG>(st, s, pb, k >= t_full, (k + kt0) * BC, N, my_q, lane, c, tau,
                                               t_pre);
      clk.phase_then<0>([&] {
        wait_loads();
        phase_barrier();
      });
      matrix_phase<D, BC, NLD>(st, s, pb, va, qreg, kb1, vt0, vh1, voffs, koffs, lane, [&] {
        load_tile<D, BC, 4>(koff, kh, Nkv, (k + 2) * BC, kb0, wave & 3, k + 2 < n_tiles);
        load_tile<D, VHR, 4>(vhoff, vh, Nkv, (k + 2) * BC, vh0, wave & 3, k + 2 < n_tiles);
        load_tile<D, VTR, 4>(vtoff, vh, Nkv, (k + 1) * BC + VHR, vt1, wave & 3, k + 1 < n_tiles);
      }, [&] { pre_blocks(k + 1); });
      clk.phase_then<2>(odd_step_end);
    };
    int k = 0;
    for (; k + 1 < n_tiles; k += 2) {
      pair(k, kbuf0, kbuf1, vhd0, vhd1, vtl0, vtl1);
      pair(k + 1, kbuf1, kbuf0, vhd1, vhd0, vtl1, vtl0);
    }
    if (k < n_tiles) pair(k, kbuf0, kbuf1, vhd0, vhd1, vtl0, vtl1);
    wait_loads();  // the last steps' loads (past the last tile: zero-size) are done
    phase_barrier();
  } else {
    phase_barrier();  // step 0: group B starts one phase behind
    // Steps 2k+1 (softmax(k)) and 2k+2 (matrix(k)).
    auto pair = [&](int k, char* kb1, char* vh1, char* vt0) {
      softmax_phase<D, BC, CAUSAL, POLY8, NEG>(st, s, pb, k >= t_full, (k + kt0) * BC, N, my_q, lane, c, tau,
                                               t_pre);
      clk.phase_then<0>(odd_step_end);
      matrix_phase<D, BC, 0>(st, s, pb, va, qreg, kb1, vt0, vh1, voffs, koffs, lane, [] {},
                             [&] { pre_blocks(k + 1); });
      clk.phase_then<2>(phase_barrier);
    };
    int k = 0;
    for (; k + 1 < n_tiles; k += 2) {
      pair(k, kbuf1, vhd1, vtl0);
      pair(k + 1, kbuf0, vhd0, vtl1);
    }
    if (k < n_tiles) pair(k, kbuf1, vhd1, vtl0);
  }
  }  // pipelined schedule

  // Every wavefront has passed the last barrier, so no LDS tile and no Q
  // register is read again: the next tile's loads can go out now and land
  // while this tile's output is written.
  Tile next;
  int next_slot = slot + (int)gridDim.x;
  const bool more = find_tile(next_slot, next);
  if (more) issue_loads(next);

  const float l_tot = pair_sum(st.l_sum);
  // split keys: this unit's partial result goes to its workspace slice (a row that
  // sees none of the unit's keys stores a value the merge does not read)
  float* const o_out = SPLIT ? p.ws_o + (size_t)tile.sp * p.split_stride * D : (float*)p.o;
  float* const lse_out = SPLIT ? p.ws_lse + (size_t)tile.sp * p.split_stride : p.lse;
  const float inv = 1.f / l_tot;
  // bf16 output: lanes l and l ^ 32 hold the same row, lane half hl the features
  // 32 mt + 8 gq + 4 hl + e (register 4 gq + e). One lane-half exchange per pair of
  // gq gives each lane 8 consecutive features (gq = 2 pp + hl, 16 bytes), so a row
  // takes 8 stores of 16 bytes per lane instead of 16 of 8 bytes. The exchange
  // runs in every lane (a row past N only skips the stores).
  u32x4 ob[OF32 ? 1 : MT][2];
  if (!OF32) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        bf16x4 a, b;  // gq = 2 pp (kept by hl = 0) and gq = 2 pp + 1 (kept by hl = 1)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = (__bf16)(st.oacc[mt][8 * pp + e] * inv);
          b[e] = (__bf16)(st.oacc[mt][8 * pp + 4 + e] * inv);
        }
        u32x2 x = __builtin_bit_cast(u32x2, a), y = __builtin_bit_cast(u32x2, b);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          // x of the upper lane half <-> y of the lower lane half
          const auto r = __builtin_amdgcn_permlane32_swap(x[j], y[j], false, false);
          x[j] = r[0];
          y[j] = r[1];
        }
        ob[OF32 ? 0 : mt][pp] = u32x4{x[0], x[1], y[0], y[1]};
      }
  }
  if (my_q < N) {
    const size_t row = row0 + my_q;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (OF32) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = st.oacc[mt][4 * gq + e] * inv;
          *(f32x4*)(o_out + row * D + 32 * mt + 8 * gq + 4 * hl) = w;
        }
      } else {
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
          *(u32x4*)((__bf16*)p.o + row * D + 32 * mt + 16 * pp + 8 * hl) = ob[OF32 ? 0 : mt][pp];
      }
    }
    if (hl == 0) {
      lse_out[row] = 0.69314718055994531f * (st.m_used + log2f(l_tot));
#ifndef ATTN_PHASE_CLOCKS
      if (!SPLIT && p.rescale_count) p.rescale_count[row] = st.n_rescale;
#endif
    }
  }
  if (!more) break;
  tile = next;
  slot = next_slot;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load into LDS outlives the workgroup
  clk.store(SPLIT ? nullptr : p.rescale_count, blockIdx.x, wave, lane, grp);
}

// Merge of split-key partial results: for query row i of a head, the units
// s = 0 .. last(i) / split_keys (last(i) = i causal, N - 1 otherwise) hold O_s and
// LSE_s over their keys; LSE = log sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s.
// One wavefront per row (D/64 features per lane), four rows per workgroup.
template <int D, bool CAUSAL, bool OF32>
__global__ void __launch_bounds__(256) attn_merge_kernel(const Params p, int rows_total, int split_keys) {
  constexpr int F = D / 64;  // features per lane
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows_total) return;
  const int i = row % p.N;
  const int last = CAUSAL ? i : p.N - 1;
  const int ns = min(p.n_splits, last / split_keys + 1);
  float m = -INFINITY;
  for (int sp = 0; sp < ns; ++sp) m = fmaxf(m, p.ws_lse[(size_t)sp * p.split_stride + row]);
  float z = 0.f;
  float acc[F];
#pragma unroll
  for (int f = 0; f < F; ++f) acc[f] = 0.f;
  for (int sp = 0; sp < ns; ++sp) {
    const float w = __builtin_amdgcn_exp2f((p.ws_lse[(size_t)sp * p.split_stride + row] - m) * 1.44269504088896341f);
    z += w;
    const float* o = p.ws_o + ((size_t)sp * p.split_stride + row) * D + F * lane;
#pragma unroll
    for (int f = 0; f < F; ++f) acc[f] = fmaf(w, o[f], acc[f]);
  }
  const float inv = 1.f / z;
#pragma unroll
  for (int f = 0; f < F; ++f) {
    if (OF32)
      ((float*)p.o)[(size_t)row * D + F * lane + f] = acc[f] * inv;
    else
      ((__bf16*)p.o)[(size_t)row * D + F * lane + f] = (__bf16)(acc[f] * inv);
  }
  if (lane == 0) p.lse[row] = m + logf(z);
}

}  // namespace attn

#endif
