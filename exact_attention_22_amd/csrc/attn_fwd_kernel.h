// attn_fwd_kernel.h - tiled exact-attention forward kernel for gfx950 (MI355X).
//
// One workgroup computes BR = 32*NW query rows of one (batch, head); each of
// its NW wavefronts owns 32 rows. The keys and values stream through LDS in
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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct Params {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  void* o;
  float* lse;
  int* rescale_count;  // optional [B][H][N] int32
  int N;
  int nq_tiles;        // ceil(N / BR)
  int total_tiles;     // B * H * nq_tiles
  int per_xcd;         // ceil(total_tiles / 8): workgroups per XCD slice
  float c;             // scale * log2(e) in fp32; +-2^-100 stands in for 0 (see the launcher)
  float tau;           // rescale threshold, log2 units
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Four consecutive keys (rows row0 + e, e = 0..3) of value feature col0 + (lane % 16)
// from a row-major LDS tile with a row stride of `stride` elements.
__device__ __forceinline__ s16x4 lds_col4(const __bf16* tile, int stride, int row0, int col0, int lane) {
  const int i = lane & 15;
  const __bf16* p = tile + (row0 + (i >> 2)) * stride + col0 + 4 * (i & 3);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(__attribute__((address_space(3))) void*)p);
}

// Buffer resource over `bytes` bytes at `base`: raw loads at byte offsets >= bytes
// return zeros, which zero-fills the rows past N with no branch. The third
// descriptor word selects 32-bit data format (DATA_FORMAT = 4 in bits 15..18),
// which raw untyped loads require on gfx9-family parts.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Max of a value with its copy in lane l^32 (the other half of the same query row).
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

// One KV tile of the online softmax for the 32 query rows of a wavefront:
// S^T = K Q^T, mask (boundary tiles only), tile maximum, adaptive rescale,
// P = 2^(s*c - m) with the row sum, and O^T += V^T P^T.
template <int D, int BC, bool CAUSAL, int POLY8, bool NEG>
__device__ __forceinline__ void tile_step(const __bf16* __restrict__ ks, const __bf16* __restrict__ vs,
                                          const bf16x8 (&qreg)[D / 16], f32x16 (&oacc)[D / 32], float& m_used,
                                          float& l_sum, int& n_rescale, int j0, int N, int my_q, int l32, int hl,
                                          float c, float tau, bool masked) {
  constexpr int NC = BC / 32;
  constexpr int KK = D / 16;
  constexpr int MT = D / 32;
  constexpr int KSTR = D + 8;
  constexpr int VSTR = D + 32;
  constexpr float mask_val = NEG ? INFINITY : -INFINITY;
  const int lane = 32 * hl + l32;
  const int g = lane >> 4;  // 16-lane group: value features 16*(g%2).., keys +4*(g/2)

  // ---- S^T = K_t Q^T on the matrix cores
  // (k-step outer, chunk inner: the NC accumulation chains interleave)
  f32x16 s[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) s[cc] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const bf16x8 a = *(const bf16x8*)(ks + (32 * cc + l32) * KSTR + 16 * kk + 8 * hl);
      s[cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], s[cc], 0, 0, 0);
    }

  // ---- mask: keys past N, and (causal) keys after the query
  if (masked) {  // boundary tiles only: wave-uniform branch
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 32 * cc + 8 * (r / 4) + 4 * hl + (r % 4);
        const bool hide = key >= N || (CAUSAL && key > my_q);
        s[cc][r] = hide ? mask_val : s[cc][r];
      }
  }

  // ---- tile row maximum (of s*c): in-lane, then the lane pair
  float red;
  if (!NEG) {
    red = s[0][0];
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
#pragma unroll
      for (int r = 0; r < 16; ++r) red = fmaxf(red, s[cc][r]);
    red = pair_max(red);
  } else {
    red = s[0][0];
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
#pragma unroll
      for (int r = 0; r < 16; ++r) red = fminf(red, s[cc][r]);
    red = pair_min(red);
  }
  const float m_tile = (red == mask_val) ? -INFINITY : red * c;

  // ---- adaptive rescale: only when the maximum grows by more than tau
  const float m_new = fmaxf(m_used, m_tile);
  const bool need = (m_new - m_used) > tau;  // +inf on the row's first tile; NaN (false) if both -inf
  if (__any(need)) {
    const float alpha = need ? __builtin_amdgcn_exp2f(m_used - m_new) : 1.f;
    n_rescale += (need && m_used != -INFINITY) ? 1 : 0;
    m_used = need ? m_new : m_used;
    l_sum *= alpha;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[mt][r] *= alpha;
  }

  // ---- P = 2^(s*c - m), row sum in fp32, bf16 pack in the PV operand order
  const float mc = -m_used;
  bf16x8 pb[NC][2];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float x = fmaf(s[cc][r], c, mc);
      float e;
      if (POLY8 == 8 || (POLY8 == 4 && (r & 4)))
        e = attn_exp2_poly(x);
      else
        e = __builtin_amdgcn_exp2f(x);
      l_sum += e;
      pb[cc][r / 8][r % 8] = (__bf16)e;
    }
  }

  // ---- O^T += V_t^T P^T on the matrix cores
#pragma unroll
  for (int cc = 0; cc < NC; ++cc)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row0 = 32 * cc + 16 * h + 4 * (g >> 1);
        const int col0 = 32 * mt + 16 * (g & 1);
        const s16x4 lo = lds_col4(vs, VSTR, row0, col0, lane);
        const s16x4 hi = lds_col4(vs, VSTR, row0 + 8, col0, lane);
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[cc][h], oacc[mt], 0, 0, 0);
      }
}

template <int D, int BC, int NW, bool CAUSAL, bool OF32, int POLY8, bool NEG>
__global__ void __launch_bounds__(NW * 64, 2) attn_fwd_kernel(const Params p) {
  constexpr int BR = 32 * NW;      // query rows per workgroup
  constexpr int NT = NW * 64;      // threads per workgroup
  constexpr int NC = BC / 32;      // 32-key chunks per KV tile
  constexpr int KK = D / 16;       // k-steps of S^T = K Q^T
  constexpr int MT = D / 32;       // 32-row blocks of O^T
  constexpr int KSTR = D + 8;      // K row stride in LDS (elements)
  constexpr int VSTR = D + 32;     // V row stride in LDS (elements): conflict-free transpose reads
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  constexpr int NLD = (BC / 4) * CPR / NT;  // 4-row x 16-byte blocks per thread per tile
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert((BC / 4) * CPR % NT == 0, "load split");
  static_assert(POLY8 == 0 || POLY8 == 4 || POLY8 == 8, "poly split");

  __shared__ __attribute__((aligned(16))) __bf16 ks[BC * KSTR];
  __shared__ __attribute__((aligned(16))) __bf16 vs[BC * VSTR];

  // ---- work decomposition: workgroups are dealt round-robin to the 8 XCDs, so
  // give XCD x the contiguous slice [x*per_xcd, (x+1)*per_xcd) of tiles: the
  // q-tiles of one head then share that XCD's L2 for their K/V re-reads.
  const int wg = blockIdx.x;
  const int logical = (wg & 7) * p.per_xcd + (wg >> 3);
  if (logical >= p.total_tiles) return;
  const int bh = logical / p.nq_tiles;
  int qt = logical - bh * p.nq_tiles;
  if (CAUSAL) qt = p.nq_tiles - 1 - qt;  // longest rows first
  const int N = p.N;
  const int i0 = qt * BR;
  const size_t head = (size_t)bh * (size_t)N * D;
  const __bf16* qh = p.q + head;
  const __bf16* kh = p.k + head;
  const __bf16* vh = p.v + head;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  const int wq0 = i0 + wave * 32;
  const int my_q = wq0 + l32;  // the query row this lane owns

  // ---- Q tile -> registers (B operand of S^T = K Q^T): lane holds Q[my_q][16kk + 8hl + 0..7]
  bf16x8 qreg[KK];
  {
    const __amdgpu_buffer_rsrc_t qrsrc = buffer_rsrc(qh, (uint32_t)N * D * 2);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qreg[kk] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrsrc, (uint32_t)(my_q * D + 16 * kk + 8 * hl) * 2, 0, 0));
  }

  f32x16 oacc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) oacc[mt] = f32x16{};
  float m_used = -INFINITY;  // maximum in use, log2 units
  float l_sum = 0.f;         // this lane's partial row sum (its 16*NC keys per tile)
  int n_rescale = 0;

  const float c = p.c;
  const float tau = p.tau;

  const int kv_end = CAUSAL ? min(N, i0 + BR) : N;
  const int n_tiles = (kv_end + BC - 1) / BC;
  int t_full = N / BC;  // tiles [0, t_full) need no mask
  if (CAUSAL) t_full = min(t_full, (i0 + 1) / BC);

  // ---- K/V staging through registers: thread loads NLD blocks of 4 rows x 16 B
  u32x4 kst[NLD][4], vst[NLD][4];
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const __amdgpu_buffer_rsrc_t krsrc = buffer_rsrc(kh, head_bytes);
  const __amdgpu_buffer_rsrc_t vrsrc = buffer_rsrc(vh, head_bytes);
  auto gload = [&](int t) {
    const int j0 = t * BC;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int blk = tid + i * NT;
      const int col = blk % CPR;
      const int grp = blk / CPR;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t off = (uint32_t)((j0 + 4 * grp + r) * D + 8 * col) * 2;  // >= head_bytes past N: zeros
        kst[i][r] = __builtin_amdgcn_raw_buffer_load_b128(krsrc, off, 0, 0);
        vst[i][r] = __builtin_amdgcn_raw_buffer_load_b128(vrsrc, off, 0, 0);
      }
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int blk = tid + i * NT;
      const int col = blk % CPR;
      const int grp = blk / CPR;
#pragma unroll
      for (int r = 0; r < 4; ++r) *(u32x4*)(ks + (4 * grp + r) * KSTR + 8 * col) = kst[i][r];
#pragma unroll
      for (int r = 0; r < 4; ++r) *(u32x4*)(vs + (4 * grp + r) * VSTR + 8 * col) = vst[i][r];
    }
  };

  if (n_tiles > 0) gload(0);
  for (int t = 0; t < n_tiles; ++t) {
    __syncthreads();  // every wave is done reading the previous tile
    lstore();
    __syncthreads();
    if (t + 1 < n_tiles) gload(t + 1);  // next tile's global loads overlap this tile's math

    const int j0 = t * BC;
    if (CAUSAL && j0 > wq0 + 31) continue;  // whole tile above this wave's diagonal
    // One instantiation of the tile body for every tile: a second (masked) copy
    // makes the register allocator shuttle the output accumulators between
    // register sets on every iteration.
    tile_step<D, BC, CAUSAL, POLY8, NEG>(ks, vs, qreg, oacc, m_used, l_sum, n_rescale, j0, N, my_q, l32, hl, c, tau,
                                         t >= t_full);
  }

  // ---- epilogue: O = acc / l, LSE = ln2 * (m + log2 l), written once
  const float l_tot = pair_sum(l_sum);
  if (my_q < N) {
    const float inv = 1.f / l_tot;
    const size_t row = (size_t)bh * N + my_q;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dv = 32 * mt + 8 * g + 4 * hl;
        if (OF32) {
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = oacc[mt][4 * g + e] * inv;
          *(f32x4*)((float*)p.o + row * D + dv) = w;
        } else {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (__bf16)(oacc[mt][4 * g + e] * inv);
          *(bf16x4*)((__bf16*)p.o + row * D + dv) = w;
        }
      }
    if (hl == 0) {
      p.lse[row] = 0.69314718055994531f * (m_used + log2f(l_tot));
      if (p.rescale_count) p.rescale_count[row] = n_rescale;
    }
  }
}

}  // namespace attn

#endif
