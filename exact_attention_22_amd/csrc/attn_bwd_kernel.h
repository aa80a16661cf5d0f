// attn_bwd_kernel.h - exact-attention backward kernels for gfx950 (MI355X).
//
// The backward pass recomputes the attention probabilities on chip from Q, K
// and the stored log-sum-exp instead of reading a stored N x N matrix (page
// "Flash Attention" glossary, section "Online softmax and recomputation"), and
// forms the gradients without atomic additions (page "FlashAttention-4:
// algorithm-kernel fused pipeline for asymmetric hardware scaling", section 2,
// names shared-memory traffic and atomics as the costs of the backward pass).
// With dO the gradient arriving at O, for one head:
//
//   P = exp(scale * Q K^T - LSE)   dV = P^T dO   dP = dO V^T
//   D_i = dO_i . O_i               dS = P * (dP - D)
//   dQ = scale * dS K              dK = scale * dS^T Q
//
// Two kernels, each owning its outputs (no atomics):
//   dq kernel:   a workgroup owns 128 query rows (32 per wavefront, one per
//                lane). It computes D for its rows (and stores it), then walks
//                the key tiles: S^T = K Q^T and dP^T = V dO^T on the matrix
//                cores, dS^T on the VALU, dQ^T += K^T dS^T.
//   dkdv kernel: a workgroup owns 128 key rows of one key/value head (one per
//                lane) and walks the query tiles of every query head that
//                reads it: S = Q K^T and dP = dO V^T, then dV^T += dO^T P and
//                dK^T += Q^T dS. It reads D from the dq kernel, which runs first.
// Both use the 32x32x16 bf16 MFMA in the layout of the forward kernel: lane l
// holds column l % 32 of the accumulator, so the row that a lane owns needs no
// cross-lane reduction, and the bf16 P (or dS) of one product is the B operand
// of the next. The A operands are 16-byte row reads of an LDS tile (K, V, Q,
// dO) or transpose reads of the same tile (ds_read_b64_tr_b16), so every LDS
// tile uses one XOR swizzle that is free of bank conflicts for both: 16
// consecutive rows at one 16-byte chunk, and 4 aligned rows at 4 aligned chunks.
#ifndef ATTN_BWD_KERNEL_H
#define ATTN_BWD_KERNEL_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace attn_grad {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

struct BwdParams {
  const __bf16* q;    // [B][H][N][D]
  const __bf16* k;    // [B][Hkv][N][D]
  const __bf16* v;    // [B][Hkv][N][D]
  const __bf16* o;    // [B][H][N][D]
  const float* lse;   // [B][H][N], natural log
  const __bf16* dout; // [B][H][N][D]
  __bf16* dq;         // [B][H][N][D]
  __bf16* dk;         // [B][Hkv][N][D]
  __bf16* dv;         // [B][Hkv][N][D]
  float* delta;       // [B][H][N]: D_i = dO_i . O_i (written by the dq kernel)
  // packed variable-length batches: every tensor is [heads][total][D] (lse, delta
  // [H][total]) and sequence s owns tokens cu_seqlens[s] .. cu_seqlens[s+1]-1
  const int* cu_seqlens;  // nseq + 1 cumulative lengths (device)
  int nseq;
  int N;              // dense: sequence length; packed: total tokens
  int H;
  int G;              // query heads per key/value head
  int n_tiles;        // ceil(N / 128) row tiles per head (packed: per longest sequence)
  float scale;
  float c;            // scale * log2(e)
  int n_xcd;          // XCDs the dispatcher deals workgroups to in turn (1: no renumbering)
  int cus_per_xcd;    // compute units of one XCD
};

// (head, row tile) of this workgroup: bg = head index (dense b * heads + h; packed
// h * nseq + sequence), rank = row tile in the kernel's own order (rank 0 is the
// tile with the most work under causal masking).
// The dispatcher deals workgroups to the n_xcd XCDs in turn (workgroup i to XCD
// i mod n_xcd); numbered XCD-major, each XCD holds a contiguous range of whole heads,
// so the workgroups of one head, which load the same tiles at about the same time,
// share one L2. Under causal masking the row tiles differ in length; when a head has
// no more tiles than the XCD runs workgroups at once (PER_CU per compute unit), the
// XCD runs several heads together anyway, and within its range the workgroups go by
// rank first, so every head's long tiles start before any short one (with more tiles
// per head, head order keeps one head's workgroups together and the short tiles of
// one head fill in beside the long ones of the next). Plain numbering when the grid
// does not divide evenly.
struct BlockCoords {
  int bg, rank;
};
template <bool CAUSAL, int PER_CU>
__device__ __forceinline__ BlockCoords block_coords(const BwdParams& p) {
  const int n = gridDim.x, b = blockIdx.x, n_xcd = p.n_xcd, n_tiles = p.n_tiles;
  const bool split = n_xcd > 1 && n % n_xcd == 0;
  const int per = split ? n / n_xcd : n;  // workgroups of one XCD
  const int blk = split ? (b % n_xcd) * per + b / n_xcd : b;
  if (CAUSAL && per % n_tiles == 0 && n_tiles <= PER_CU * p.cus_per_xcd) {
    const int heads = per / n_tiles;  // whole heads per XCD range
    const int base = blk - blk % per, k = blk - base;
    return {base / n_tiles + k % heads, k / heads};
  }
  return {blk / n_tiles, blk % n_tiles};
}

// Four wavefronts per workgroup (one per SIMD). The dq kernel (and the dk/dv kernel
// at D = 64) fits two workgroups per compute unit, so each SIMD runs two wavefronts
// whose matrix and vector work overlap. At D = 128 the one-wavefront dk/dv kernel
// holds two 128-feature accumulators per lane and runs one workgroup per compute
// unit; it serves as the reference schedule there, and the wavefront-pair kernel
// below (one accumulator per wavefront, eight wavefronts) does the work.
constexpr int kWaves = 4;
constexpr int kRows = 32 * kWaves;   // rows a workgroup owns
constexpr int kTile = 64;            // rows of the streamed tiles

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Chunk swizzle of LDS row r (16-byte chunks; D/8 per row).
template <int D>
__device__ __forceinline__ int swz(int r) {
  return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// 16-byte chunk c of row R (row read; A operand rows).
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const char* t, int R, int c) {
  return *(const bf16x8*)(t + R * (2 * D) + ((c ^ swz<D>(R)) << 4));
}

// Transpose read: lane l receives column col0 + l % 32 of rows row0 + 4*(l/32) + e,
// e = 0..3 (lane l supplies the address of row row0 + 4*(l/32) + (l%16)/4, columns
// col0 + 16*((l/16)%2) + 4*(l%4) .. +3).
template <int D>
__device__ __forceinline__ s16x4 tr4(const char* t, int row0, int col0, int lane) {
  const int r = row0 + 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const char* a = t + r * (2 * D) + (((col >> 3) ^ swz<D>(r)) << 4) + ((col & 7) << 1);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(lds_void*)a);
}

// A operand of a product contracting over tile rows: k-step covering rows
// row0 .. row0+15 (lane l's eight rows: row0 + 8*(j/4) + 4*(l/32) + j%4), feature
// block col0 .. col0+31 (lane l: feature col0 + l%32).
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const char* t, int row0, int col0, int lane) {
  const s16x4 lo = tr4<D>(t, row0, col0, lane);
  const s16x4 hi = tr4<D>(t, row0 + 8, col0, lane);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Loads rows r0 .. r0+63 of a row-major [n][D] bf16 matrix at `base` into an LDS
// tile with the swizzle; rows >= n read as zeros. Four wavefronts share the work,
// each lane fills 16 bytes per load at tile + 1 KiB * load + 16 * lane.
template <int D>
__device__ __forceinline__ void load_tile64(const __bf16* base, int n, int r0, char* tile, int wave, int lane) {
  constexpr int CH = D / 8;          // chunks per row
  constexpr int RPL = 64 / CH;       // rows per wave-load
  constexpr int LOADS = kTile / RPL; // wave-loads per tile
  const uint32_t bytes = r0 < n ? (uint32_t)(n - r0) * D * 2 : 0u;
  const __amdgpu_buffer_rsrc_t rs = rsrc(base + (size_t)(r0 < n ? r0 : 0) * D, __builtin_amdgcn_readfirstlane(bytes));
  static_assert(LOADS % kWaves == 0, "tile load split");
#pragma unroll
  for (int ii = 0; ii < LOADS / kWaves; ++ii) {
    const int i = ii * kWaves + wave;
    const int r = i * RPL + lane / CH;
    const int c = (lane % CH) ^ swz<D>(r);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(tile + i * 1024), 16, (uint32_t)(r * D + 8 * c) * 2, 0,
                                             0, 0);
  }
}

// 64 floats at base[r0 ..] (zeros past n) into LDS, by one wavefront.
__device__ __forceinline__ void load_vec64(const float* base, int n, int r0, float* dst, int lane) {
  const uint32_t bytes = r0 < n ? (uint32_t)(n - r0) * 4 : 0u;
  const __amdgpu_buffer_rsrc_t rs = rsrc(base + (r0 < n ? r0 : 0), __builtin_amdgcn_readfirstlane(bytes));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 4, (uint32_t)lane * 4, 0, 0, 0);
}

// B operand rows of a lane: row `row` of a [n][D] matrix, features 16*kk + 8*hl .. +7.
template <int D>
__device__ __forceinline__ void load_row_operand(bf16x8 (&dst)[D / 16], const __bf16* base, int n, int row, int hl) {
  const __amdgpu_buffer_rsrc_t rs = rsrc(base, (uint32_t)n * D * 2);
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    dst[kk] = __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(row * D + 16 * kk + 8 * hl) * 2, 0, 0));
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Stores accumulator rows: lane l owns row `row`, accumulator block mt holds
// features 32*mt + 8*(r/4) + 4*(l/32) + r%4 in register r; multiplied by `mul`.
template <int D>
__device__ __forceinline__ void store_rows(__bf16* out, size_t row, const f32x16 (&acc)[D / 32], float mul, int hl) {
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[mt][4 * gq + e] * mul);
      *(bf16x4*)(out + row * D + 32 * mt + 8 * gq + 4 * hl) = w;
    }
}

__device__ __forceinline__ void sync_tiles() {
  __builtin_amdgcn_s_waitcnt(0);  // this wavefront's tile loads and LDS accesses are done
  __syncthreads();
}

// Packed batches: the clamped bounds [a, e) of sequence s (the forward kernel's
// reading: any contents of cu_seqlens stay inside [0, total]).
__device__ __forceinline__ void seq_bounds(const BwdParams& p, int s, int& a, int& e) {
  a = min(max(p.cu_seqlens[s], 0), p.N);
  e = min(max(p.cu_seqlens[s + 1], a), p.N);
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wavefront's LDS accesses; loads in flight may stay
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Keeps the matrix products and LDS reads on either side in source order (vector
// and scalar ALU work may still move across): operand reads written a few products
// ahead then stay ahead, where the scheduler would otherwise sink each read to just
// before its product and make the product wait for it.
__device__ __forceinline__ void keep_order() { __builtin_amdgcn_sched_barrier(0x0002 | 0x0004 | 0x0400); }

// Per-lane byte offsets of the A operands in a swizzled [64][D] LDS tile,
// independent of the buffer and of the 32-row block (row reads) or 16-row group
// (transpose reads): those add a constant that the read instruction carries.
//   row[kk]:   row 32 cc + l % 32, chunk 2 kk + l / 32 (row_frag), + cc * 64 * D
//   tr[mt][h]: the rows 16 j + 8 h + 4 (l / 32) + (l % 16) / 4 and columns
//              32 mt + 16 ((l / 16) % 2) + 4 (l % 4) of tr4, + j * 32 * D
template <int D>
struct OperandOffsets {
  int row[D / 16];
  int tr[D / 32][2];
  __device__ __forceinline__ void init(int lane) {
    const int l32 = lane & 31, hl = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) row[kk] = l32 * (2 * D) + (((2 * kk + hl) ^ swz<D>(l32)) << 4);
    const int rl = 4 * (lane >> 5) + ((lane & 15) >> 2);
    const int cl = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 8 * h + rl, col = 32 * mt + cl;
        tr[mt][h] = r * (2 * D) + (((col >> 3) ^ swz<D>(r)) << 4) + ((col & 7) << 1);
      }
  }
  // From here on the compiler takes the offsets as changed: it adds the buffer's
  // constant at each read instead of keeping one register per read and buffer.
  __device__ __forceinline__ void launder() {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(row[kk]));
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) {
      asm volatile("" : "+v"(tr[mt][0]));
      asm volatile("" : "+v"(tr[mt][1]));
    }
  }
};
__device__ __forceinline__ bf16x8 row_at(const char* t, int off) { return *(const bf16x8*)(t + off); }
__device__ __forceinline__ bf16x8 tr_at(const char* t, int off_lo, int off_hi) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(lds_void*)(t + off_lo));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(lds_void*)(t + off_hi));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---------------------------------------------------------------------------
// dq kernel: workgroup = (b, h, 128 query rows); packed batches (VARLEN):
// workgroup = (h, sequence, 128 query rows of that sequence).
template <int D, bool CAUSAL, bool VARLEN = false>
__global__ void __launch_bounds__(256, 2) attn_bwd_dq_kernel(const BwdParams p) {
  constexpr int KK = D / 16, MT = D / 32, NC = kTile / 32;
  constexpr int TB = kTile * D * 2;
  // Separate arrays per buffer (not one [2][TB] array): the compiler then sees that
  // the loads into one buffer do not alias the reads of the other and does not
  // wait for the next tile's loads before reading the current one.
  __shared__ __attribute__((aligned(1024))) char kt0[TB];
  __shared__ __attribute__((aligned(1024))) char kt1[TB];
  __shared__ __attribute__((aligned(1024))) char vt0[TB];
  __shared__ __attribute__((aligned(1024))) char vt1[TB];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const BlockCoords bc = block_coords<CAUSAL, 2>(p);
  const int hb = bc.bg;
  // causal: a query block sees the key tiles up to its own, so rank 0 is the last block
  const int i0 = (CAUSAL ? p.n_tiles - 1 - bc.rank : bc.rank) * kRows;
  int N;             // rows (and keys) of this workgroup's sequence
  size_t qrow0, kvrow0;  // first row of the query head / key-value head in memory
  if (VARLEN) {
    const int h = hb / p.nseq, sq = hb - h * p.nseq;
    int a, e;
    seq_bounds(p, sq, a, e);
    N = e - a;
    if (i0 >= N) return;  // whole workgroup: past its sequence
    qrow0 = (size_t)h * p.N + a;
    kvrow0 = (size_t)(h / p.G) * p.N + a;
  } else {
    N = p.N;
    const int b = hb / p.H, h = hb - b * p.H;
    qrow0 = (size_t)hb * N;
    kvrow0 = (size_t)(b * (p.H / p.G) + h / p.G) * N;
  }
  const size_t qhead = qrow0 * D;
  const size_t kvhead = kvrow0 * D;
  const int my_q = i0 + 32 * wave + l32;

  bf16x8 qreg[KK], doreg[KK], oreg[KK];
  load_row_operand<D>(qreg, p.q + qhead, N, my_q, hl);
  load_row_operand<D>(doreg, p.dout + qhead, N, my_q, hl);
  load_row_operand<D>(oreg, p.o + qhead, N, my_q, hl);
  const __amdgpu_buffer_rsrc_t lrs = rsrc(p.lse + qrow0, (uint32_t)N * 4);
  const float lse2 =
      __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(lrs, (uint32_t)my_q * 4, 0, 0)) * 1.44269504088896341f;
  float dpart = 0.f;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
#pragma unroll
    for (int e = 0; e < 8; ++e) dpart = fmaf((float)doreg[kk][e], (float)oreg[kk][e], dpart);
  const float Di = pair_sum(dpart);
  if (my_q < N && hl == 0) p.delta[qrow0 + my_q] = Di;

  const int kv_end = CAUSAL ? min(N, i0 + kRows) : N;
  const int n_kt = (kv_end + kTile - 1) / kTile;
  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};

  load_tile64<D>(p.k + kvhead, N, 0, kt0, wave, lane);
  load_tile64<D>(p.v + kvhead, N, 0, vt0, wave, lane);
  sync_tiles();
  OperandOffsets<D> oo;
  oo.init(lane);
  // The products' A operands are read ahead of their use: the K and V row fragments
  // of S and dP RA k-steps ahead, the transpose operands of dQ RT products ahead
  // (the first RT of a block before its dS).
  constexpr int NRF = NC * KK, RA = 2, NTR = 2 * MT, RT = 2;
  // Step t computes on (K, V) while tile t+1 loads into (Kn, Vn); the loads are
  // unconditional (past the last tile they read beyond kv_end or, past N, nothing).
  auto step = [&](int t, const char* K, const char* V, char* Kn, char* Vn) {
    oo.launder();
    const int j0 = t * kTile;
    load_tile64<D>(p.k + kvhead, N, j0 + kTile, Kn, wave, lane);
    load_tile64<D>(p.v + kvhead, N, j0 + kTile, Vn, wave, lane);
    const bool edge = j0 + kTile > N || (CAUSAL && j0 + kTile - 1 > i0 + 32 * wave);
    bf16x8 kr[NRF], vr[NRF];
    auto rd = [&](int f) {
      kr[f] = row_at(K + (f / KK) * 64 * D, oo.row[f % KK]);
      vr[f] = row_at(V + (f / KK) * 64 * D, oo.row[f % KK]);
    };
#pragma unroll
    for (int f = 0; f < RA; ++f) rd(f);
    // One 32-key block at a time, so that only one block's scores are live.
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int f = cc * KK + kk;
        if (f + RA < NRF) rd(f + RA);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[f], qreg[kk], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[f], doreg[kk], dp, 0, 0, 0);
        keep_order();
      }
      // transpose operands of this block's dQ products, i = 2 * hh + ... (hh, mt)
      bf16x8 tq[NTR];
      auto trd = [&](int j) { tq[j] = tr_at(K + (2 * cc + j / MT) * 32 * D, oo.tr[j % MT][0], oo.tr[j % MT][1]); };
#pragma unroll
      for (int j = 0; j < RT; ++j) trd(j);
      // dS^T in the B-operand order of the next product: k-step 2*cc + hh holds keys
      // 32*cc + 16*hh + 8*(j/4) + 4*hl + j%4 (register r = 8*hh + j of the block).
      // The masked form runs only on boundary tiles (a branch on the wavefront-uniform
      // `edge`): written as one loop with a select, the compiler if-converts the mask
      // and every tile pays its compares and selects.
      bf16x8 dsb[2];
      auto ds_block = [&](auto masked) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pr = __builtin_amdgcn_exp2f(fmaf(s[r], p.c, -lse2));
          if (decltype(masked)::value) {
            const int key = j0 + 32 * cc + 8 * (r / 4) + 4 * hl + (r % 4);
            pr = (key >= N || (CAUSAL && key > my_q)) ? 0.f : pr;
          }
          dsb[r / 8][r % 8] = (__bf16)(pr * (dp[r] - Di));
        }
      };
      if (edge)
        ds_block(std::true_type{});
      else
        ds_block(std::false_type{});
#pragma unroll
      for (int j = 0; j < NTR; ++j) {
        if (j + RT < NTR) trd(j + RT);
        acc[j % MT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tq[j], dsb[j / MT], acc[j % MT], 0, 0, 0);
        keep_order();
      }
    }
    sync_tiles();
  };
  int t = 0;
  for (; t + 1 < n_kt; t += 2) {
    step(t, kt0, vt0, kt1, vt1);
    step(t + 1, kt1, vt1, kt0, vt0);
  }
  if (t < n_kt) step(t, kt0, vt0, kt1, vt1);
  if (my_q < N) store_rows<D>(p.dq, qrow0 + my_q, acc, p.scale, hl);
}

// ---------------------------------------------------------------------------
// dkdv kernel: workgroup = (b, key/value head g, 128 key rows); walks the query
// tiles of query heads g*G .. g*G + G - 1. Packed batches (VARLEN): workgroup =
// (g, sequence, 128 key rows of that sequence).
template <int D, bool CAUSAL, bool VARLEN = false>
__global__ void __launch_bounds__(256, D == 128 ? 1 : 2) attn_bwd_dkdv_kernel(const BwdParams p) {
  constexpr int KK = D / 16, MT = D / 32, NC = kTile / 32;
  constexpr int TB = kTile * D * 2;
  // One array per buffer, as in the dq kernel.
  __shared__ __attribute__((aligned(1024))) char qt0[TB];
  __shared__ __attribute__((aligned(1024))) char qt1[TB];
  __shared__ __attribute__((aligned(1024))) char dot0[TB];
  __shared__ __attribute__((aligned(1024))) char dot1[TB];
  __shared__ __attribute__((aligned(16))) float lse0[kTile];
  __shared__ __attribute__((aligned(16))) float lse1[kTile];
  __shared__ __attribute__((aligned(16))) float del0[kTile];
  __shared__ __attribute__((aligned(16))) float del1[kTile];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const int Hkv = p.H / p.G;
  // causal: a key block sees the query tiles from its own on, so rank 0 is block 0
  const BlockCoords bc = block_coords<CAUSAL, D == 128 ? 1 : 2>(p);
  const int bg = bc.bg;  // dense: b * Hkv + g; packed: g * nseq + sequence
  const int j0w = bc.rank * kRows;
  int N, g;
  size_t kvrow0, qrow_first, qrow_step;  // query head hq starts at row qrow_first + hq * qrow_step
  if (VARLEN) {
    g = bg / p.nseq;
    const int sq = bg - g * p.nseq;
    int a, e;
    seq_bounds(p, sq, a, e);
    N = e - a;
    if (j0w >= N) return;  // whole workgroup: past its sequence
    kvrow0 = (size_t)g * p.N + a;
    qrow_first = a;
    qrow_step = p.N;
  } else {
    N = p.N;
    const int b = bg / Hkv;
    g = bg - b * Hkv;
    kvrow0 = (size_t)bg * N;
    qrow_first = (size_t)b * p.H * N;
    qrow_step = N;
  }
  const size_t kvhead = kvrow0 * D;
  const int my_k = j0w + 32 * wave + l32;

  bf16x8 kreg[KK], vreg[KK];
  load_row_operand<D>(kreg, p.k + kvhead, N, my_k, hl);
  load_row_operand<D>(vreg, p.v + kvhead, N, my_k, hl);

  f32x16 dka[MT], dva[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    dka[mt] = f32x16{};
    dva[mt] = f32x16{};
  }
  // query tiles: causal rows below the workgroup's first key see none of its keys
  const int it0 = CAUSAL ? j0w / kTile : 0;
  const int n_qt = (N + kTile - 1) / kTile;
  const int per_head = n_qt - it0;
  const int steps = per_head * p.G;
  // Loads of step `st` (query head g*G + st/per_head, query tile it0 + st%per_head);
  // a step past the last reloads the last tile, so every step issues the same loads.
  auto issue = [&](int st, char* Qb, char* dOb, float* lb, float* db) {
    st = min(st, steps - 1);
    const int hq = g * p.G + st / per_head;
    const int iq0 = (it0 + st % per_head) * kTile;
    const size_t qhead = qrow_first + (size_t)hq * qrow_step;
    load_tile64<D>(p.q + qhead * D, N, iq0, Qb, wave, lane);
    load_tile64<D>(p.dout + qhead * D, N, iq0, dOb, wave, lane);
    if (wave == 0) load_vec64(p.lse + qhead, N, iq0, lb, lane);
    if (wave == 1) load_vec64(p.delta + qhead, N, iq0, db, lane);
  };
  issue(0, qt0, dot0, lse0, del0);
  sync_tiles();
  auto step = [&](int t, const char* Q, const char* dO, const float* lt, const float* dt, char* Qn, char* dOn,
                  float* ln, float* dn) {
    issue(t + 1, Qn, dOn, ln, dn);
    const int iq0 = (it0 + t % per_head) * kTile;
    const bool edge = iq0 + kTile > N || (CAUSAL && iq0 < j0w + 32 * wave + 32);
    // One 32-query block at a time, so that only one block's scores are live. Lane l
    // holds key my_k (column) and, in register r, query row 32*cc + 8*(r/4) + 4*hl + r%4.
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(Q, 32 * cc + l32, 2 * kk + hl), kreg[kk], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(dO, 32 * cc + l32, 2 * kk + hl), vreg[kk], dp, 0, 0,
                                                     0);
      }
      // Boundary tiles hide their scores first (as -inf, so P = 2^-inf = 0) in a branch
      // of their own; the rest of the block is the same code for every tile.
      if (edge) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = iq0 + 32 * cc + 8 * (r / 4) + 4 * hl + (r % 4);
          s[r] = (qi >= N || (CAUSAL && my_k > qi)) ? -INFINITY : s[r];
        }
      }
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int qr = 32 * cc + 8 * gq + 4 * hl;
        const f32x4 l4 = *(const f32x4*)&lt[qr];
        const f32x4 d4 = *(const f32x4*)&dt[qr];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * gq + e;
          const float pr = __builtin_amdgcn_exp2f(fmaf(s[r], p.c, -l4[e] * 1.44269504088896341f));
          pb[r / 8][r % 8] = (__bf16)pr;
          dsb[r / 8][r % 8] = (__bf16)(pr * (dp[r] - d4[e]));
        }
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          dva[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(dO, 32 * cc + 16 * hh, 32 * mt, lane),
                                                            pb[hh], dva[mt], 0, 0, 0);
          dka[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(Q, 32 * cc + 16 * hh, 32 * mt, lane),
                                                            dsb[hh], dka[mt], 0, 0, 0);
        }
    }
    sync_tiles();
  };
  int t = 0;
  for (; t + 1 < steps; t += 2) {
    step(t, qt0, dot0, lse0, del0, qt1, dot1, lse1, del1);
    step(t + 1, qt1, dot1, lse1, del1, qt0, dot0, lse0, del0);
  }
  if (t < steps) step(t, qt0, dot0, lse0, del0, qt1, dot1, lse1, del1);
  if (my_k < N) {
    store_rows<D>(p.dk, kvrow0 + my_k, dka, p.scale, hl);
    store_rows<D>(p.dv, kvrow0 + my_k, dva, 1.f, hl);
  }
}

// ---------------------------------------------------------------------------
// dkdv kernel in wavefront pairs (used at D = 128): eight wavefronts, two per
// SIMD, 128 key rows per workgroup. Wavefront w < 4 (the P wavefront) and
// wavefront w + 4 (the dS wavefront) own the same 32 keys and run on the same
// SIMD (wavefronts are dealt to the SIMDs round-robin). Per query tile:
//   P wavefront:  S = Q K^T, P = exp2(S*c - LSE*log2 e) (masked), P to LDS in
//                 fp32; barrier; dV^T += dO^T P.
//   dS wavefront: dP = dO V^T; barrier; P from LDS, dS = P * (dP - D),
//                 dK^T += Q^T dS.
// Each holds one 128-feature accumulator and one operand row set (K or V), so
// both fit 256 registers and the SIMD interleaves one wavefront's products with
// the other's vector work. The arithmetic, and the order of every accumulation,
// is that of attn_bwd_dkdv_kernel; P crosses LDS in fp32, so dK and dV are the
// same bits. The dS wavefronts issue the next step's tile loads right after
// their dP products (the P wavefront's exponentials make them wait there
// anyway); the P buffer has one slot per pair, written after the barrier that
// ends a step and read before the next one. Wavefront 4 (the first dS
// wavefront) stores each LSE tile pre-multiplied by -log2(e) in LDS once it has
// landed (the product the exponent needs per score).
template <int D, bool CAUSAL, bool VARLEN = false>
__global__ void __launch_bounds__(512, 1) attn_bwd_dkdv_pair_kernel(const BwdParams p) {
  constexpr int KK = D / 16, MT = D / 32, NC = kTile / 32;
  constexpr int TB = kTile * D * 2;
  __shared__ __attribute__((aligned(1024))) char qt0[TB];
  __shared__ __attribute__((aligned(1024))) char qt1[TB];
  __shared__ __attribute__((aligned(1024))) char dot0[TB];
  __shared__ __attribute__((aligned(1024))) char dot1[TB];
  __shared__ __attribute__((aligned(16))) float lse0[kTile];
  __shared__ __attribute__((aligned(16))) float lse1[kTile];
  __shared__ __attribute__((aligned(16))) float del0[kTile];
  __shared__ __attribute__((aligned(16))) float del1[kTile];
  // P of a pair's score block cc: registers 4g .. 4g+3 of lane l at [wave][cc][g][l]
  __shared__ __attribute__((aligned(1024))) f32x4 pbuf[kWaves][NC][4][64];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave = wv & 3;      // key block of the pair
  const bool pw = wv < kWaves;  // P wavefront (K, dV) or dS wavefront (V, dK)
  const int l32 = lane & 31, hl = lane >> 5;
  const int Hkv = p.H / p.G;
  // causal: a key block sees the query tiles from its own on, so rank 0 is block 0
  const BlockCoords bc = block_coords<CAUSAL, 1>(p);
  const int bg = bc.bg;  // dense: b * Hkv + g; packed: g * nseq + sequence
  const int j0w = bc.rank * kRows;
  int N, g;
  size_t kvrow0, qrow_first, qrow_step;  // query head hq starts at row qrow_first + hq * qrow_step
  if (VARLEN) {
    g = bg / p.nseq;
    const int sq = bg - g * p.nseq;
    int a, e;
    seq_bounds(p, sq, a, e);
    N = e - a;
    if (j0w >= N) return;  // whole workgroup: past its sequence
    kvrow0 = (size_t)g * p.N + a;
    qrow_first = a;
    qrow_step = p.N;
  } else {
    N = p.N;
    const int b = bg / Hkv;
    g = bg - b * Hkv;
    kvrow0 = (size_t)bg * N;
    qrow_first = (size_t)b * p.H * N;
    qrow_step = N;
  }
  const size_t kvhead = kvrow0 * D;
  const int my_k = j0w + 32 * wave + l32;

  bf16x8 kvreg[KK];  // K rows (P wavefront) or V rows (dS wavefront) of the lane's key
  load_row_operand<D>(kvreg, (pw ? p.k : p.v) + kvhead, N, my_k, hl);
  f32x16 acc[MT];  // dV^T (P wavefront) or dK^T (dS wavefront)
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};
  OperandOffsets<D> oo;
  oo.init(lane);
  const int it0 = CAUSAL ? j0w / kTile : 0;
  const int n_qt = (N + kTile - 1) / kTile;
  const int per_head = n_qt - it0;
  const int steps = per_head * p.G;
  auto issue = [&](int st, char* Qb, char* dOb, float* lb, float* db) {
    st = min(st, steps - 1);
    const int hq = g * p.G + st / per_head;
    const int iq0 = (it0 + st % per_head) * kTile;
    const size_t qhead = qrow_first + (size_t)hq * qrow_step;
    load_tile64<D>(p.q + qhead * D, N, iq0, Qb, wave, lane);
    load_tile64<D>(p.dout + qhead * D, N, iq0, dOb, wave, lane);
    if (wave == 0) load_vec64(p.lse + qhead, N, iq0, lb, lane);
    if (wave == 1) load_vec64(p.delta + qhead, N, iq0, db, lane);
  };
  // the dS wavefronts issue the tile loads (in the part of a step where they would
  // otherwise wait for P); the first of them loads the LSE tile and, once it has
  // landed, stores -LSE * log2(e)
  auto scale_lse = [&](float* lb) {
    if (wv == kWaves) lb[lane] = -lb[lane] * 1.44269504088896341f;
  };
  if (!pw) issue(0, qt0, dot0, lse0, del0);
  __builtin_amdgcn_s_waitcnt(0);
  scale_lse(lse0);
  __syncthreads();
  // P of score block cc (lane: key my_k, register r: query row 32 cc + 8 (r / 4) + 4 hl + r % 4)
  // into the P buffer (fp32) and, as bf16, the B operands of dV
  auto p_block = [&](auto masked, int cc, const f32x16& s, const float* nl, int iq0, bf16x8 (&pbc)[2]) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int qr = 32 * cc + 8 * gq + 4 * hl;
      const f32x4 l4 = *(const f32x4*)&nl[qr];
      f32x4 p4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * gq + e;
        float pr = __builtin_amdgcn_exp2f(fmaf(s[r], p.c, l4[e]));
        if (decltype(masked)::value) {
          const int qi = iq0 + qr + e;
          pr = (qi >= N || (CAUSAL && my_k > qi)) ? 0.f : pr;
        }
        p4[e] = pr;
        pbc[r / 8][r % 8] = (__bf16)pr;
      }
      pbuf[wave][cc][gq][lane] = p4;
    }
  };
  // One loop per role (the role is uniform per wavefront), so that each keeps its
  // accumulator in the same registers across the loop; both pass 2 barriers per step.
  auto end_step = [&](float* lnx) {  // lnx: the next LSE tile (dS wavefronts), else null
    __builtin_amdgcn_s_waitcnt(0);     // the next tile's loads landed; this wavefront's LDS accesses done
    if (lnx) scale_lse(lnx);
    __syncthreads();
  };
  // The products' A operands come from LDS: row fragments (S, dP) and transpose
  // reads (dV, dK). Each is read RA products ahead of its use, so a product never
  // waits for the read that feeds it; the transpose reads of the second products
  // start before the barrier between the two halves of a step (the tiles are
  // resident from the step's first barrier on).
  constexpr int NRF = NC * KK;      // row-fragment products per step (S or dP)
  constexpr int NTR = NC * 2 * MT;  // transpose-operand products per step (dV or dK)
  constexpr int RA = 4;
  // row-fragment chain: x[cc] = sum_kk A(tile rows 32 cc.., chunk kk) . kvreg[kk]; `after(cc)`
  // runs when block cc's chain has been issued
  auto row_chain = [&](const char* T, f32x16 (&x)[NC], auto&& after) {
    bf16x8 rf[NRF];
    auto rd = [&](int f) { rf[f] = row_at(T + (f / KK) * 64 * D, oo.row[f % KK]); };
#pragma unroll
    for (int f = 0; f < RA; ++f) rd(f);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int f = cc * KK + kk;
        if (f + RA < NRF) rd(f + RA);
        x[cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rf[f], kvreg[kk], kk == 0 ? f32x16{} : x[cc], 0, 0, 0);
      }
      if (cc == 0) __builtin_amdgcn_sched_group_barrier(0x100, RA, 0);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (cc * KK + kk + RA < NRF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      after(cc);
    }
  };
  // transpose operand i = (2 cc + hh) * MT + mt of tile T
  auto tr_read = [&](const char* T, int i) {
    return tr_at(T + (i / MT) * 32 * D, oo.tr[i % MT][0], oo.tr[i % MT][1]);
  };
  auto p_step = [&](int t, const char* Q, const char* dO, const float* lt) {
    oo.launder();
    const int iq0 = (it0 + t % per_head) * kTile;
    const bool edge = iq0 + kTile > N || (CAUSAL && iq0 < j0w + 32 * wave + 32);
    bf16x8 pb[NC][2];
    f32x16 s[NC];
    row_chain(Q, s, [&](int cc) {
      if (edge)
        p_block(std::true_type{}, cc, s[cc], lt, iq0, pb[cc]);
      else
        p_block(std::false_type{}, cc, s[cc], lt, iq0, pb[cc]);
    });
    bf16x8 vf[NTR];
#pragma unroll
    for (int i = 0; i < RA; ++i) vf[i] = tr_read(dO, i);
    lds_barrier();  // P of this step in LDS
#pragma unroll
    for (int i = 0; i < NTR; ++i) {
      if (i + RA < NTR) vf[i + RA] = tr_read(dO, i + RA);
      const int cc = i / (2 * MT), hh = (i / MT) % 2, mt = i % MT;
      acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pb[cc][hh], acc[mt], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NTR; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + RA < NTR) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    end_step(nullptr);
  };
  auto ds_step = [&](int t, const char* Q, const char* dO, const float* dt, char* Qn, char* dOn, float* lnx,
                     float* dn) {
    oo.launder();
    f32x16 dp[NC];
    row_chain(dO, dp, [](int) {});
    issue(t + 1, Qn, dOn, lnx, dn);
    bf16x8 kf[NTR];
#pragma unroll
    for (int i = 0; i < RA; ++i) kf[i] = tr_read(Q, i);
    lds_barrier();  // P of this step in LDS
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      bf16x8 dsb[2];
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int qr = 32 * cc + 8 * gq + 4 * hl;
        const f32x4 d4 = *(const f32x4*)&dt[qr];
        const f32x4 p4 = pbuf[wave][cc][gq][lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * gq + e;
          dsb[r / 8][r % 8] = (__bf16)(p4[e] * (dp[cc][r] - d4[e]));
        }
      }
#pragma unroll
      for (int j = 0; j < 2 * MT; ++j) {
        const int i = cc * 2 * MT + j;
        if (i + RA < NTR) kf[i + RA] = tr_read(Q, i + RA);
        const int hh = j / MT, mt = j % MT;
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], dsb[hh], acc[mt], 0, 0, 0);
      }
    }
    end_step(lnx);
  };
  if (pw) {
    int t = 0;
    for (; t + 1 < steps; t += 2) {
      p_step(t, qt0, dot0, lse0);
      p_step(t + 1, qt1, dot1, lse1);
    }
    if (t < steps) p_step(t, qt0, dot0, lse0);
  } else {
    int t = 0;
    for (; t + 1 < steps; t += 2) {
      ds_step(t, qt0, dot0, del0, qt1, dot1, lse1, del1);
      ds_step(t + 1, qt1, dot1, del1, qt0, dot0, lse0, del0);
    }
    if (t < steps) ds_step(t, qt0, dot0, del0, qt1, dot1, lse1, del1);
  }
  if (my_k < N) {
    if (pw)
      store_rows<D>(p.dv, kvrow0 + my_k, acc, 1.f, hl);
    else
      store_rows<D>(p.dk, kvrow0 + my_k, acc, p.scale, hl);
  }
}

}  // namespace attn_grad

#endif
