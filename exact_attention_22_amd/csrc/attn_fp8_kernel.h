// attn_fp8_kernel.h - FP8 (e4m3) exact-attention forward kernel for gfx950.
//
// The FP8 form of the method: both products run on 8-bit floating-point
// operands (page "Flash Attention" glossary, section "FlashAttention-3 and the
// FP8 era", and its hardware section on FP8 and lower-precision formats).
// Everything else is the tiled online softmax of the
// bf16 kernel (page "Flash Attention" glossary, sections "Tiling with SRAM" and
// "Online softmax and recomputation"), with the adaptive rescale of page
// "FlashAttention 4: ...", section "Smarter online softmax rescaling (new in FA4)".
//
// Inputs are OCP e4m3 ("e4m3fn") codes with one fp32 dequantisation scale per
// tensor; the softmax scale and the q and k scales fold into one fp32 factor
// c = scale * q_scale * k_scale * log2(e) applied to the fp32 scores, and the v
// scale into the final normalisation.
//
// Matrix instruction: v_mfma_scale_f32_32x32x64_f8f6f4 (block scales fixed at
// 2^0). Its A and B operands are 32 bytes per lane: lane l supplies row l % 32
// (A) or column l % 32 (B) and 32 of the 64 k-slots, the lane half l / 32
// selecting which; the two operands use the same k-slot assignment, so any
// relabelling of the contraction index applied to both leaves the product
// unchanged (checked on the device with random codes). The kernel therefore
// assigns k-slots to features and keys as it likes:
//   S^T = K . Q^T: register byte s of lane half h is feature 64*m + 32*h + s
//     for the product over features 64*m .. 64*m+63;
//   O^T += V^T . P^T: register byte s = 16*c + r of lane half h is key
//     32*h + 16*c + r of the 64-key tile.
// The first product's output row 32*c + 8*(r/4) + 4*h + r%4 (register r of
// accumulator c in lane half h) is the K tile's row of that index, and the K
// tile holds its keys permuted: row 32*c + 8*a + 4*h + b holds key
// 32*h + 16*c + 4*a + b. Register r of accumulator c in lane half h is then
// the score of key 32*h + 16*c + r, exactly the key of byte 16*c + r of the
// second product's B operand: P^T goes from the first product's output to the
// second one's B operand without leaving the lane, and the A operand of the
// second product (value feature f, keys 32*h .. 32*h+31) is one contiguous
// 32-byte run of the transposed V tile in key order. V is handed over
// transposed, [B][H][d][ldv] (ldv = N rounded up to 16), so its tile rows are
// runs of consecutive keys.
//
// P is rounded to e4m3 (v_cvt_pk_fp8_f32, round to nearest even) before the
// second product; P = 2^(x - m_used) <= 2^tau with tau <= 8, inside e4m3's
// range (448). The row sum is taken from the fp32 P before rounding.
//
// Layout: one workgroup = 4 wavefronts = 128 query rows of one (b, h), one
// query row per lane (the S and O accumulators hold one query column per
// lane), Q in registers; three workgroups share a compute unit at d = 128 (at
// most 168 registers per lane) and four at d = 64. K and
// V^T tiles of 64 keys go from memory straight into LDS (buffer loads with the
// LDS as destination, 16 bytes per lane), two tiles ahead of the products,
// into three buffers: step t waits for tile t's loads (issued two steps
// earlier), passes one barrier, issues tile t+2's loads into the buffer tile
// t-1 used, and computes tile t. The per-lane global addresses place each
// 16-byte chunk at its swizzled LDS position, so the tiles need no register
// staging and no LDS stores.
//
// REF = true instantiates a reference schedule for race checks: each tile is
// loaded into one buffer between two block-wide barriers, with every load
// complete before the second, and only then read. The arithmetic is the same
// instructions in the same order, so its results are bitwise equal to the
// pipelined schedule's.
#ifndef ATTN_FP8_KERNEL_H
#define ATTN_FP8_KERNEL_H

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "lds_dma.h"

namespace attn_fp8 {

using attn_dma::dma16;
using attn_dma::i32x4;
using attn_dma::rsrc_words;
using attn_dma::wait_barrier;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Wavefronts per workgroup (32 query rows each) for head dim D. Eight wavefronts
// at D = 128 (one workgroup per compute unit instead of two) measured within 2 % of
// four on an earlier form of this kernel.
template <int D>
struct Shape {
  static constexpr int NW = 4;
  static constexpr int ROWS = 32 * NW;  // query rows per workgroup
  static constexpr int PER_CU = D == 128 ? 3 : 4;  // workgroups per compute unit (registers, LDS)
};
constexpr int kMinRows = 128;  // smallest Shape<D>::ROWS
constexpr int kBC = 64;        // keys per tile

struct Fp8Params {
  const uint8_t* q;   // [B][H][N][D] e4m3
  const uint8_t* k;   // [B][H][N][D] e4m3
  const uint8_t* vt;  // [B][H][D][ldv] e4m3 (V transposed)
  __bf16* o;          // [B][H][N][D]
  float* lse;         // [B][H][N]
  int N;
  int ldv;
  int nq_tiles;       // ceil(N / Shape<D>::ROWS)
  int total_tiles;    // B * H * nq_tiles
  int n_xcd;          // XCDs of the device (workgroup slot i runs on XCD i % n_xcd)
  int per_xcd;        // ceil(total_tiles / n_xcd)
  int cus_per_xcd;    // compute units of one XCD
  float c;            // scale * q_scale * k_scale * log2(e) (> 0)
  float ov;           // v_scale
  float tau;          // rescale threshold, log2 units, in [0, 8]
  float psum_thr;     // 2^tau * (1 - 2^-10): a lane's partial sum above it may hide a P above 2^tau
};

// One matrix instruction: 32x32 fp32 += A (32 x 64 e4m3) . B (64 x 32 e4m3).
__device__ __forceinline__ f32x16 mma(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 16-byte chunk swizzles of the LDS tiles (chunk c of row r is stored at chunk
// position c ^ swz(r)). The reads take one logical chunk of 16 consecutive
// rows per 16 lanes (or of 8 rows per 8 lanes); the swizzles below make them
// hit distinct banks whether the LDS serves 128 or 256 bytes per pass (checked
// on the CPU against both bank models). The tile loads write whole 1 KiB runs.
// 128-byte rows (K at D = 128): chunk bits 0..2 from the row, bit 0 also from row bit 3.
// 64-byte rows (V^T, and K at D = 64): with a, b, c = row bits 1, 2, 3:
//   swz = 2 * (a ^ b) + (b ^ c).
__device__ __forceinline__ int vswz(int r) { return ((((r >> 1) ^ (r >> 2)) & 1) << 1) | (((r >> 2) ^ (r >> 3)) & 1); }
template <int D>
__device__ __forceinline__ int kswz(int r) {
  return D == 128 ? ((r & 7) ^ ((r >> 3) & 1)) : vswz(r);
}

__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource over `bytes` bytes at `base` (raw loads past the end return zeros;
// DATA_FORMAT = 32-bit in the third descriptor word, as raw loads require).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Direct-to-LDS loads of one 64-key tile: each instruction writes 1 KiB (16 bytes
// per lane, lane l at byte 16 l); K needs 64*D/1024 instructions, V^T as many.
template <int D>
struct TileLoads {
  static constexpr int NW = Shape<D>::NW;
  static constexpr int KI = kBC * D / 1024;  // K instructions per tile
  static constexpr int VI = D * kBC / 1024;  // V^T instructions per tile
  static constexpr int KPW = KI / NW;        // per wavefront
  static constexpr int VPW = VI / NW;
  static constexpr int PW = KPW + VPW;
  static_assert(KPW * NW == KI && VPW * NW == VI, "tile split");
};

// Byte offsets, relative to the tile's first key, of this lane's 16-byte chunks.
// K instruction i of wavefront w writes LDS bytes 1024 (i NW + w) .. +1023: lane
// l's chunk is tile row R = (that byte + 16 l) / D at chunk position p, i.e.
// logical chunk p ^ kswz(R) of the key the row holds, 32h + 16c + 4a + b for
// R = 32c + 8a + 4h + b. V^T: row F (feature) at chunk position p holds logical
// chunk p ^ vswz(F), keys 16 (p ^ vswz(F)) .. +15 of the tile.
template <int D>
__device__ __forceinline__ void load_offsets(uint32_t* koff, uint32_t* voff, int wave, int lane, int ldv) {
  using L = TileLoads<D>;
#pragma unroll
  for (int i = 0; i < L::KPW; ++i) {
    const int byte = 1024 * (i * L::NW + wave) + 16 * lane;
    const int R = byte / D, pos = (byte % D) / 16;
    const int c = R >> 5, a = (R >> 3) & 3, h = (R >> 2) & 1, b = R & 3;
    const int key = 32 * h + 16 * c + 4 * a + b;
    koff[i] = (uint32_t)(key * D + 16 * (pos ^ kswz<D>(R)));
  }
#pragma unroll
  for (int i = 0; i < L::VPW; ++i) {
    const int byte = 1024 * (i * L::NW + wave) + 16 * lane;
    const int F = byte / kBC, pos = (byte % kBC) / 16;
    voff[i] = (uint32_t)(F * ldv + 16 * (pos ^ vswz(F)));
  }
}

// Issue the loads of the tile at key j0 (live: the tile exists) into kb and vb.
// K reads through a resource that ends at row N, so keys past N load as zeros;
// V^T through one that ends at the head's end (the last tile's columns past N
// hold padding or the next row's keys; the products never see them, see
// mask_tail). A tile that does not exist loads zeros from an empty resource,
// so every step issues the same number of loads.
template <int D>
__device__ __forceinline__ void load_tile(const uint32_t* koff, const uint32_t* voff, const uint8_t* kh,
                                          const uint8_t* vth, int N, int ldv, int j0, bool live, char* kb, char* vb,
                                          int wave) {
  using L = TileLoads<D>;
  const uint32_t krec = __builtin_amdgcn_readfirstlane(live ? (uint32_t)(N - j0) * D : 0u);
  const uint32_t vrec = __builtin_amdgcn_readfirstlane(live ? (uint32_t)(D * ldv - j0) : 0u);
  const i32x4 kr = rsrc_words(kh + (size_t)(live ? j0 : 0) * D, krec);
  const i32x4 vr = rsrc_words(vth + (live ? j0 : 0), vrec);
  const uint32_t kl = attn_dma::lds_addr(kb) + 1024u * wave, vl = attn_dma::lds_addr(vb) + 1024u * wave;
#pragma unroll
  for (int i = 0; i < L::KPW; ++i) dma16(kr, koff[i], kl + 1024u * i * L::NW);
#pragma unroll
  for (int i = 0; i < L::VPW; ++i) dma16(vr, voff[i], vl + 1024u * i * L::NW);
}

// 32 bytes of row `r` starting at logical chunk `ch` (two swizzled 16-byte chunks).
template <int ROWB>
__device__ __forceinline__ i32x8 read32(const char* base, int r, int ch, int swz) {
  const u32x4 a = *(const u32x4*)(base + r * ROWB + ((ch ^ swz) << 4));
  const u32x4 b = *(const u32x4*)(base + r * ROWB + (((ch + 1) ^ swz) << 4));
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

// Zero the bytes of a V^T operand (keys 32 h .. 32 h + 31 of the tile) whose key is
// at or past `valid` (the real keys of the last tile).
__device__ __forceinline__ i32x8 mask_tail(i32x8 a, int h, int valid) {
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const int keep = valid - 32 * h - 4 * w;  // real bytes in word w
    const uint32_t m = keep >= 4 ? 0xFFFFFFFFu : keep <= 0 ? 0u : ((1u << (8 * keep)) - 1u);
    a[w] = (int)((uint32_t)a[w] & m);
  }
  return a;
}

template <int D, bool CAUSAL, bool REF = false>
__global__ void __launch_bounds__(64 * Shape<D>::NW, Shape<D>::PER_CU) attn_fwd_fp8_kernel(const Fp8Params p) {
  constexpr int kRows = Shape<D>::ROWS;
  constexpr int MQ = D / 64;  // QK products per 32-key block
  constexpr int MT = D / 32;  // PV products (value-feature blocks)
  using L = TileLoads<D>;
  __shared__ __attribute__((aligned(1024))) char kbuf0[kBC * D], kbuf1[kBC * D], kbuf2[kBC * D];
  __shared__ __attribute__((aligned(1024))) char vbuf0[D * kBC], vbuf1[D * kBC], vbuf2[D * kBC];

  // XCD-aware tile order: workgroups are dealt round-robin to the X XCDs, so slot
  // i runs tile (i % X) * per_xcd + i / X and each XCD works through a contiguous
  // range (the query tiles of a head share that XCD's L2 for their K/V reads).
  // Causal: longest query tiles first. When the range holds whole heads of no more
  // tiles than the XCD runs workgroups at once, it runs several heads together
  // anyway, and the range goes by tile rank first (every head's long tiles before
  // any short one); otherwise head by head, longest first within each.
  const int slot = blockIdx.x;
  const int x = slot % p.n_xcd, k = slot / p.n_xcd;  // XCD, position in its range
  int bh, qt;
  if (CAUSAL && p.per_xcd % p.nq_tiles == 0 && p.nq_tiles <= Shape<D>::PER_CU * p.cus_per_xcd) {
    const int heads = p.per_xcd / p.nq_tiles;
    bh = x * heads + k % heads;
    if (bh * p.nq_tiles >= p.total_tiles) return;
    qt = p.nq_tiles - 1 - k / heads;
  } else {
    const int tile = x * p.per_xcd + k;
    if (tile >= p.total_tiles) return;
    bh = tile / p.nq_tiles;
    qt = tile % p.nq_tiles;
    if (CAUSAL) qt = p.nq_tiles - 1 - qt;
  }

  const int tid = threadIdx.x;
  // wave index in a scalar register: the tile loads' LDS destinations are then scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l32 = lane & 31, hl = lane >> 5;
  const int N = p.N;
  const int ldv = p.ldv;
  const int q_base = qt * kRows;
  const int q0 = q_base + 32 * wave;  // this wavefront's first query row
  const int my_q = q0 + l32;

  const uint8_t* kh = p.k + (size_t)bh * N * D;
  const uint8_t* vth = p.vt + (size_t)bh * D * ldv;

  const int n_kv = (N + kBC - 1) / kBC;
  const int nt = CAUSAL ? min(n_kv, (q_base + kRows + kBC - 1) / kBC) : n_kv;

  uint32_t koff[L::KPW], voff[L::VPW];
  load_offsets<D>(koff, voff, wave, lane, ldv);

  // Q (B operand of S^T = K Q^T): features 64m + 32h .. +31 of row my_q. Loaded
  // after the first tiles' loads are issued and waited for at once (a wait the
  // compiler sees), so that its own wait insertion finds no load outstanding in
  // the tile loop.
  i32x8 qreg[MQ];
  auto load_q = [&] {
    const __amdgpu_buffer_rsrc_t qr = rsrc(p.q + (size_t)bh * N * D, (uint32_t)N * D);
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      const uint32_t off = (uint32_t)(my_q * D + 64 * m + 32 * hl);
      const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, off, 0, 0));
      const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, off + 16, 0, 0));
      qreg[m] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  };

  f32x16 oacc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) oacc[mt] = f32x16{};
  // P of the current tile (B operand of the second product). Each 32-bit word is
  // packed from four exponentials by two conversions that each write half of it;
  // the first one keeps the other half of the word it is given, here the previous
  // tile's P, which is dead by then (no separate zeroing per tile).
  i32x8 pb = {};
  // Per-lane byte offsets of a V^T operand in a tile buffer: row f = 32 mt + l32 at
  // logical chunks 2 hl and 2 hl + 1 (the swizzle depends on f's bits 1..3 only, so
  // value-feature block mt adds 32 mt rows, folded into the read instruction).
  const int vo0 = l32 * kBC + (((2 * hl) ^ vswz(l32)) << 4);
  const int vo1 = l32 * kBC + (((2 * hl + 1) ^ vswz(l32)) << 4);
  float m_used = -INFINITY, thr = -INFINITY, l_sum = 0.f;
  const float c = p.c, tau = p.tau, psum_thr = p.psum_thr;

  // Products and softmax of tile t from the LDS tiles kb (K, rows permuted) and vb (V^T).
  auto tile_step = [&](const char* kb, const char* vb, int t) __attribute__((always_inline)) {
    const int j0 = t * kBC;

    // S^T = K Q^T for the two 32-row blocks of the K tile
    f32x16 s[2];
    // Issue priority up while this wavefront feeds the matrix core, so the other
    // wavefronts' softmax work on the same SIMD does not delay its products.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      s[cc] = f32x16{};
      const int r = 32 * cc + l32;
#pragma unroll
      for (int m = 0; m < MQ; ++m) s[cc] = mma(read32<D>(kb, r, 4 * m + 2 * hl, kswz<D>(r)), qreg[m], s[cc]);
    }
    __builtin_amdgcn_s_setprio(0);

    // register r of block cc holds key j0 + 32 hl + 16 cc + r; mask keys past N and
    // (causal) keys after the query, on boundary tiles only
    const bool masked = (j0 + kBC > N) || (CAUSAL && j0 + kBC - 1 > q0);
    if (masked) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + 32 * hl + 16 * cc + r;
          const bool hide = key >= N || (CAUSAL && key > my_q);
          s[cc][r] = hide ? -INFINITY : s[cc][r];
        }
    }

    // P = 2^(s c - m) with the maximum in use and this lane's partial sum, packed to
    // e4m3: byte 16 cc + r of the B operand is register r of block cc.
    auto exponentials = [&](float mc) -> float {
      float part[2] = {0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          float e[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            e[b] = __builtin_amdgcn_exp2f(fmaf(s[cc][4 * a + b], c, mc));
            part[b & 1] += e[b];
          }
          int w = pb[4 * cc + a];
          w = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], w, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], w, true);
          pb[4 * cc + a] = w;
        }
      return part[0] + part[1];
    };
    // The tile maximum is needed only when a rescale may be due: a row whose tile
    // maximum exceeds m + tau has a P above 2^tau, so the partial sum of the lane
    // holding that key exceeds 2^tau. The exponentials are taken with the maximum
    // in use first; only a wavefront with such a sum (or with m still -inf, which
    // gives +inf or NaN) computes the exact tile maximum, applies the threshold
    // rule per row and takes the exponentials again.
    float tsum = exponentials(-m_used);
    if (__any(!(tsum <= psum_thr))) {
      float red = s[0][0];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int r = 0; r < 16; ++r) red = fmaxf(red, s[cc][r]);
      const float m_tile = pair_max(red) * c;  // c > 0; -inf if every key of the row is masked
      const bool need = m_tile > thr;
      if (__any(need)) {
        const float alpha = need ? __builtin_amdgcn_exp2f(m_used - m_tile) : 1.f;
        m_used = need ? m_tile : m_used;
        thr = m_used + tau;
        l_sum *= alpha;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[mt][r] *= alpha;
        tsum = exponentials(-m_used);
      }
    }
    l_sum += tsum;

    // O^T += V^T P^T: value features 32 mt + l32, keys 32 hl .. 32 hl + 31
    i32x8 va[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x4 a = *(const u32x4*)(vb + vo0 + 32 * kBC * mt);
      const u32x4 b = *(const u32x4*)(vb + vo1 + 32 * kBC * mt);
      va[mt] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    }
    if (j0 + kBC > N) {  // last tile: keys past N
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) va[mt] = mask_tail(va[mt], hl, N - j0);
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) oacc[mt] = mma(va[mt], pb, oacc[mt]);
    __builtin_amdgcn_s_setprio(0);
  };

  if (REF) {
    load_q();
    for (int t = 0; t < nt; ++t) {
      wait_barrier<0>();  // every wavefront is done reading the previous tile
      load_tile<D>(koff, voff, kh, vth, N, ldv, t * kBC, true, kbuf0, vbuf0, wave);
      wait_barrier<0>();  // this tile is in LDS for every wavefront
      tile_step(kbuf0, vbuf0, t);
    }
  } else {
    // Step t waits for tile t (this wavefront's loads of tile t+1 may still be in
    // flight: PW of them), passes the barrier (every wavefront's loads of tile t
    // landed and every wavefront finished step t-1, the last reader of the buffer
    // tile t+2 goes to), issues tile t+2 and computes tile t. Tile t's buffer is
    // buf[t % 3]; the loop is unrolled by three so the buffers are constants.
    load_tile<D>(koff, voff, kh, vth, N, ldv, 0, true, kbuf0, vbuf0, wave);
    load_tile<D>(koff, voff, kh, vth, N, ldv, kBC, nt > 1, kbuf1, vbuf1, wave);
    load_q();  // waits for tiles 0 and 1 too: they were issued at the same time
    auto step = [&](int t, const char* kb, const char* vb, char* kn, char* vn) __attribute__((always_inline)) {
      wait_barrier<L::PW>();
      load_tile<D>(koff, voff, kh, vth, N, ldv, (t + 2) * kBC, t + 2 < nt, kn, vn, wave);
      tile_step(kb, vb, t);
    };
    for (int t = 0; t < nt; t += 3) {
      step(t, kbuf0, vbuf0, kbuf2, vbuf2);
      if (t + 1 < nt) step(t + 1, kbuf1, vbuf1, kbuf0, vbuf0);
      if (t + 2 < nt) step(t + 2, kbuf2, vbuf2, kbuf1, vbuf1);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load into LDS outlives the workgroup

  const float l_tot = pair_sum(l_sum);
  // Lanes l and l ^ 32 hold the same row, lane half hl the features 32 mt + 8 gq +
  // 4 hl + e (register 4 gq + e). One lane-half exchange per pair of gq gives each
  // lane 8 consecutive features (gq = 2 pp + hl), stored as 16 bytes. The exchange
  // runs in every lane (a row past N only skips the stores).
  const float inv = p.ov / l_tot;
  u32x4 ob[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      bf16x4 a, b;  // gq = 2 pp (kept by hl = 0) and gq = 2 pp + 1 (kept by hl = 1)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = (__bf16)(oacc[mt][8 * pp + e] * inv);
        b[e] = (__bf16)(oacc[mt][8 * pp + 4 + e] * inv);
      }
      u32x2 x = __builtin_bit_cast(u32x2, a), y = __builtin_bit_cast(u32x2, b);
#pragma unroll
      for (int j = 0; j < 2; ++j) {  // x of the upper lane half <-> y of the lower lane half
        const auto r = __builtin_amdgcn_permlane32_swap(x[j], y[j], false, false);
        x[j] = r[0];
        y[j] = r[1];
      }
      ob[mt][pp] = u32x4{x[0], x[1], y[0], y[1]};
    }
  if (my_q < N) {
    const size_t row = (size_t)bh * N + my_q;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) *(u32x4*)(p.o + row * D + 32 * mt + 16 * pp + 8 * hl) = ob[mt][pp];
    if (hl == 0) p.lse[row] = 0.69314718055994531f * (m_used + log2f(l_tot));
  }
}

}  // namespace attn_fp8

#endif
