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
//     32*c + 8*(r/4) + 4*h + r%4 of the 64-key tile - exactly the keys whose
//     scores lane l holds in register r of the S accumulator of key block c, so
//     P^T goes from the first product's output to the second one's B operand
//     without leaving the lane.
// The A operand of the second product (value feature f, those 32 keys) is one
// contiguous 32-byte run of the transposed V tile in LDS, because the tile's
// columns are stored permuted: key 32c + 8a + 4h + b sits at column
// 32h + 16c + 4a + b. V is handed over transposed, [B][H][d][ldv]
// (ldv = N rounded up to 16), so the kernel's loads of V^T rows are 16-byte
// runs of consecutive keys.
//
// P is rounded to e4m3 (v_cvt_pk_fp8_f32, round to nearest even) before the
// second product; P = 2^(x - m_used) <= 2^tau with tau <= 8, inside e4m3's
// range (448). The row sum is taken from the fp32 P before rounding.
//
// Layout: one workgroup = 4 wavefronts = 128 query rows of one (b, h), one
// query row per lane (the S and O accumulators hold one query column per
// lane), Q in registers. K and V^T tiles of 64 keys are staged through
// registers into double-buffered LDS, one barrier per tile: the global loads of
// tile t+1 are issued before tile t's products and written to the other buffer
// after them. Two workgroups share a compute unit.
//
// REF = true instantiates a reference schedule for race checks: each tile is
// loaded and stored to LDS between two block-wide barriers and only then read,
// with one buffer and no load in flight during the products. The arithmetic is
// the same instructions in the same order, so its results are bitwise equal to
// the pipelined schedule's.
#ifndef ATTN_FP8_KERNEL_H
#define ATTN_FP8_KERNEL_H

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

namespace attn_fp8 {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Wavefronts per workgroup (32 query rows each) for head dim D. Eight wavefronts
// at D = 128 (one workgroup per compute unit instead of two) measured within 2 %.
template <int D>
struct Shape {
  static constexpr int NW = 4;
  static constexpr int ROWS = 32 * NW;  // query rows per workgroup
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
  int per_xcd;        // ceil(total_tiles / 8)
  float c;            // scale * q_scale * k_scale * log2(e) (> 0)
  float ov;           // v_scale
  float tau;          // rescale threshold, log2 units, in [0, 8]
};

// One matrix instruction: 32x32 fp32 += A (32 x 64 e4m3) . B (64 x 32 e4m3).
__device__ __forceinline__ f32x16 mma(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 16-byte chunk swizzles of the LDS tiles (chunk c of row r is stored at chunk
// position c ^ swz(r)). The reads take one logical chunk of 16 consecutive
// rows per 16 lanes (or of 8 rows per 8 lanes); the V^T writes put 8-byte runs
// of 4 or 8 consecutive rows at two chunk positions. The swizzles below make
// all of these hit distinct banks whether the LDS serves 128 or 256 bytes per
// pass (checked on the CPU against both bank models).
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

// Per-thread staging of one tile: K rows (D bytes each) and V^T rows (64 keys each).
template <int D>
struct Stage {
  static constexpr int NT = 64 * Shape<D>::NW;  // threads
  static constexpr int KCH = kBC * D / 16 / NT;  // 16-byte K chunks per thread
  static constexpr int VCH = D * kBC / 16 / NT;  // 16-byte V^T chunks per thread
  static_assert(KCH * NT * 16 == kBC * D && VCH * NT * 16 == D * kBC, "tile split");
  u32x4 kc[KCH];
  u32x4 vc[VCH];
};

// Buffer resource over `bytes` bytes at `base` (raw loads past the end return zeros;
// DATA_FORMAT = 32-bit in the third descriptor word, as raw loads require).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Loads of the tile at key j0. K: a resource starting at row j0 and ending at row N,
// so rows past N read as zeros. V^T: a resource over the rest of the head from
// column j0; the per-thread offsets (koff, voff) are fixed for the whole kernel.
// Chunks at or past column N (only in the last tile) may hold padding or the next
// row's keys; `edge` zeroes those bytes (N - key bytes of the chunk are real keys).
template <int D>
__device__ __forceinline__ void stage_load(Stage<D>& st, const uint8_t* kh, const uint8_t* vth, int N, int ldv, int j0,
                                           const uint32_t (&koff)[Stage<D>::KCH],
                                           const uint32_t (&voff)[Stage<D>::VCH], int vkey, bool edge) {
  const __amdgpu_buffer_rsrc_t kr = rsrc(kh + (size_t)j0 * D, (uint32_t)(N - j0) * D);
  const __amdgpu_buffer_rsrc_t vr = rsrc(vth + j0, (uint32_t)(D * ldv - j0));
#pragma unroll
  for (int i = 0; i < Stage<D>::KCH; ++i)
    st.kc[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, koff[i], 0, 0));
#pragma unroll
  for (int i = 0; i < Stage<D>::VCH; ++i)
    st.vc[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vr, voff[i], 0, 0));
  if (edge) {
    const int valid = N - (j0 + vkey);  // real keys in this thread's V^T chunks (same column for every i)
#pragma unroll
    for (int i = 0; i < Stage<D>::VCH; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int keep = valid - 4 * e;  // bytes kept in word e
        const uint32_t m = keep >= 4 ? 0xFFFFFFFFu : keep <= 0 ? 0u : ((1u << (8 * keep)) - 1u);
        st.vc[i][e] &= m;
      }
  }
}

template <int D>
__device__ __forceinline__ void stage_store(const Stage<D>& st, char* kb, char* vb, int tid) {
  constexpr int KCPR = D / 16;
#pragma unroll
  for (int i = 0; i < Stage<D>::KCH; ++i) {
    const int id = tid + i * Stage<D>::NT;
    const int row = id / KCPR, ch = id % KCPR;
    *(u32x4*)(kb + row * D + ((ch ^ kswz<D>(row)) << 4)) = st.kc[i];
  }
#pragma unroll
  for (int i = 0; i < Stage<D>::VCH; ++i) {
    const int id = tid + i * Stage<D>::NT;
    const int f = id >> 2, jc = id & 3;
    // keys 16jc + e: e in {0..3, 8..11} (h = 0) and {4..7, 12..15} (h = 1); each set
    // lands as 8 contiguous bytes at column 32h + 16*(jc/2) + 8*(jc%2)
    const int c0 = 16 * (jc >> 1) + 8 * (jc & 1);
    const int c1 = 32 + c0;
    char* rowp = vb + f * kBC;
    *(u32x2*)(rowp + (((c0 >> 4) ^ vswz(f)) << 4) + (c0 & 15)) = u32x2{st.vc[i][0], st.vc[i][2]};
    *(u32x2*)(rowp + (((c1 >> 4) ^ vswz(f)) << 4) + (c1 & 15)) = u32x2{st.vc[i][1], st.vc[i][3]};
  }
}

// 32 bytes of row `r` starting at logical chunk `ch` (two swizzled 16-byte chunks).
template <int ROWB>
__device__ __forceinline__ i32x8 read32(const char* base, int r, int ch, int swz) {
  const u32x4 a = *(const u32x4*)(base + r * ROWB + ((ch ^ swz) << 4));
  const u32x4 b = *(const u32x4*)(base + r * ROWB + (((ch + 1) ^ swz) << 4));
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

template <int D, bool CAUSAL, bool REF = false>
__global__ void __launch_bounds__(64 * Shape<D>::NW, 8 / Shape<D>::NW) attn_fwd_fp8_kernel(const Fp8Params p) {
  constexpr int kRows = Shape<D>::ROWS;
  constexpr int MQ = D / 64;  // QK products per 32-key block
  constexpr int MT = D / 32;  // PV products (value-feature blocks)
  __shared__ __attribute__((aligned(16))) char kbuf[2][kBC * D];
  __shared__ __attribute__((aligned(16))) char vbuf[2][D * kBC];

  // XCD-aware tile order: workgroups are dealt round-robin to the 8 XCDs, so slot
  // i runs tile (i % 8) * per_xcd + i / 8 and each XCD works through a contiguous
  // range (the query tiles of a head share that XCD's L2 for their K/V reads).
  const int slot = blockIdx.x;
  const int tile = (slot & 7) * p.per_xcd + (slot >> 3);
  if (tile >= p.total_tiles) return;
  const int bh = tile / p.nq_tiles;
  int qt = tile % p.nq_tiles;
  if (CAUSAL) qt = p.nq_tiles - 1 - qt;  // longest query tiles first

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hl = lane >> 5;
  const int N = p.N;
  const int q_base = qt * kRows;
  const int q0 = q_base + 32 * wave;  // this wavefront's first query row
  const int my_q = q0 + l32;

  const uint8_t* kh = p.k + (size_t)bh * N * D;
  const uint8_t* vth = p.vt + (size_t)bh * D * p.ldv;

  // Q (B operand of S^T = K Q^T): features 64m + 32h .. +31 of row my_q.
  i32x8 qreg[MQ];
#pragma unroll
  for (int m = 0; m < MQ; ++m) {
    if (my_q < N) {
      const uint8_t* qp = p.q + ((size_t)bh * N + my_q) * D + 64 * m + 32 * hl;
      const u32x4 a = *(const u32x4*)qp, b = *(const u32x4*)(qp + 16);
      qreg[m] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    } else {
      qreg[m] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  const int n_kv = (N + kBC - 1) / kBC;
  const int nt = CAUSAL ? min(n_kv, (q_base + kRows + kBC - 1) / kBC) : n_kv;

  f32x16 oacc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) oacc[mt] = f32x16{};
  float m_used = -INFINITY, thr = -INFINITY, l_sum = 0.f;
  const float c = p.c, tau = p.tau;

  Stage<D> stg;
  uint32_t koff[Stage<D>::KCH], voff[Stage<D>::VCH];
#pragma unroll
  for (int i = 0; i < Stage<D>::KCH; ++i) {
    const int id = tid + i * Stage<D>::NT;
    koff[i] = (uint32_t)((id / (D / 16)) * D + 16 * (id % (D / 16)));
  }
  // V^T chunk id: feature id / 4, keys 16 * (id % 4) .. +15; id % 4 is the same for every i
  const int vkey = 16 * (tid & 3);
#pragma unroll
  for (int i = 0; i < Stage<D>::VCH; ++i) {
    const int id = tid + i * Stage<D>::NT;
    voff[i] = (uint32_t)((id >> 2) * p.ldv + 16 * (id & 3));
  }
  stage_load<D>(stg, kh, vth, N, p.ldv, 0, koff, voff, vkey, kBC > N);
  stage_store<D>(stg, kbuf[0], vbuf[0], tid);
  __syncthreads();

  // Products and softmax of tile t from the LDS tiles kb (K) and vb (V^T).
  auto tile_step = [&](const char* kb, const char* vb, int t) __attribute__((always_inline)) {
    const int j0 = t * kBC;

    // S^T = K Q^T for the two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      s[cc] = f32x16{};
      const int r = 32 * cc + l32;
#pragma unroll
      for (int m = 0; m < MQ; ++m) s[cc] = mma(read32<D>(kb, r, 4 * m + 2 * hl, kswz<D>(r)), qreg[m], s[cc]);
    }

    // mask keys past N and (causal) keys after the query, on boundary tiles only
    const bool masked = (j0 + kBC > N) || (CAUSAL && j0 + kBC - 1 > q0);
    if (masked) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + 32 * cc + 8 * (r / 4) + 4 * hl + (r % 4);
          const bool hide = key >= N || (CAUSAL && key > my_q);
          s[cc][r] = hide ? -INFINITY : s[cc][r];
        }
    }
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
    }
    // P = 2^(s c - m_used), fp32 row sum, packed to e4m3: byte 16cc + r of the B operand
    const float mc = -m_used;
    i32x8 pb;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float e[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          e[b] = __builtin_amdgcn_exp2f(fmaf(s[cc][4 * a + b], c, mc));
          l_sum += e[b];
        }
        int w = 0;
        w = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], w, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], w, true);
        pb[4 * cc + a] = w;
      }

    // O^T += V^T P^T: value features 32mt + l32, this lane half's 32 keys
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int f = 32 * mt + l32;
      oacc[mt] = mma(read32<kBC>(vb, f, 2 * hl, vswz(f)), pb, oacc[mt]);
    }
  };

  // One pipelined tile step; the loop below is unrolled by two so that each step's
  // LDS buffer (BUF) is a compile-time constant and the LDS addresses fold into the
  // instructions.
  auto step = [&](auto buf_tag, int t) {
    constexpr int BUF = decltype(buf_tag)::value;
    const int j0 = t * kBC;
    const bool more = t + 1 < nt;
    if (more) stage_load<D>(stg, kh, vth, N, p.ldv, j0 + kBC, koff, voff, vkey, j0 + 2 * kBC > N);
    tile_step(kbuf[BUF], vbuf[BUF], t);
    if (more) stage_store<D>(stg, kbuf[BUF ^ 1], vbuf[BUF ^ 1], tid);
    __syncthreads();
  };
  if (REF) {
    for (int t = 0; t < nt; ++t) {
      if (t > 0) {
        __syncthreads();
        stage_load<D>(stg, kh, vth, N, p.ldv, t * kBC, koff, voff, vkey, (t + 1) * kBC > N);
        stage_store<D>(stg, kbuf[0], vbuf[0], tid);
        __syncthreads();
      }
      tile_step(kbuf[0], vbuf[0], t);
    }
  } else {
    for (int t = 0; t < nt; t += 2) {
      step(std::integral_constant<int, 0>{}, t);
      if (t + 1 < nt) step(std::integral_constant<int, 1>{}, t + 1);
    }
  }


  const float l_tot = pair_sum(l_sum);
  if (my_q < N) {
    const float inv = p.ov / l_tot;
    const size_t row = (size_t)bh * N + my_q;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(oacc[mt][4 * gq + e] * inv);
        *(bf16x4*)(p.o + row * D + 32 * mt + 8 * gq + 4 * hl) = w;
      }
    if (hl == 0) p.lse[row] = 0.69314718055994531f * (m_used + log2f(l_tot));
  }
}

}  // namespace attn_fp8

#endif
