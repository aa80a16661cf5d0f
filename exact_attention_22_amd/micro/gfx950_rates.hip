// gfx950_rates.hip - issue-rate and bandwidth microbenchmarks for the units the
// attention kernels share: LDS read bandwidth per compute unit (16-byte reads and
// the 8-byte transpose read), matrix-core products with vector work from the same
// or another wavefront, and matrix-core products fed from LDS.
//
// Every test launches one workgroup per compute unit (a 96 KiB LDS allocation
// keeps a second one off the unit), times each wavefront with the shader clock
// (s_memtime) and the 100 MHz constant clock (s_memrealtime), and prints the
// median over wavefronts of cycles per loop iteration, the derived rate, and the
// shader clock the run saw. All LDS addresses are masked into the allocation;
// results are stored to a per-thread slot so no load is dead.
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         exact_attention_22_amd/micro/gfx950_rates.hip -o _build/gfx950_rates
//   ./_build/gfx950_rates
#include <hip/hip_runtime.h>

#include <algorithm>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                      \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) {                                                           \
      fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
      exit(1);                                                                        \
    }                                                                                 \
  } while (0)

constexpr int LDS_BYTES = 96 * 1024;  // one workgroup per compute unit
constexpr int LDS_MASK = 64 * 1024 - 1;  // reads stay in the first 64 KiB

struct Stamp {
  unsigned long long c0, c1, w0, w1;
};

__device__ __forceinline__ void stamp_begin(Stamp& s) {
  __builtin_amdgcn_s_waitcnt(0);
  s.w0 = __builtin_amdgcn_s_memrealtime();
  s.c0 = __builtin_amdgcn_s_memtime();
}
__device__ __forceinline__ void stamp_end(Stamp& s) {
  __builtin_amdgcn_s_waitcnt(0);
  s.c1 = __builtin_amdgcn_s_memtime();
  s.w1 = __builtin_amdgcn_s_memrealtime();
}

// --- LDS read bandwidth -----------------------------------------------------
// Each wavefront reads U consecutive 1 KiB (b128) or 512 B (transpose) blocks per
// iteration; every lane's address is its own 16- or 8-byte slot in the block, so
// the reads are free of bank conflicts.
template <int KIND>  // 0: ds_read_b128, 1: ds_read_b64_tr_b16
__global__ void __launch_bounds__(1024) lds_read(int iters, Stamp* st, float* outf, float) {
  u32x4* out = (u32x4*)outf;
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid * 16; i < LDS_BYTES; i += blockDim.x * 16) *(u32x4*)(lds + i) = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  constexpr int U = 8;
  constexpr int BLK = KIND == 0 ? 1024 : 512;
  u32x4 acc = {0, 0, 0, 0};
  Stamp s;
  stamp_begin(s);
  for (int it = 0; it < iters; ++it) {
    // all U reads are issued before any result is used
    u32x4 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int a = (((it * U + u + wave * 7) * BLK) + lane * (BLK / 64)) & LDS_MASK;
      if (KIND == 0) {
        r[u] = *(const u32x4*)(lds + a);
      } else {
        const uint64_t t = __builtin_bit_cast(uint64_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) char*)(lds) + a)));
        r[u] = u32x4{(uint32_t)t, (uint32_t)(t >> 32), 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= r[u];
  }
  stamp_end(s);
  if (lane == 0) st[blockIdx.x * (blockDim.x / 64) + wave] = s;
  out[blockIdx.x * blockDim.x + tid] = acc;
}

// --- matrix core with vector work in the same wavefront -----------------------
// Per iteration: 4 independent v_mfma_f32_32x32x16_bf16 (128 cycles if the matrix
// core is the bound) and NF independent FMAs plus NE exp2 on separate registers,
// interleaved by the scheduler (sched_group_barrier) so that vector work follows
// each product. One wavefront per SIMD.
template <int NF, int NE, bool K16>
__global__ void __launch_bounds__(256) mfma_valu(int iters, Stamp* st, float* out, float seed) {
  extern __shared__ char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  bf16x8 a = {}, b = {};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (lane + i));
    b[i] = (__bf16)(seed * (lane - i));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  f32x4 d0 = {}, d1 = {}, d2 = {}, d3 = {};
  float f[16], e[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    f[i] = seed * (lane + i);
    e[i] = -seed * i;
  }
  Stamp s;
  stamp_begin(s);
  for (int it = 0; it < iters; ++it) {
    if (K16) {
      d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, d0, 0, 0, 0);
      d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, d1, 0, 0, 0);
      d2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, d2, 0, 0, 0);
      d3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, d3, 0, 0, 0);
    } else {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NF; ++i) f[i % 16] = fmaf(f[i % 16], 1.0001f, 0.5f);
#pragma unroll
    for (int i = 0; i < NE; ++i) e[i % 16] = __builtin_amdgcn_exp2f(e[i % 16]);
    // one product, then a quarter of the vector work, four times
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (NF + NE > 0) __builtin_amdgcn_sched_group_barrier(0x002, (NF + NE + 3) / 4, 0);
    }
  }
  stamp_end(s);
  if (lane == 0) st[blockIdx.x * (blockDim.x / 64) + wave] = s;
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += f[i] + e[i] + c0[i] + c1[i] + c2[i] + c3[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) r += d0[i] + d1[i] + d2[i] + d3[i];
  out[blockIdx.x * blockDim.x + tid] = r;
}

// --- two wavefronts per SIMD: one runs products, the other vector work ---------
// Wavefronts 0-3 run 4 products per iteration; wavefronts 4-7 run NF FMAs and NE
// exp2 per iteration (one of each kind per SIMD).
template <int NF, int NE>
__global__ void __launch_bounds__(512) mfma_beside_valu(int iters, Stamp* st, float* out, float seed) {
  extern __shared__ char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  bf16x8 a = {}, b = {};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (lane + i));
    b[i] = (__bf16)(seed * (lane - i));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  float f[16], e[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    f[i] = seed * (lane + i);
    e[i] = -seed * i;
  }
  Stamp s;
  stamp_begin(s);
  if (wave < 4) {
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
  } else {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < NF; ++i) f[i % 16] = fmaf(f[i % 16], 1.0001f, 0.5f);
#pragma unroll
      for (int i = 0; i < NE; ++i) e[i % 16] = __builtin_amdgcn_exp2f(e[i % 16]);
    }
  }
  stamp_end(s);
  if (lane == 0) st[blockIdx.x * (blockDim.x / 64) + wave] = s;
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += f[i] + e[i] + c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * blockDim.x + tid] = r;
}

// --- matrix core fed from LDS ---------------------------------------------------
// Per iteration each wavefront reads U 16-byte A operands (1 KiB per wave
// instruction, conflict-free) and runs U products with them against a B operand
// held in registers: the operand traffic of a product whose A side streams from
// LDS. W wavefronts per workgroup.
template <int U>
__global__ void __launch_bounds__(1024) mfma_from_lds(int iters, Stamp* st, float* out, float seed) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid * 16; i < LDS_BYTES; i += blockDim.x * 16) {
    bf16x8 v;
    for (int j = 0; j < 8; ++j) v[j] = (__bf16)(seed * ((i / 16 + j) & 31));
    *(bf16x8*)(lds + i) = v;
  }
  __syncthreads();
  bf16x8 b;
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = (__bf16)(seed * (lane - i));
  f32x16 c[4] = {};
  Stamp s;
  stamp_begin(s);
  for (int it = 0; it < iters; ++it) {
    bf16x8 a[U];
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = *(const bf16x8*)(lds + ((((it * U + u + wave * 5) * 1024) + lane * 16) & LDS_MASK));
#pragma unroll
    for (int u = 0; u < U; ++u) c[u & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b, c[u & 3], 0, 0, 0);
  }
  stamp_end(s);
  if (lane == 0) st[blockIdx.x * (blockDim.x / 64) + wave] = s;
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += c[0][i] + c[1][i] + c[2][i] + c[3][i];
  out[blockIdx.x * blockDim.x + tid] = r;
}

// --- LDS reads beside products / vector work in one wavefront ---------------------
// Per iteration: NM independent 32x32x16 products, NF independent FMAs and NR LDS
// reads (16-byte, or 8-byte transpose reads when TR), results kept live without
// extra instructions. One wavefront per SIMD. Shows which units an LDS read
// competes with for issue.
template <int NM, int NF, int NR, bool TR>
__global__ void __launch_bounds__(256) mix_lds(int iters, Stamp* st, float* out, float seed) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid * 16; i < LDS_BYTES; i += blockDim.x * 16) *(u32x4*)(lds + i) = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  bf16x8 a = {}, b = {};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (lane + i));
    b[i] = (__bf16)(seed * (lane - i));
  }
  f32x16 c[4] = {};
  float f[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) f[i] = seed * (lane + i);
  Stamp s;
  stamp_begin(s);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < NM; ++i) c[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[i & 3], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < NF; ++i) f[i % 16] = fmaf(f[i % 16], 1.0001f, 0.5f);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int addr = ((i * 1024 + wave * 4096) + lane * (TR ? 8 : 16)) & LDS_MASK;
      if (TR) {
        s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) char*)(lds) + addr));
        asm volatile("" ::"v"(r));
      } else {
        u32x4 r = *(const u32x4*)(lds + addr);
        asm volatile("" ::"v"(r));
      }
    }
  }
  stamp_end(s);
  if (lane == 0) st[blockIdx.x * (blockDim.x / 64) + wave] = s;
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += f[i] + c[0][i] + c[1][i] + c[2][i] + c[3][i];
  out[blockIdx.x * blockDim.x + tid] = r;
}

// --- softmax-like vector work -------------------------------------------------------
// Per iteration 16 scores (fresh each iteration: an empty asm marks them changed)
// each go through x = s*c - m (FMA); KIND 0 sums x, KIND 1 sums exp2(x), into NC
// partial sums, the pattern of the row sum. One wavefront per SIMD.
template <int KIND, int NC>
__global__ void __launch_bounds__(256) chains(int iters, Stamp* st, float* out, float seed) {
  extern __shared__ char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float sc[16], acc[NC];
#pragma unroll
  for (int i = 0; i < 16; ++i) sc[i] = seed * (lane - i);
#pragma unroll
  for (int i = 0; i < NC; ++i) acc[i] = 0.f;
  const float cc = 0.18f, m = seed * 3.f;
  Stamp s;
  stamp_begin(s);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      asm volatile("" : "+v"(sc[j]));
      const float x = fmaf(sc[j], cc, -m);
      acc[j % NC] += KIND ? __builtin_amdgcn_exp2f(x) : x;
    }
  }
  stamp_end(s);
  if (lane == 0) st[blockIdx.x * (blockDim.x / 64) + wave] = s;
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) r += acc[i];
  out[blockIdx.x * blockDim.x + tid] = r;
}

// --- LDS read bursts ----------------------------------------------------------------
// Per iteration each wavefront issues 8 reads back to back into distinct registers
// and waits for them inside the same asm block (the outputs are written when the
// block ends), so the loop measures LDS read throughput per wavefront. 16-byte
// reads cover 8 KiB, transpose reads 4 KiB, conflict-free. With PROD, wavefronts
// 0-3 instead run 4 products per iteration beside the reading wavefronts 4-7.
template <bool TR, bool PROD>
__global__ void __launch_bounds__(1024) lds_burst(int iters, Stamp* st, float* out, float seed) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid * 16; i < LDS_BYTES; i += blockDim.x * 16) *(u32x4*)(lds + i) = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  // byte address within the first 64 KiB; 8 blocks of 1 KiB (512 B) from it stay below 64 KiB
  const uint32_t base = (uint32_t)(size_t)(lds) + (((wave & 7) * 8192 + lane * (TR ? 8 : 16)) & (LDS_MASK >> 1));
  u32x4 x = {0, 0, 0, 0};
  bf16x8 a = {}, b = {};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (lane + i));
    b[i] = (__bf16)(seed * (lane - i));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  Stamp s;
  stamp_begin(s);
  if (PROD && wave < 4) {
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
  } else {
    for (int it = 0; it < iters; ++it) {
      if (TR) {
        uint64_t r0, r1, r2, r3, r4, r5, r6, r7;
        asm volatile(
            "ds_read_b64_tr_b16 %0, %8 offset:0\n\tds_read_b64_tr_b16 %1, %8 offset:512\n\t"
            "ds_read_b64_tr_b16 %2, %8 offset:1024\n\tds_read_b64_tr_b16 %3, %8 offset:1536\n\t"
            "ds_read_b64_tr_b16 %4, %8 offset:2048\n\tds_read_b64_tr_b16 %5, %8 offset:2560\n\t"
            "ds_read_b64_tr_b16 %6, %8 offset:3072\n\tds_read_b64_tr_b16 %7, %8 offset:3584\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=v"(r0), "=v"(r1), "=v"(r2), "=v"(r3), "=v"(r4), "=v"(r5), "=v"(r6), "=v"(r7)
            : "v"(base));
        x.x ^= (uint32_t)(r0 ^ r7);  // every read has completed inside the asm block
      } else {
        u32x4 r0, r1, r2, r3, r4, r5, r6, r7;
        asm volatile(
            "ds_read_b128 %0, %8 offset:0\n\tds_read_b128 %1, %8 offset:1024\n\t"
            "ds_read_b128 %2, %8 offset:2048\n\tds_read_b128 %3, %8 offset:3072\n\t"
            "ds_read_b128 %4, %8 offset:4096\n\tds_read_b128 %5, %8 offset:5120\n\t"
            "ds_read_b128 %6, %8 offset:6144\n\tds_read_b128 %7, %8 offset:7168\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=v"(r0), "=v"(r1), "=v"(r2), "=v"(r3), "=v"(r4), "=v"(r5), "=v"(r6), "=v"(r7)
            : "v"(base));
        x.x ^= r0.x ^ r7.w;  // every read has completed inside the asm block
      }
    }
  }
  stamp_end(s);
  if (lane == 0) st[blockIdx.x * (blockDim.x / 64) + wave] = s;
  float r = (float)(x.x ^ x.y ^ x.z ^ x.w);
#pragma unroll
  for (int i = 0; i < 16; ++i) r += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * blockDim.x + tid] = r;
}

// --- vector work beside LDS traffic ---------------------------------------------------
// Wavefronts 4-7 run 32 independent FMAs per iteration. Wavefronts 8-11 (RD) read
// LDS in bursts of 8 (16-byte or transpose reads) and wavefronts 0-3 (MM) run 4
// products per iteration; absent roles idle. Each SIMD holds one of each role.
template <bool MM, int RD>  // RD: 0 none, 1 ds_read_b128, 2 ds_read_b64_tr_b16
__global__ void __launch_bounds__(768) valu_beside(int iters, Stamp* st, float* out, float seed) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid * 16; i < LDS_BYTES; i += blockDim.x * 16) *(u32x4*)(lds + i) = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  const uint32_t base = (uint32_t)(size_t)(lds) + (((wave & 7) * 8192 + lane * (RD == 2 ? 8 : 16)) & (LDS_MASK >> 1));
  bf16x8 a = {}, b = {};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (lane + i));
    b[i] = (__bf16)(seed * (lane - i));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  float f[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) f[i] = seed * (lane + i);
  uint32_t x = 0;
  Stamp s;
  stamp_begin(s);
  const int role = wave >> 2;  // 0: products, 1: FMAs, 2: LDS reads
  if (role == 0) {
    if (MM)
      for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
      }
  } else if (role == 1) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 32; ++i) f[i % 16] = fmaf(f[i % 16], 1.0001f, 0.5f);
    }
  } else if (RD == 1) {
    for (int it = 0; it < iters * 2; ++it) {
      u32x4 r0, r1, r2, r3, r4, r5, r6, r7;
      asm volatile(
          "ds_read_b128 %0, %8 offset:0\n\tds_read_b128 %1, %8 offset:1024\n\t"
          "ds_read_b128 %2, %8 offset:2048\n\tds_read_b128 %3, %8 offset:3072\n\t"
          "ds_read_b128 %4, %8 offset:4096\n\tds_read_b128 %5, %8 offset:5120\n\t"
          "ds_read_b128 %6, %8 offset:6144\n\tds_read_b128 %7, %8 offset:7168\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=v"(r0), "=v"(r1), "=v"(r2), "=v"(r3), "=v"(r4), "=v"(r5), "=v"(r6), "=v"(r7)
          : "v"(base));
      x ^= r0.x ^ r7.w;  // every read has completed inside the asm block
    }
  } else if (RD == 2) {
    for (int it = 0; it < iters * 2; ++it) {
      uint64_t r0, r1, r2, r3, r4, r5, r6, r7;
      asm volatile(
          "ds_read_b64_tr_b16 %0, %8 offset:0\n\tds_read_b64_tr_b16 %1, %8 offset:512\n\t"
          "ds_read_b64_tr_b16 %2, %8 offset:1024\n\tds_read_b64_tr_b16 %3, %8 offset:1536\n\t"
          "ds_read_b64_tr_b16 %4, %8 offset:2048\n\tds_read_b64_tr_b16 %5, %8 offset:2560\n\t"
          "ds_read_b64_tr_b16 %6, %8 offset:3072\n\tds_read_b64_tr_b16 %7, %8 offset:3584\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=v"(r0), "=v"(r1), "=v"(r2), "=v"(r3), "=v"(r4), "=v"(r5), "=v"(r6), "=v"(r7)
          : "v"(base));
      x ^= (uint32_t)(r0 ^ r7);  // every read has completed inside the asm block
    }
  }
  stamp_end(s);
  if (lane == 0) st[blockIdx.x * (blockDim.x / 64) + wave] = s;
  float r = (float)x;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += f[i] + c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * blockDim.x + tid] = r;
}

// ---------------------------------------------------------------------------------
struct Result {
  double cyc_per_iter, mhz;
};

// Median over the wavefronts whose index within the workgroup lies in [w0, w1).
static Result summarise(const std::vector<Stamp>& s, int iters, int wpb, int w0, int w1) {
  std::vector<double> cyc, mhz;
  for (size_t i = 0; i < s.size(); ++i) {
    const int w = (int)(i % wpb);
    if (w < w0 || w >= w1) continue;
    const Stamp& x = s[i];
    const double c = (double)(x.c1 - x.c0), t = (double)(x.w1 - x.w0);
    cyc.push_back(c / iters);
    if (t > 0) mhz.push_back(c / t * 100.0);
  }
  std::sort(cyc.begin(), cyc.end());
  std::sort(mhz.begin(), mhz.end());
  return {cyc[cyc.size() / 2], mhz.empty() ? 0.0 : mhz[mhz.size() / 2]};
}

typedef void (*KernelFn)(int, Stamp*, float*, float);

// Two launches (the first warms the clock); returns the stamps of the second.
static std::vector<Stamp> launch(KernelFn kernel, int blocks, int threads, int iters, Stamp* d_st, void* d_out,
                                 float seed) {
  const int waves = blocks * threads / 64;
  CHECK(hipMemset(d_st, 0, sizeof(Stamp) * waves));
  for (int rep = 0; rep < 2; ++rep) {
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(threads), LDS_BYTES, 0, iters, d_st, (float*)d_out, seed);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
  }
  std::vector<Stamp> h(waves);
  CHECK(hipMemcpy(h.data(), d_st, sizeof(Stamp) * waves, hipMemcpyDeviceToHost));
  return h;
}

static Result run(KernelFn kernel, int blocks, int threads, int iters, Stamp* d_st, void* d_out, float seed) {
  const int wpb = threads / 64;
  return summarise(launch(kernel, blocks, threads, iters, d_st, d_out, seed), iters, wpb, 0, wpb);
}

int main() {
  int dev = 0, cus = 0;
  CHECK(hipGetDevice(&dev));
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, dev));
  printf("device %s (%s), %d compute units\n", prop.name, prop.gcnArchName, cus);
  const int blocks = cus;
  Stamp* d_st;
  void* d_out;
  CHECK(hipMalloc(&d_st, sizeof(Stamp) * blocks * 16));
  CHECK(hipMalloc(&d_out, sizeof(u32x4) * blocks * 1024));
  for (auto k : {(const void*)lds_read<0>, (const void*)lds_read<1>, (const void*)mfma_from_lds<4>,
                 (const void*)mfma_from_lds<8>})
    CHECK(hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES));

  printf("\n[LDS read bandwidth] one workgroup per CU, 8 conflict-free reads per wavefront per iteration\n");
  for (int kind = 0; kind < 2; ++kind)
    for (int w : {4, 8, 16}) {
      const int iters = 4096;
      Result r = run(kind == 0 ? lds_read<0> : lds_read<1>, blocks, 64 * w, iters, d_st, d_out, 0.f);
      const double bytes = (double)w * 8 * (kind == 0 ? 1024 : 512);
      printf("  %-18s waves/CU %2d: %7.1f cycles/iter  -> %6.1f bytes/clk/CU  (sclk %4.0f MHz)\n",
             kind == 0 ? "ds_read_b128" : "ds_read_b64_tr_b16", w, r.cyc_per_iter, bytes / r.cyc_per_iter, r.mhz);
    }

  printf("\n[products fed from LDS] U 16-byte A-operand reads + U 32x32x16 bf16 products per iteration\n");
  for (int w : {4, 8, 16})
    for (int u : {4, 8}) {
      const int iters = 2048;
      Result r = run(u == 4 ? mfma_from_lds<4> : mfma_from_lds<8>, blocks, 64 * w, iters, d_st, d_out, 0.001f);
      const double per_simd = (double)w / 4 * u * 32;  // matrix-core cycles per SIMD per iteration
      printf("  waves/CU %2d U %d: %7.1f cycles/iter, matrix core busy %5.1f %%, LDS %6.1f bytes/clk/CU (sclk %4.0f)\n",
             w, u, r.cyc_per_iter, 100.0 * per_simd / r.cyc_per_iter, (double)w * u * 1024 / r.cyc_per_iter, r.mhz);
    }

  printf("\n[products and vector work in one wavefront] 1 wavefront per SIMD, 4 products per iteration\n");
#define MV(NF, NE, K16)                                                                                      \
  {                                                                                                          \
    Result r = run(mfma_valu<NF, NE, K16>, blocks, 256, 4096, d_st, d_out, 0.001f);                         \
    printf("  %s + %2d FMA + %2d exp2: %7.1f cycles/iter (products alone %d)  (sclk %4.0f)\n",              \
           K16 ? "4x 16x16x32" : "4x 32x32x16", NF, NE, r.cyc_per_iter, K16 ? 64 : 128, r.mhz);              \
  }
  MV(0, 0, false) MV(8, 0, false) MV(16, 0, false) MV(20, 0, false) MV(24, 0, false) MV(28, 0, false)
  MV(32, 0, false) MV(0, 4, false) MV(0, 8, false) MV(0, 12, false) MV(0, 16, false) MV(16, 8, false)
  MV(12, 8, false) MV(0, 0, true) MV(8, 0, true) MV(12, 0, true)

  printf("\n[LDS read bursts] 8 reads back to back, one wait, per wavefront and iteration\n");
  for (int tr = 0; tr < 2; ++tr)
    for (int w : {4, 8, 16}) {
      KernelFn f = tr ? lds_burst<true, false> : lds_burst<false, false>;
      CHECK(hipFuncSetAttribute((const void*)f, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES));
      Result r = run(f, blocks, 64 * w, 2048, d_st, d_out, 0.f);
      const double bytes = 8.0 * (tr ? 512 : 1024);
      printf("  %-18s waves/CU %2d: %6.1f cycles/burst -> %5.1f bytes/clk per wavefront, %6.1f per CU (sclk %4.0f)\n",
             tr ? "ds_read_b64_tr_b16" : "ds_read_b128", w, r.cyc_per_iter, bytes / r.cyc_per_iter,
             bytes * w / r.cyc_per_iter, r.mhz);
    }
  for (int tr = 0; tr < 2; ++tr) {
    KernelFn f = tr ? lds_burst<true, true> : lds_burst<false, true>;
    CHECK(hipFuncSetAttribute((const void*)f, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES));
    std::vector<Stamp> h = launch(f, blocks, 512, 2048, d_st, d_out, 0.001f);
    Result m = summarise(h, 2048, 8, 0, 4), v = summarise(h, 2048, 8, 4, 8);
    printf("  4 products | burst of 8 %-18s: product waves %6.1f, reading waves %6.1f cycles/iter (sclk %4.0f)\n",
           tr ? "ds_read_b64_tr_b16" : "ds_read_b128", m.cyc_per_iter, v.cyc_per_iter, m.mhz);
  }

  printf("\n[vector work beside LDS reads and products] per SIMD: one FMA wavefront (32 FMAs per iteration),\n"
         "  optionally one product wavefront (4 products per iteration) and one LDS-reading wavefront\n");
#define VB(MM, RD)                                                                                          \
  {                                                                                                         \
    CHECK(hipFuncSetAttribute((const void*)valu_beside<MM, RD>, hipFuncAttributeMaxDynamicSharedMemorySize, \
                              LDS_BYTES));                                                                  \
    std::vector<Stamp> h = launch(valu_beside<MM, RD>, blocks, 768, 2048, d_st, d_out, 0.001f);            \
    Result m = summarise(h, 2048, 12, 0, 4), v = summarise(h, 2048, 12, 4, 8),                              \
           l = summarise(h, 2048 * 2, 12, 8, 12);                                                           \
    printf("  products %-3s reads %-18s: FMA waves %6.1f, product waves %6.1f, reading waves %6.1f cycles/iter (sclk %4.0f)\n", \
           MM ? "yes" : "no", RD == 0 ? "none" : RD == 1 ? "ds_read_b128" : "ds_read_b64_tr_b16",          \
           v.cyc_per_iter, MM ? m.cyc_per_iter : 0.0, RD ? l.cyc_per_iter : 0.0, v.mhz);                    \
  }
  VB(false, 0) VB(false, 1) VB(false, 2) VB(true, 0) VB(true, 1) VB(true, 2)

  printf("\n[LDS reads beside products and vector work] 1 wavefront per SIMD; per iteration\n");
#define ML(NM, NF, NR, TR)                                                                                     \
  {                                                                                                            \
    CHECK(hipFuncSetAttribute((const void*)mix_lds<NM, NF, NR, TR>, hipFuncAttributeMaxDynamicSharedMemorySize, \
                              LDS_BYTES));                                                                     \
    Result r = run(mix_lds<NM, NF, NR, TR>, blocks, 256, 2048, d_st, d_out, 0.001f);                         \
    printf("  %d products + %2d FMA + %2d %s: %7.1f cycles/iter (sclk %4.0f)\n", NM, NF, NR,                   \
           TR ? "ds_read_b64_tr_b16" : "ds_read_b128", r.cyc_per_iter, r.mhz);                                  \
  }
  ML(0, 0, 16, false) ML(0, 0, 16, true) ML(0, 16, 0, false) ML(0, 16, 16, false) ML(0, 16, 16, true)
  ML(4, 0, 0, false) ML(4, 0, 4, false) ML(4, 0, 8, false) ML(4, 0, 16, false) ML(4, 0, 8, true)
  ML(4, 0, 16, true) ML(4, 12, 4, false) ML(4, 12, 8, true)

  printf("\n[softmax-like vector work] 1 wavefront per SIMD; 16 scores per iteration: FMA (+exp2) + add into NC sums\n");
#define CH(KIND, NC)                                                                                          \
  {                                                                                                           \
    Result r = run(chains<KIND, NC>, blocks, 256, 4096, d_st, d_out, 0.001f);                                \
    printf("  %s, %d partial sums: %7.1f cycles/iter = %5.2f cycles per score (sclk %4.0f)\n",               \
           KIND ? "FMA+exp2+add" : "FMA+add", NC, r.cyc_per_iter, r.cyc_per_iter / 16, r.mhz);                \
  }
  CH(0, 1) CH(0, 2) CH(0, 4) CH(1, 1) CH(1, 2) CH(1, 4)

  printf("\n[two wavefronts per SIMD] wavefronts 0-3: 4 products per iteration; 4-7: vector work\n");
#define MB(NF, NE)                                                                                           \
  {                                                                                                          \
    std::vector<Stamp> h = launch(mfma_beside_valu<NF, NE>, blocks, 512, 4096, d_st, d_out, 0.001f);       \
    Result m = summarise(h, 4096, 8, 0, 4), v = summarise(h, 4096, 8, 4, 8);                                 \
    printf("  4 products | %2d FMA + %2d exp2: product waves %7.1f, vector waves %7.1f cycles/iter (sclk %4.0f)\n", \
           NF, NE, m.cyc_per_iter, v.cyc_per_iter, m.mhz);                                                   \
  }
  MB(0, 0) MB(16, 0) MB(24, 0) MB(28, 0) MB(32, 0) MB(0, 8) MB(0, 12) MB(0, 16)
  CHECK(hipFree(d_st));
  CHECK(hipFree(d_out));
  return 0;
}
