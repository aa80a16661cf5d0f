// mfma_issue.hip - issue cost of matrix-core products beside vector FMAs in the
// same wavefront (one wavefront per SIMD, one workgroup per compute unit, shader
// clock from s_memtime, median over wavefronts):
//   bf16 v_mfma_f32_32x32x16_bf16 with the accumulators in VGPRs, in AGPRs (inline
//   asm, "a" constraint) and with C = 0 (no accumulator input);
//   fp8 v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales in a VGPR) and the plain
//   v_mfma_f32_32x32x64_f8f6f4, plus a check that the two give the same bits.
// Every product and FMA is inline asm so their order is the one written.
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         exact_attention_22_amd/micro/mfma_issue.hip -o _build/mfma_issue
//   ./_build/mfma_issue
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include <stdint.h>
#include <vector>
#include <algorithm>
#include <string.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define CHECK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_)); exit(1);} } while (0)

template <int MODE, int NF>
__global__ void __launch_bounds__(256) k(int iters, unsigned long long* cyc, float* out, float seed) {
  const int tid = threadIdx.x, lane = tid & 63;
  __shared__ char pad[96 * 1024];  // one workgroup per compute unit
  if (seed < -1.f) pad[tid * 256] = (char)tid;
  bf16x8 a = {}, b = {};
#pragma unroll
  for (int i = 0; i < 8; ++i) { a[i] = (__bf16)(seed * (lane + i)); b[i] = (__bf16)(seed * (lane - i)); }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  i32x8 a8, b8;
#pragma unroll
  for (int i = 0; i < 8; ++i) { a8[i] = (int)(0x38383838u + lane + i); b8[i] = (int)(0x30303030u + lane * i); }
  const int sc127 = 127 + (int)(seed * 0.f);
  float f[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) f[i] = seed * (lane + i);
  __builtin_amdgcn_s_waitcnt(0);
  unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    f32x16* cs[4] = {&c0, &c1, &c2, &c3};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (MODE == 0) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(*cs[g]) : "v"(a), "v"(b));
      else if (MODE == 1) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(*cs[g]) : "v"(a), "v"(b));
      else if (MODE == 2) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(*cs[g]) : "v"(a), "v"(b));
      else if (MODE == 3)
        asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
                     : "+v"(*cs[g]) : "v"(a8), "v"(b8), "v"(sc127));
      else asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(*cs[g]) : "v"(a8), "v"(b8));
#pragma unroll
      for (int i = 0; i < NF / 4; ++i) {
        const int j = (g * (NF / 4) + i) % 16;
        asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(f[j]) : "v"(seed), "v"(1.0f));
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if (lane == 0) cyc[blockIdx.x * 4 + (tid >> 6)] = t1 - t0;
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += f[i] + c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * blockDim.x + tid] = r + (seed < -1.f ? (float)pad[tid * 256 + 1] : 0.f);
}

__global__ void cmp_fp8(const int* in, float* out) {
  const int lane = threadIdx.x;
  i32x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) { a[i] = in[lane * 8 + i]; b[i] = in[512 + lane * 8 + i]; }
  f32x16 c0 = {}, c1 = {};
  c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 127, 0, 127);
  c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, 0, 0, 0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 16; ++i) { out[lane * 16 + i] = c0[i]; out[1024 + lane * 16 + i] = c1[i]; }
}

template <int MODE, int NF>
void run(int cus, unsigned long long* d_cyc, float* d_out, const char* name) {
  const int iters = 4096;
  hipLaunchKernelGGL((k<MODE, NF>), dim3(cus), dim3(256), 0, 0, iters, d_cyc, d_out, 0.001f);
  CHECK(hipDeviceSynchronize());
  hipLaunchKernelGGL((k<MODE, NF>), dim3(cus), dim3(256), 0, 0, iters, d_cyc, d_out, 0.001f);
  CHECK(hipDeviceSynchronize());
  std::vector<unsigned long long> h(cus * 4);
  CHECK(hipMemcpy(h.data(), d_cyc, h.size() * 8, hipMemcpyDeviceToHost));
  std::sort(h.begin(), h.end());
  printf("  %-22s + %2d FMA: %7.1f cycles/iter\n", name, NF, (double)h[h.size() / 2] / iters);
}

int main() {
  int cus = 0;
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  unsigned long long* d_cyc; float* d_out;
  CHECK(hipMalloc(&d_cyc, cus * 4 * 8));
  CHECK(hipMalloc(&d_out, cus * 256 * 4));
  {
    std::vector<int> h(1024);
    uint32_t x = 12345u;
    for (auto& v : h) { x = x * 1664525u + 1013904223u; uint32_t w = x;
      // clear NaN codes (S.1111.111) byte by byte
      for (int k2 = 0; k2 < 4; ++k2) if (((w >> (8 * k2)) & 0x7F) == 0x7F) w &= ~(1u << (8 * k2));
      v = (int)w; }
    int* d_in; float* d_o;
    CHECK(hipMalloc(&d_in, 1024 * 4)); CHECK(hipMalloc(&d_o, 2048 * 4));
    CHECK(hipMemcpy(d_in, h.data(), 4096, hipMemcpyHostToDevice));
    hipLaunchKernelGGL(cmp_fp8, dim3(1), dim3(64), 0, 0, d_in, d_o);
    CHECK(hipDeviceSynchronize());
    std::vector<float> o(2048);
    CHECK(hipMemcpy(o.data(), d_o, 8192, hipMemcpyDeviceToHost));
    int diff = 0, nz = 0;
    for (int i = 0; i < 1024; ++i) { diff += memcmp(&o[i], &o[1024 + i], 4) != 0; nz += o[i] != 0.f; }
    printf("plain vs scale(127) fp8 product: %d of 1024 outputs differ bitwise (%d nonzero); sample %g %g\n", diff, nz, o[0], o[1024]);
  }
#define R(M, NF, N) run<M, NF>(cus, d_cyc, d_out, N)
  R(0, 0, "vgpr acc (builtin)"); R(0, 8, "vgpr acc (builtin)"); R(0, 16, "vgpr acc (builtin)"); R(0, 24, "vgpr acc (builtin)"); R(0, 32, "vgpr acc (builtin)");
  R(1, 0, "agpr acc (asm)"); R(1, 8, "agpr acc (asm)"); R(1, 16, "agpr acc (asm)"); R(1, 24, "agpr acc (asm)"); R(1, 32, "agpr acc (asm)");
  R(2, 0, "vgpr, C=0 (asm)"); R(2, 8, "vgpr, C=0 (asm)"); R(2, 16, "vgpr, C=0 (asm)"); R(2, 24, "vgpr, C=0 (asm)"); R(2, 32, "vgpr, C=0 (asm)");
  R(3, 0, "fp8 scale form"); R(3, 8, "fp8 scale form"); R(3, 16, "fp8 scale form"); R(3, 32, "fp8 scale form"); R(3, 48, "fp8 scale form");
  R(4, 0, "fp8 plain form"); R(4, 8, "fp8 plain form"); R(4, 16, "fp8 plain form"); R(4, 32, "fp8 plain form"); R(4, 48, "fp8 plain form");
  printf("(4 products per iteration; shader-clock cycles from s_memtime)\n");
  return 0;
}
