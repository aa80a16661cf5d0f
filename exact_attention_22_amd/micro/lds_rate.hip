// lds_rate.hip - LDS throughput of one compute unit for the access forms the
// attention kernels use, with 4, 8 and 16 wavefronts per compute unit (one
// workgroup per unit, held there by its LDS size), shader clock from s_memtime:
//   ds_read_b128 at 16 consecutive bytes per lane (row fragments),
//   ds_read_b64_tr_b16 at 8 consecutive bytes per lane (transpose reads),
//   ds_read_b128 with two distinct addresses per wavefront (per-row vectors),
//   ds_write_b128 at 16 consecutive bytes per lane (P buffer),
//   ds_read_b32 at 4 consecutive bytes per lane.
// Each wavefront issues 16 accesses per loop iteration into distinct 1 KiB runs
// (no bank conflicts); results are kept live by empty asm uses, so no vector
// instruction runs beside them. Reported: bytes moved per shader-clock cycle per
// compute unit (sum over its wavefronts / the median wavefront's cycles).
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         exact_attention_22_amd/micro/lds_rate.hip -o _build/lds_rate
//   ./_build/lds_rate
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include <stdint.h>
#include <vector>
#include <algorithm>

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
// LDS-qualified types: volatile accesses through them stay ds_* instructions
typedef __attribute__((address_space(3))) char lchar;
typedef __attribute__((address_space(3))) f32x4 lf32x4;
typedef __attribute__((address_space(3))) float lfloat;
typedef __attribute__((address_space(3))) s16x4 ls16x4;

#define CHECK(x)                                                             \
  do {                                                                       \
    hipError_t e_ = (x);                                                     \
    if (e_ != hipSuccess) {                                                  \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                \
      exit(1);                                                               \
    }                                                                        \
  } while (0)

constexpr int kLds = 96 * 1024;  // one workgroup per compute unit
constexpr int kOps = 16;         // accesses per wavefront and iteration

template <int MODE>
__global__ void __launch_bounds__(1024) lds_kernel(int iters, unsigned long long* cyc, float seed) {
  __shared__ __attribute__((aligned(1024))) char lds[kLds];
  const int tid = threadIdx.x, lane = tid & 63;
  lchar* const L = (lchar*)lds;
  // fill what the reads touch (the first 32 KiB) so the values are defined
  for (int i = tid; i < 32 * 1024 / 4; i += blockDim.x) ((float*)lds)[i] = seed * i;
  __syncthreads();
  __builtin_amdgcn_s_waitcnt(0);
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    const int half = (it & 1) * 16384;  // two 16 KiB halves, alternated
    if (MODE == 0) {
      f32x4 x[kOps];
#pragma unroll
      for (int k = 0; k < kOps; ++k) x[k] = *(const volatile lf32x4*)(L + half + k * 1024 + lane * 16);
#pragma unroll
      for (int k = 0; k < kOps; ++k) asm volatile("" ::"v"(x[k]));
    } else if (MODE == 1) {
      s16x4 x[kOps];
#pragma unroll
      for (int k = 0; k < kOps; ++k)
        x[k] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ls16x4*)(L + half + k * 512 + lane * 8));
#pragma unroll
      for (int k = 0; k < kOps; ++k) asm volatile("" ::"v"(x[k]));
    } else if (MODE == 2) {
      f32x4 x[kOps];
#pragma unroll
      for (int k = 0; k < kOps; ++k) x[k] = *(const volatile lf32x4*)(L + half + k * 1024 + (lane >> 5) * 16);
#pragma unroll
      for (int k = 0; k < kOps; ++k) asm volatile("" ::"v"(x[k]));
    } else if (MODE == 3) {
      const f32x4 v = {seed, seed + 1.f, seed + 2.f, (float)it};
#pragma unroll
      for (int k = 0; k < kOps; ++k) *(volatile lf32x4*)(L + half + k * 1024 + lane * 16) = v;
    } else {
      float x[kOps];
#pragma unroll
      for (int k = 0; k < kOps; ++k) x[k] = *(const volatile lfloat*)(L + half + k * 256 + lane * 4);
#pragma unroll
      for (int k = 0; k < kOps; ++k) asm volatile("" ::"v"(x[k]));
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if (lane == 0) cyc[blockIdx.x * 16 + (tid >> 6)] = t1 - t0;
}

template <int MODE>
void run(int cus, int waves, unsigned long long* d_cyc, const char* name, int bytes_per_lane) {
  const int iters = 2048;
  for (int rep = 0; rep < 2; ++rep) {  // the first launch warms up
    hipLaunchKernelGGL(lds_kernel<MODE>, dim3(cus), dim3(64 * waves), 0, 0, iters, d_cyc, 0.5f);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
  }
  std::vector<unsigned long long> h(cus * 16);
  CHECK(hipMemcpy(h.data(), d_cyc, h.size() * 8, hipMemcpyDeviceToHost));
  std::vector<unsigned long long> t;
  for (int b = 0; b < cus; ++b)
    for (int w = 0; w < waves; ++w) t.push_back(h[b * 16 + w]);
  std::sort(t.begin(), t.end());
  const double cycles = (double)t[t.size() / 2];
  const double bytes = (double)waves * iters * kOps * 64 * bytes_per_lane;
  printf("  %-34s %2d waves/CU: %6.1f B/cycle/CU (%7.1f cycles per wavefront access)\n", name, waves, bytes / cycles,
         cycles / (iters * kOps));
}

int main() {
  int cus = 0;
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  unsigned long long* d_cyc;
  CHECK(hipMalloc(&d_cyc, (size_t)cus * 16 * 8));
  const int wv[3] = {4, 8, 16};
  for (int w : wv) run<0>(cus, w, d_cyc, "ds_read_b128 (16 B/lane)", 16);
  for (int w : wv) run<1>(cus, w, d_cyc, "ds_read_b64_tr_b16 (8 B/lane)", 8);
  for (int w : wv) run<2>(cus, w, d_cyc, "ds_read_b128, 2 addresses/wave", 16);
  for (int w : wv) run<3>(cus, w, d_cyc, "ds_write_b128 (16 B/lane)", 16);
  for (int w : wv) run<4>(cus, w, d_cyc, "ds_read_b32 (4 B/lane)", 4);
  printf("(bytes counted per lane, broadcast included; cycles from s_memtime)\n");
  CHECK(hipFree(d_cyc));
  return 0;
}
