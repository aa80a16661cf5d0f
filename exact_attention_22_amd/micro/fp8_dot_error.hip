// fp8_dot_error.hip - error of the gfx950 e4m3 matrix-core dot product that the
// FP8 attention kernel uses for S = K Q^T (v_mfma_scale_f32_32x32x64_f8f6f4 with
// both block scales 2^0), against the exact dot product of the decoded codes.
//
// Each wavefront runs one 32x32x64 product on its own random codes. Lane l
// supplies 32 bytes of row l % 32 of each operand; both operands use the same
// k-slot assignment, so output (i, j) is the dot product of rows i and i + 32 of
// A's lanes with rows j and j + 32 of B's lanes over all 64 bytes, whatever the
// order the instruction gives the slots internally. The host decodes the codes
// from the e4m3 field layout (bias 7, subnormals, S.1111.111 = NaN, never drawn)
// and reports, per distribution, the largest |C - C_exact| / sum_k |a_k b_k|.
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         exact_attention_22_amd/micro/fp8_dot_error.hip -o _build/fp8_dot_error
//   ./_build/fp8_dot_error
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <vector>

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define CHECK(x)                                                                                \
  do {                                                                                          \
    hipError_t e_ = (x);                                                                        \
    if (e_ != hipSuccess) {                                                                     \
      fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_));         \
      exit(1);                                                                                  \
    }                                                                                           \
  } while (0)

// a, b: per wavefront 64 lanes x 32 bytes; c: per wavefront 64 lanes x 16 floats
__global__ void __launch_bounds__(256) dot_kernel(const i32x8* a, const i32x8* b, f32x16* c, int waves) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  if (w >= waves) return;
  f32x16 acc = {};
  // format 0 (e4m3) for both operands, block scale exponents 127 (2^0)
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[w * 64 + l], b[w * 64 + l], acc, 0, 0, 0, 127, 0, 127);
  c[w * 64 + l] = acc;
}

static double e4m3(uint8_t code) {
  const int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  const double v = e == 0 ? (m / 8.0) * ldexp(1.0, 1 - 7) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
  return s ? -v : v;
}

// Round to nearest e4m3 code (ties to even) by search over the finite codes.
static uint8_t to_e4m3(double x) {
  uint8_t best = 0;
  double bd = INFINITY;
  for (int c = 0; c < 256; ++c) {
    if ((c & 0x7F) == 0x7F) continue;
    const double d = fabs(e4m3((uint8_t)c) - x);
    if (d < bd || (d == bd && (c & 1) == 0)) {
      bd = d;
      best = (uint8_t)c;
    }
  }
  return best;
}

int main() {
  const int waves = 4096;
  const size_t bytes = (size_t)waves * 64 * 32;
  std::mt19937_64 rng(20241203);
  std::vector<uint8_t> a(bytes), b(bytes);
  std::vector<float> c((size_t)waves * 64 * 16);
  i32x8 *da, *db;
  f32x16* dc;
  CHECK(hipMalloc(&da, bytes));
  CHECK(hipMalloc(&db, bytes));
  CHECK(hipMalloc(&dc, c.size() * sizeof(float)));
  double dec[256];
  for (int i = 0; i < 256; ++i) dec[i] = e4m3((uint8_t)i);
  uint8_t table[4096];
  {  // N(0,1) draws quantised with scale amax/448 (amax about 4.5), as the workload generator does
    std::normal_distribution<double> nd(0.0, 1.0);
    for (int i = 0; i < 4096; ++i) table[i] = to_e4m3(nd(rng) * 448.0 / 4.5);
  }
  for (int dist = 0; dist < 2; ++dist) {
    for (size_t i = 0; i < bytes; ++i) {
      if (dist == 0) {  // every finite code equally likely: the widest exponent spread
        uint8_t x;
        do x = (uint8_t)(rng() & 0xFF); while ((x & 0x7F) == 0x7F);
        a[i] = x;
        do x = (uint8_t)(rng() & 0xFF); while ((x & 0x7F) == 0x7F);
        b[i] = x;
      } else {
        a[i] = table[rng() & 4095];
        b[i] = table[rng() & 4095];
      }
    }
    CHECK(hipMemcpy(da, a.data(), bytes, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(db, b.data(), bytes, hipMemcpyHostToDevice));
    hipLaunchKernelGGL(dot_kernel, dim3((waves + 3) / 4), dim3(256), 0, 0, da, db, dc, waves);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    CHECK(hipMemcpy(c.data(), dc, c.size() * sizeof(float), hipMemcpyDeviceToHost));
    double worst = 0.0, sum_rel = 0.0;
    long n = 0, exact = 0;
    for (int w = 0; w < waves; ++w) {
      const uint8_t* A = &a[(size_t)w * 64 * 32];
      const uint8_t* B = &b[(size_t)w * 64 * 32];
      for (int l = 0; l < 64; ++l)
        for (int r = 0; r < 16; ++r) {
          const int i = 8 * (r / 4) + 4 * (l / 32) + r % 4, j = l % 32;  // 32x32 accumulator layout
          double s = 0.0, t = 0.0;
          for (int h = 0; h < 2; ++h)
            for (int q = 0; q < 32; ++q) {
              const double p = dec[A[(i + 32 * h) * 32 + q]] * dec[B[(j + 32 * h) * 32 + q]];
              s += p;
              t += fabs(p);
            }
          const double got = c[((size_t)w * 64 + l) * 16 + r];
          if (t == 0.0) continue;
          const double rel = fabs(got - s) / t;
          worst = rel > worst ? rel : worst;
          sum_rel += rel;
          exact += got == s;
          ++n;
        }
    }
    printf("%s: %ld dot products of 64 e4m3 terms; max |C - exact| / sum|a_k b_k| = %.3e = 2^%.2f; "
           "mean %.3e; exact %.1f %%\n",
           dist == 0 ? "codes uniform over all finite e4m3 values" : "N(0,1) quantised with scale amax/448", n,
           worst, worst > 0 ? log2(worst) : -INFINITY, sum_rel / n, 100.0 * exact / n);
  }
  CHECK(hipFree(da));
  CHECK(hipFree(db));
  CHECK(hipFree(dc));
  return 0;
}
