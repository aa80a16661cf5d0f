// exp2_poly.h - software 2^x on the vector ALU (host and device).
//
// The pages describe replacing part of the hardware exponential with a cubic
// polynomial evaluated on the general-purpose FMA units, so that the special
// function unit stops limiting the softmax (page "FlashAttention 4: faster,
// more memory-efficient attention for LLMs", section "Software exponential on
// CUDA cores"; page "FlashAttention-4: algorithm-kernel fused pipeline for
// asymmetric hardware scaling", section 2). The routine here is our own:
//
//   2^x = 2^n * p(f),  n = floor(x), f = x - n in [0, 1),
//   p(f) = 1 + C1 f + C2 f^2 + C3 f^3  with p(0) = 1 and p(1) = 2 exactly,
//
// the coefficients being the discretised minimax (linear-programming) fit of
// the relative error of p(f) / 2^f on [0, 1], produced by gen_exp2_poly.py in
// this directory: max relative error 1.03e-4, below the bfloat16 half-ulp
// (2^-9) that the probabilities are rounded to afterwards. p(0) = 1 makes
// 2^0 = 1 exactly, as with the hardware instruction. Inputs below -150 are
// clamped to -150, where 2^n underflows to exactly 0: a masked key (x = -inf)
// gets P = 0, as with the hardware instruction.
#ifndef ATTN_EXP2_POLY_H
#define ATTN_EXP2_POLY_H

#include <math.h>

#define ATTN_EXP2_C1 6.954243183e-01f
#define ATTN_EXP2_C2 2.263074964e-01f
#define ATTN_EXP2_C3 7.826816291e-02f

#if defined(__HIPCC__)
#define ATTN_HD __host__ __device__
#else
#define ATTN_HD
#endif

ATTN_HD inline float attn_exp2_poly(float x) {
  x = fmaxf(x, -150.0f);
  const float n = floorf(x);
  const float f = x - n;
  const float p = fmaf(fmaf(fmaf(ATTN_EXP2_C3, f, ATTN_EXP2_C2), f, ATTN_EXP2_C1), f, 1.0f);
  return ldexpf(p, (int)n);
}

#endif
