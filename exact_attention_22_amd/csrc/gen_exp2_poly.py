"""Derive the cubic used by the kernel's software 2^x (prints the C constants).

Method: discretised minimax (Chebyshev) approximation solved as a linear
program. For f in [0, 1] we seek p(f) = 1 + c1 f + c2 f^2 + c3 f^3 (so
p(0) = 1 exactly) with p(1) = 2 exactly (continuous across integer x), that
minimises max |p(f) / 2^f - 1| over a dense grid. The pages only say the
polynomial is cubic and runs on the general-purpose FMA units (page
"FlashAttention 4: faster, more memory-efficient attention for LLMs", section
"Software exponential on CUDA cores"); the coefficients are ours.

Run:  python exact_attention_22_amd/csrc/gen_exp2_poly.py
"""
import numpy as np
from scipy.optimize import linprog


def solve(grid=20001):
    f = np.linspace(0.0, 1.0, grid)
    w = 2.0 ** -f                      # relative error weight
    # unknowns: c2, c3, t ; c1 = 1 - c2 - c3 (from p(1) = 2)
    # p(f) = 1 + f + c2 (f^2 - f) + c3 (f^3 - f)
    a2, a3 = (f * f - f) * w, (f ** 3 - f) * w
    r = (1.0 + f) * w - 1.0            # residual without c2, c3
    # |r + a2 c2 + a3 c3| <= t
    A = np.concatenate([np.stack([a2, a3, -np.ones_like(f)], 1),
                        np.stack([-a2, -a3, -np.ones_like(f)], 1)])
    b = np.concatenate([-r, r])
    res = linprog(c=[0, 0, 1], A_ub=A, b_ub=b, bounds=[(None, None)] * 3, method="highs")
    c2, c3, t = res.x
    return 1.0 - c2 - c3, c2, c3, t


if __name__ == "__main__":
    c1, c2, c3, t = solve()
    c = [np.float32(x) for x in (c1, c2, c3)]
    print(f"max rel err (exact coefficients) = {t:.3e}")
    for i, x in enumerate(c, 1):
        print(f"#define ATTN_EXP2_C{i} {float(x):.9e}f")
