"""CPU oracle for exact attention (test infrastructure only).

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package. The product path (the HIP library and its Python
binding) never imports, links or calls it, and shares no code with it.
"""
from .exact import (  # noqa: F401
    attention,
    attention_rows,
    attention_probs,
    tiled_online_attention,
    brute_force_attention,
    attention_gqa,
    attention_gqa_rows,
    brute_force_attention_gqa,
    kv_head,
    attention_varlen,
    attention_varlen_rows,
    brute_force_attention_varlen,
)
from .fp8 import attention_fp8, attention_fp8_rows, fp8_error_bound, fp8_error_bound_rows, e4m3_decode  # noqa: F401
from .backward import attention_backward, attention_backward_rows, attention_backward_varlen  # noqa: F401
