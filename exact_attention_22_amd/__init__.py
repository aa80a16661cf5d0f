"""MI355X (gfx950) exact-attention forward: a HIP library behind a C ABI.

    from exact_attention_22_amd.binding import attention
    o, lse = attention(q, k, v, causal=True)

The library is built in-tree by `python -m exact_attention_22_amd.build`.
Importing this package loads nothing; `binding.lib()` loads the library on
first use and raises if it is missing.
"""
