"""ctypes binding of libattn_fwd.so (argument marshalling only).

Every step of the attention forward runs inside the HIP library. PyTorch only
provides device memory and the current stream. If the library is missing the
calls raise; there is no other code path.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# EXACT_ATTN_LIB selects another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("EXACT_ATTN_LIB") or os.path.join(_PKG, "libattn_fwd.so")

ATTN_OK = 0
STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_DIM", 3: "ATTN_ERR_UNSUPPORTED",
          4: "ATTN_ERR_MISALIGNED", 5: "ATTN_ERR_SCALE", 6: "ATTN_ERR_ALIAS", 7: "ATTN_ERR_HIP",
          8: "ATTN_ERR_OPTS"}
O_BF16, O_F32 = 0, 1
EXPORTS = ["attn_fwd", "attn_fwd_ex", "attn_fwd_check", "attn_fwd_opts_init", "attn_status_str",
           "attn_last_error", "attn_abi_version", "attn_exp2_poly_host", "attn_fwd_tile_shape",
           "attn_fwd_gqa", "attn_fwd_gqa_check", "attn_fwd_varlen", "attn_fwd_varlen_check",
           "attn_bwd", "attn_bwd_check", "attn_fwd_splitkv", "attn_fwd_splitkv_workspace_size",
           "attn_fwd_fp8", "attn_fwd_fp8_check", "attn_bwd_varlen", "attn_bwd_varlen_check",
           "attn_fwd_splitkv_noalloc", "attn_fwd_fp8_ex", "attn_bwd_ex"]
ABI_VERSION = 10
SCHEDULE_PIPELINED, SCHEDULE_REFERENCE = 0, 1
NOALLOC_SCRATCH_BYTES = 64 << 20  # ATTN_NOALLOC_SCRATCH_BYTES


class AttnFwdOpts(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_size_t), ("rescale_tau_log2", ctypes.c_float),
                ("exp2_poly_eighths", ctypes.c_int), ("o_dtype", ctypes.c_int),
                ("rescale_count", ctypes.c_void_p), ("schedule", ctypes.c_int)]


class AttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m exact_attention_22_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        tensor_args = [vp, vp, vp, vp, vp, i, i, i, i, i, f]
        L.attn_fwd.argtypes = tensor_args + [vp]
        L.attn_fwd.restype = i
        L.attn_fwd_ex.argtypes = tensor_args + [ctypes.POINTER(AttnFwdOpts), vp]
        L.attn_fwd_ex.restype = i
        L.attn_fwd_check.argtypes = tensor_args + [ctypes.POINTER(AttnFwdOpts)]
        L.attn_fwd_check.restype = i
        gqa_args = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, ctypes.POINTER(AttnFwdOpts)]
        L.attn_fwd_gqa.argtypes = gqa_args + [vp]
        L.attn_fwd_gqa.restype = i
        L.attn_fwd_gqa_check.argtypes = gqa_args
        L.attn_fwd_gqa_check.restype = i
        varlen_args = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, ctypes.POINTER(AttnFwdOpts)]
        L.attn_fwd_varlen.argtypes = varlen_args + [vp]
        L.attn_fwd_varlen.restype = i
        L.attn_fwd_varlen_check.argtypes = varlen_args
        L.attn_fwd_varlen_check.restype = i
        L.attn_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, ctypes.c_size_t,
                                       ctypes.POINTER(AttnFwdOpts), vp]
        L.attn_fwd_splitkv.restype = i
        L.attn_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i,
                                               ctypes.POINTER(AttnFwdOpts), vp]
        L.attn_fwd_splitkv_noalloc.restype = i
        L.attn_fwd_splitkv_workspace_size.argtypes = [i, i, i, i, i]
        L.attn_fwd_splitkv_workspace_size.restype = ctypes.c_size_t
        bwd_args = [vp] * 10 + [i, i, i, i, i, i, f]
        L.attn_bwd.argtypes = bwd_args + [vp]
        L.attn_bwd.restype = i
        L.attn_bwd_ex.argtypes = bwd_args + [i, vp]
        L.attn_bwd_ex.restype = i
        L.attn_bwd_check.argtypes = bwd_args
        L.attn_bwd_check.restype = i
        bwdv_args = [vp] * 11 + [i, i, i, i, i, i, i, f]
        L.attn_bwd_varlen.argtypes = bwdv_args + [vp]
        L.attn_bwd_varlen.restype = i
        L.attn_bwd_varlen_check.argtypes = bwdv_args
        L.attn_bwd_varlen_check.restype = i
        fp8_args = [vp, vp, vp, vp, vp, i, i, i, i, i, f, f, f, f, f]
        L.attn_fwd_fp8.argtypes = fp8_args + [vp]
        L.attn_fwd_fp8.restype = i
        L.attn_fwd_fp8_ex.argtypes = fp8_args + [i, vp]
        L.attn_fwd_fp8_ex.restype = i
        L.attn_fwd_fp8_check.argtypes = fp8_args
        L.attn_fwd_fp8_check.restype = i
        L.attn_fwd_opts_init.argtypes = [ctypes.POINTER(AttnFwdOpts)]
        L.attn_fwd_opts_init.restype = None
        L.attn_status_str.argtypes = [i]
        L.attn_status_str.restype = ctypes.c_char_p
        L.attn_last_error.argtypes = []
        L.attn_last_error.restype = ctypes.c_char_p
        L.attn_abi_version.argtypes = []
        L.attn_abi_version.restype = i
        L.attn_exp2_poly_host.argtypes = [vp, vp, ctypes.c_size_t]
        L.attn_exp2_poly_host.restype = None
        L.attn_fwd_tile_shape.argtypes = [i, ctypes.POINTER(i), ctypes.POINTER(i)]
        L.attn_fwd_tile_shape.restype = i
        _lib = L
    return _lib


def make_opts(tau: float = 8.0, poly_eighths: int = 0, o_dtype: int = O_BF16, rescale_count: int | None = None,
              schedule: int = SCHEDULE_PIPELINED):
    opts = AttnFwdOpts()
    lib().attn_fwd_opts_init(ctypes.byref(opts))
    opts.rescale_tau_log2 = tau
    opts.exp2_poly_eighths = poly_eighths
    opts.o_dtype = o_dtype
    opts.rescale_count = rescale_count
    opts.schedule = schedule
    return opts


def tile_shape(d: int) -> tuple[int, int]:
    """(query rows per workgroup, keys per KV tile) of the kernel for head dim d."""
    rows, keys = ctypes.c_int(), ctypes.c_int()
    st = lib().attn_fwd_tile_shape(d, ctypes.byref(rows), ctypes.byref(keys))
    if st != ATTN_OK:
        raise AttnError(st, last_error())
    return rows.value, keys.value


def last_error() -> str:
    return lib().attn_last_error().decode()


def attn_fwd(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, d: int, causal: int,
             scale: float, stream: int | None) -> int:
    """The C entry point with raw device addresses; returns the status code."""
    return lib().attn_fwd(q, k, v, o, lse, B, H, N, d, int(causal), scale, stream)


def attn_fwd_ex(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, d: int, causal: int,
                scale: float, opts: AttnFwdOpts | None, stream: int | None) -> int:
    return lib().attn_fwd_ex(q, k, v, o, lse, B, H, N, d, int(causal), scale,
                             ctypes.byref(opts) if opts is not None else None, stream)


def attn_fwd_check(q, k, v, o, lse, B, H, N, d, causal, scale, opts: AttnFwdOpts | None = None) -> int:
    return lib().attn_fwd_check(q, k, v, o, lse, B, H, N, d, int(causal), scale,
                                ctypes.byref(opts) if opts is not None else None)


def attn_fwd_gqa(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Hkv: int, N: int, d: int,
                 causal: int, scale: float, opts: AttnFwdOpts | None, stream: int | None) -> int:
    return lib().attn_fwd_gqa(q, k, v, o, lse, B, H, Hkv, N, d, int(causal), scale,
                              ctypes.byref(opts) if opts is not None else None, stream)


def attn_fwd_gqa_check(q, k, v, o, lse, B, H, Hkv, N, d, causal, scale, opts: AttnFwdOpts | None = None) -> int:
    return lib().attn_fwd_gqa_check(q, k, v, o, lse, B, H, Hkv, N, d, int(causal), scale,
                                    ctypes.byref(opts) if opts is not None else None)


def attn_fwd_varlen(q: int, k: int, v: int, o: int, lse: int, cu: int, B: int, H: int, Hkv: int, total: int,
                    max_seqlen: int, d: int, causal: int, scale: float, opts: AttnFwdOpts | None,
                    stream: int | None) -> int:
    return lib().attn_fwd_varlen(q, k, v, o, lse, cu, B, H, Hkv, total, max_seqlen, d, int(causal), scale,
                                 ctypes.byref(opts) if opts is not None else None, stream)


def attn_fwd_varlen_check(q, k, v, o, lse, cu, B, H, Hkv, total, max_seqlen, d, causal, scale,
                          opts: AttnFwdOpts | None = None) -> int:
    return lib().attn_fwd_varlen_check(q, k, v, o, lse, cu, B, H, Hkv, total, max_seqlen, d, int(causal), scale,
                                       ctypes.byref(opts) if opts is not None else None)


def _check_tensor(name, t, shape=None, device=None):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous [B,H,N,d]")
    if t.dim() != 4 or (shape is not None and tuple(t.shape) != shape):
        raise ValueError(f"{name} must have shape {shape or '[B,H,N,d]'}, got {tuple(t.shape)}")


def _check_buffer(name, t, dtype, shape, device):
    """A caller-supplied output or workspace: the C layer cannot see its size, dtype
    or device, so all of them are checked here before its address is passed on."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
              scale: float | None = None, *, tau: float = 8.0, poly_eighths: int = 0,
              out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
              lse: torch.Tensor | None = None, rescale_count: bool = False, schedule: int = SCHEDULE_PIPELINED):
    """Exact attention forward on the current stream: returns (O, LSE[, rescale counts]).

    q: bfloat16 [B,H,N,d]; k, v: bfloat16 [B,Hkv,N,d] with Hkv dividing H (Hkv < H is
    grouped-query attention: query head h reads key/value head h // (H // Hkv)); all
    contiguous device tensors. scale defaults to 1/sqrt(d) (as a float32). O has
    `out_dtype` (bfloat16 or float32); LSE is float32 [B,H,N]. schedule =
    SCHEDULE_REFERENCE runs the race-check schedule (bitwise the same results).
    """
    _check_tensor("q", q)
    shape = tuple(q.shape)
    B, H, N, d = shape
    _check_tensor("k", k)
    Hkv = k.shape[1]
    _check_tensor("k", k, (B, Hkv, N, d), q.device)
    _check_tensor("v", v, (B, Hkv, N, d), q.device)
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32).item())
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be bfloat16 or float32")
    if out is None:
        out = torch.empty(shape, dtype=out_dtype, device=q.device)
    _check_buffer("out", out, out_dtype, shape, q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_buffer("lse", lse, torch.float32, (B, H, N), q.device)
    counts = torch.empty((B, H, N), dtype=torch.int32, device=q.device) if rescale_count else None
    opts = make_opts(tau, poly_eighths, O_F32 if out_dtype == torch.float32 else O_BF16,
                     counts.data_ptr() if counts is not None else None, schedule)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    if Hkv == H:
        st = attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                         B, H, N, d, causal, scale, opts, stream)
    else:
        st = attn_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                          B, H, Hkv, N, d, causal, scale, opts, stream)
    if st != ATTN_OK:
        raise AttnError(st, last_error())
    return (out, lse, counts) if rescale_count else (out, lse)


def attention_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                     max_seqlen: int | None = None, causal: bool = False, scale: float | None = None, *,
                     tau: float = 8.0, poly_eighths: int = 0, out_dtype: torch.dtype = torch.bfloat16,
                     out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                     rescale_count: bool = False, schedule: int = SCHEDULE_PIPELINED):
    """Attention over packed variable-length sequences on the current stream.

    q: bfloat16 [H,total,d]; k, v: bfloat16 [Hkv,total,d]; cu_seqlens: int32 [B+1]
    device tensor of cumulative lengths (0, ..., total). max_seqlen defaults to the
    longest sequence, read back from cu_seqlens (one device-to-host copy). Returns
    (O [H,total,d], LSE [H,total][, rescale counts]).
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be a bfloat16 CUDA (HIP) tensor")
        if t.dim() != 3 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [heads,total,d] tensor, got {tuple(t.shape)}")
        if t.device != q.device:
            raise ValueError(f"{name} must be on {q.device}, got {t.device}")
    H, T, d = q.shape
    Hkv = k.shape[0]
    if tuple(k.shape) != (Hkv, T, d) or tuple(v.shape) != (Hkv, T, d):
        raise ValueError(f"k and v must be [Hkv,{T},{d}], got {tuple(k.shape)} {tuple(v.shape)}")
    if (not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1
            or cu_seqlens.device != q.device or not cu_seqlens.is_contiguous()):
        raise TypeError("cu_seqlens must be a contiguous int32 [B+1] tensor on q's device")
    B = cu_seqlens.numel() - 1
    if B < 0:
        raise ValueError("cu_seqlens needs at least one entry")
    if max_seqlen is None:
        max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if B > 0 else 0
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32).item())
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be bfloat16 or float32")
    if out is None:
        out = torch.empty((H, T, d), dtype=out_dtype, device=q.device)
    _check_buffer("out", out, out_dtype, (H, T, d), q.device)
    if lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    _check_buffer("lse", lse, torch.float32, (H, T), q.device)
    counts = torch.empty((H, T), dtype=torch.int32, device=q.device) if rescale_count else None
    opts = make_opts(tau, poly_eighths, O_F32 if out_dtype == torch.float32 else O_BF16,
                     counts.data_ptr() if counts is not None else None, schedule)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = attn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                         cu_seqlens.data_ptr(), B, H, Hkv, T, max_seqlen, d, causal, scale, opts, stream)
    if st != ATTN_OK:
        raise AttnError(st, last_error())
    return (out, lse, counts) if rescale_count else (out, lse)


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Hkv, N, d, causal, scale, stream) -> int:
    """The C entry point with raw device addresses; returns the status code."""
    return lib().attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Hkv, N, d, int(causal), scale, stream)


def attn_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Hkv, N, d, causal, scale, schedule, stream) -> int:
    """The C entry point with a kernel schedule; returns the status code."""
    return lib().attn_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Hkv, N, d, int(causal), scale, schedule,
                             stream)


def attn_bwd_check(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Hkv, N, d, causal, scale) -> int:
    return lib().attn_bwd_check(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Hkv, N, d, int(causal), scale)


def attention_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                       dout: torch.Tensor, causal: bool = False, scale: float | None = None, *,
                       dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
                       dv: torch.Tensor | None = None, delta: torch.Tensor | None = None,
                       schedule: int = SCHEDULE_PIPELINED):
    """Exact attention backward on the current stream: returns (dQ, dK, dV, delta).

    q, o, dout: bfloat16 [B,H,N,d]; k, v: bfloat16 [B,Hkv,N,d]; lse: float32 [B,H,N]
    (o and lse from the forward pass with the same causal flag and scale). delta
    (float32 [B,H,N]) holds D_i = dout_i . o_i. schedule=SCHEDULE_REFERENCE computes
    dK and dV with the one-wavefront kernel (the race check of attn_bwd_ex).
    """
    _check_tensor("q", q)
    B, H, N, d = q.shape
    _check_tensor("k", k)
    Hkv = k.shape[1]
    _check_tensor("k", k, (B, Hkv, N, d), q.device)
    _check_tensor("v", v, (B, Hkv, N, d), q.device)
    _check_tensor("o", o, (B, H, N, d), q.device)
    _check_tensor("dout", dout, (B, H, N, d), q.device)
    if (not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N)
            or not lse.is_contiguous() or lse.device != q.device):
        raise TypeError("lse must be a contiguous float32 [B,H,N] tensor on q's device")
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32).item())
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if delta is None else delta
    for name, t, shape in (("dq", dq, (B, H, N, d)), ("dk", dk, (B, Hkv, N, d)), ("dv", dv, (B, Hkv, N, d))):
        _check_tensor(name, t, shape, q.device)
    _check_buffer("delta", delta, torch.float32, (B, H, N), q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = attn_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                     dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H, Hkv, N, d, causal, scale,
                     schedule, stream)
    if st != ATTN_OK:
        raise AttnError(st, last_error())
    return dq, dk, dv, delta


def splitkv_workspace_size(B: int, H: int, N: int, d: int, n_splits: int = 0) -> int:
    return int(lib().attn_fwd_splitkv_workspace_size(B, H, N, d, n_splits))


def attention_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                      scale: float | None = None, n_splits: int = 0, *, tau: float = 8.0,
                      out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                      lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                      schedule: int = SCHEDULE_PIPELINED):
    """Exact attention with split keys (n_splits units per query tile, 0 = automatic),
    merged by log-sum-exp weights. Same shapes and results (up to rounding) as
    `attention`. `workspace`: a uint8 device tensor of at least
    splitkv_workspace_size(...) bytes (allocated here when not given)."""
    _check_tensor("q", q)
    B, H, N, d = q.shape
    _check_tensor("k", k)
    Hkv = k.shape[1]
    _check_tensor("k", k, (B, Hkv, N, d), q.device)
    _check_tensor("v", v, (B, Hkv, N, d), q.device)
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32).item())
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be bfloat16 or float32")
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=q.device)
    _check_buffer("out", out, out_dtype, (B, H, N, d), q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_buffer("lse", lse, torch.float32, (B, H, N), q.device)
    need = splitkv_workspace_size(B, H, N, d, n_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check_buffer("workspace", workspace, torch.uint8, None, q.device)
    if workspace.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 tensor")
    opts = make_opts(tau, 0, O_F32 if out_dtype == torch.float32 else O_BF16, None, schedule)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = lib().attn_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H,
                                Hkv, N, d, int(causal), scale, n_splits, workspace.data_ptr(),
                                workspace.numel() * workspace.element_size(), ctypes.byref(opts), stream)
    if st != ATTN_OK:
        raise AttnError(st, last_error())
    return out, lse


def attention_splitkv_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                              lse: torch.Tensor, causal: bool = False, scale: float | None = None,
                              n_splits: int = 0, *, tau: float = 8.0):
    """attention_splitkv without a workspace: the partial results go to the library's
    device scratch array (NOALLOC_SCRATCH_BYTES per GPU). The caller passes the
    outputs (out: bfloat16 or float32 [B,H,N,d], lse: float32 [B,H,N]); nothing is
    allocated here either. Calls that overlap on one GPU race. Returns (out, lse)."""
    _check_tensor("q", q)
    B, H, N, d = q.shape
    _check_tensor("k", k)
    Hkv = k.shape[1]
    _check_tensor("k", k, (B, Hkv, N, d), q.device)
    _check_tensor("v", v, (B, Hkv, N, d), q.device)
    if not isinstance(out, torch.Tensor) or out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be a bfloat16 or float32 tensor")
    _check_buffer("out", out, out.dtype, (B, H, N, d), q.device)
    _check_buffer("lse", lse, torch.float32, (B, H, N), q.device)
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32).item())
    opts = make_opts(tau, 0, O_F32 if out.dtype == torch.float32 else O_BF16, None)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = lib().attn_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                        B, H, Hkv, N, d, int(causal), scale, n_splits, ctypes.byref(opts), stream)
    if st != ATTN_OK:
        raise AttnError(st, last_error())
    return out, lse


def attn_fwd_fp8(q, k, vt, o, lse, B, H, N, d, causal, scale, q_scale, k_scale, v_scale, tau, stream) -> int:
    """The C entry point with raw device addresses; returns the status code."""
    return lib().attn_fwd_fp8(q, k, vt, o, lse, B, H, N, d, int(causal), scale, q_scale, k_scale, v_scale, tau,
                              stream)


def attn_fwd_fp8_ex(q, k, vt, o, lse, B, H, N, d, causal, scale, q_scale, k_scale, v_scale, tau, schedule,
                    stream) -> int:
    """The C entry point with a kernel schedule; returns the status code."""
    return lib().attn_fwd_fp8_ex(q, k, vt, o, lse, B, H, N, d, int(causal), scale, q_scale, k_scale, v_scale, tau,
                                 schedule, stream)


def attn_fwd_fp8_check(q, k, vt, o, lse, B, H, N, d, causal, scale, q_scale, k_scale, v_scale, tau) -> int:
    return lib().attn_fwd_fp8_check(q, k, vt, o, lse, B, H, N, d, int(causal), scale, q_scale, k_scale, v_scale,
                                    tau)


def fp8_ldv(N: int) -> int:
    """Row length of the transposed V operand: N rounded up to a multiple of 16."""
    return (N + 15) // 16 * 16


def attention_fp8(q: torch.Tensor, k: torch.Tensor, vt: torch.Tensor, scales, causal: bool = False,
                  scale: float | None = None, *, tau: float = 8.0, out: torch.Tensor | None = None,
                  lse: torch.Tensor | None = None, schedule: int = SCHEDULE_PIPELINED):
    """FP8 exact attention forward on the current stream: returns (O bf16 [B,H,N,d], LSE fp32 [B,H,N]).

    q, k: e4m3 codes [B,H,N,d] (uint8 or torch.float8_e4m3fn); vt: V transposed, e4m3 codes
    [B,H,d,ldv] with ldv = fp8_ldv(N) (padding columns unused); scales = (q_scale, k_scale,
    v_scale), the per-tensor dequantisation factors; scale defaults to 1/sqrt(d).
    """
    def codes(name, t):
        if not isinstance(t, torch.Tensor) or t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError(f"{name} must be a uint8 or float8_e4m3fn tensor")
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise TypeError(f"{name} must be a contiguous 4-d CUDA tensor")
        return t
    codes("q", q)
    B, H, N, d = q.shape
    codes("k", k)
    codes("vt", vt)
    if tuple(k.shape) != (B, H, N, d):
        raise ValueError(f"k must be [{B},{H},{N},{d}], got {tuple(k.shape)}")
    if tuple(vt.shape) != (B, H, d, fp8_ldv(N)):
        raise ValueError(f"vt must be [{B},{H},{d},{fp8_ldv(N)}], got {tuple(vt.shape)}")
    if k.device != q.device or vt.device != q.device:
        raise ValueError("q, k and vt must be on one device")
    qs, ks, vs = (float(x) for x in scales)
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32).item())
    out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_buffer("out", out, torch.bfloat16, (B, H, N, d), q.device)
    _check_buffer("lse", lse, torch.float32, (B, H, N), q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = attn_fwd_fp8_ex(q.data_ptr(), k.data_ptr(), vt.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
                         causal, scale, qs, ks, vs, tau, schedule, stream)
    if st != ATTN_OK:
        raise AttnError(st, last_error())
    return out, lse


def attn_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, delta, cu, B, H, Hkv, total, max_seqlen, d, causal, scale,
                    stream) -> int:
    """The C entry point with raw device addresses; returns the status code."""
    return lib().attn_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, delta, cu, B, H, Hkv, total, max_seqlen, d,
                                 int(causal), scale, stream)


def attn_bwd_varlen_check(q, k, v, o, lse, dout, dq, dk, dv, delta, cu, B, H, Hkv, total, max_seqlen, d, causal,
                          scale) -> int:
    return lib().attn_bwd_varlen_check(q, k, v, o, lse, dout, dq, dk, dv, delta, cu, B, H, Hkv, total, max_seqlen,
                                       d, int(causal), scale)


def attention_backward_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                              dout: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int | None = None,
                              causal: bool = False, scale: float | None = None):
    """Backward of packed variable-length attention on the current stream: returns (dQ, dK, dV, delta).

    q, o, dout: bfloat16 [H,total,d]; k, v: bfloat16 [Hkv,total,d]; lse: float32 [H,total]
    (o and lse from attention_varlen with the same cu_seqlens, causal flag and scale);
    cu_seqlens: int32 [B+1] on the same device.
    """
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() \
                or t.dim() != 3:
            raise TypeError(f"{name} must be a contiguous bfloat16 3-d CUDA tensor")
        if t.device != q.device:
            raise ValueError(f"{name} must be on {q.device}, got {t.device}")
    H, T, d = q.shape
    Hkv = k.shape[0]
    if tuple(k.shape) != (Hkv, T, d) or tuple(v.shape) != (Hkv, T, d):
        raise ValueError(f"k and v must be [Hkv,{T},{d}]")
    if tuple(o.shape) != (H, T, d) or tuple(dout.shape) != (H, T, d):
        raise ValueError(f"o and dout must be [{H},{T},{d}]")
    if (not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32 or tuple(lse.shape) != (H, T)
            or not lse.is_contiguous() or lse.device != q.device):
        raise TypeError("lse must be a contiguous float32 [H,total] tensor on q's device")
    if (not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1
            or cu_seqlens.device != q.device or not cu_seqlens.is_contiguous()):
        raise TypeError("cu_seqlens must be a contiguous int32 [B+1] tensor on q's device")
    B = cu_seqlens.numel() - 1
    if B < 0:
        raise ValueError("cu_seqlens needs at least one entry")
    if max_seqlen is None:
        max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if B > 0 else 0
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32).item())
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((H, T), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = attn_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                         dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), cu_seqlens.data_ptr(), B, H,
                         Hkv, T, max_seqlen, d, causal, scale, stream)
    if st != ATTN_OK:
        raise AttnError(st, last_error())
    return dq, dk, dv, delta
