"""Compile the HIP library for gfx950 in-tree (hipcc cross-compiles without a GPU).

    python -m exact_attention_22_amd.build

writes exact_attention_22_amd/libattn_fwd.so next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libattn_fwd.so")
ARCH = "gfx950"

# Packed fp32 vector instructions are disabled for every HIP translation unit.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-command-line-argument",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


# attn_fwd.hip holds the host code of the forward entry points; the forward kernel's
# variants are instantiated per head dim and mask in their own units so that they
# compile in parallel.
SOURCES = ("attn_fwd.hip", "attn_fwd_d128_full.hip", "attn_fwd_d128_causal.hip", "attn_fwd_d64_full.hip",
           "attn_fwd_d64_causal.hip", "attn_bwd.hip", "attn_fp8.hip")


def build(out: str = LIB, extra: list[str] | None = None, verbose: bool = False,
          link_extra: list[str] | None = None, log: list | None = None) -> str:
    """Always recompiles; returns the path of the shared library.

    Each translation unit is compiled to an object in parallel, then linked.
    `extra` is added to every compile line, `link_extra` to the link line; with
    `log`, each unit's compiler output is appended to it as (source, text)."""
    tmp = out + ".tmp"
    objs = [f"{out}.{os.path.splitext(src)[0]}.o" for src in SOURCES]
    base = [hipcc(), f"--offload-arch={ARCH}", *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    procs = []
    for src, obj in zip(SOURCES, objs):
        cmd = [*base, "-c", os.path.join(CSRC, src), "-o", obj, *(extra or [])]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    failed = False
    for src, p in zip(SOURCES, procs):
        text, _ = p.communicate()
        if log is not None:
            log.append((src, text))
        if p.returncode != 0:
            sys.stderr.write(text)
            failed = True
    if failed:
        raise RuntimeError("hipcc failed")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", *objs, "-o", tmp, *(link_extra or [])]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    for obj in objs:
        if os.path.exists(obj):
            os.remove(obj)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc link failed with exit code {res.returncode}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
