"""Host-code sanitizer build of the library, for the CPU tests.

The library's host code (argument validation, size and overlap arithmetic, option
parsing, error reporting) is compiled with AddressSanitizer and
UndefinedBehaviorSanitizer; the device code is compiled as usual (sanitizer flags
go to the host pass only, through -Xarch_host). The Python interpreter is not
instrumented, so the sanitizer runtime is preloaded into the process that loads
the library (see `env`).
"""
from __future__ import annotations

import glob
import os
import re

from exact_attention_22_amd import build as lib_build

# host pass only: each flag behind its own -Xarch_host
SANITIZE = ("-Xarch_host -g -Xarch_host -fno-omit-frame-pointer -Xarch_host -fsanitize=address "
            "-Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all").split()
LINK = "-Xarch_host -fsanitize=address,undefined -Xarch_host -shared-libsan".split()


def asan_runtime() -> str:
    """The shared AddressSanitizer runtime of the ROCm clang (it also carries the
    UndefinedBehaviorSanitizer handlers)."""
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return found[-1]


def build(out_dir: str, log: list | None = None) -> str:
    """Compile the sanitized library into out_dir; returns its path. With `log`, the
    compiler's per-kernel resource remarks of every unit are appended to it."""
    extra = SANITIZE + (["-Rpass-analysis=kernel-resource-usage"] if log is not None else [])
    return lib_build.build(os.path.join(out_dir, "libattn_fwd_san.so"), extra=extra, link_extra=LINK, log=log)


def kernel_resources(log) -> dict:
    """{mangled kernel name: {"ScratchSize": bytes per lane, "VGPRs": n, ...}} from the
    remarks that build(..., log) collected."""
    res = {}
    for _, text in log:
        cur = None
        for line in text.splitlines():
            m = re.search(r"remark: Function Name: (\S+)", line)
            if m:
                cur = res.setdefault(m.group(1), {})
                continue
            m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+) \[-Rpass", line)
            if m and cur is not None:
                cur[m.group(1).strip()] = int(m.group(2))
    return res


def env(lib_path: str) -> dict:
    """Environment of a process that loads the sanitized library through the binding:
    any sanitizer report ends it with a nonzero status."""
    e = dict(os.environ)
    e["LD_PRELOAD"] = asan_runtime()
    e["EXACT_ATTN_LIB"] = lib_path
    # the interpreter itself is not instrumented: its allocations at exit are not leaks of ours
    e["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86"
    e["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=87"
    return e
