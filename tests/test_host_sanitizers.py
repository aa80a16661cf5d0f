"""The C-ABI host checks under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds the library with the host code instrumented (tests/host_sanitizers.py) and
runs tests/test_abi.py against it in a child process: every validation path those
tests drive (sizes, overflow limits, alignment, overlap checks, options structs of
both ABI sizes, split-key shapes and workspace sizes, FP8 offsets, error strings)
then runs with out-of-bounds accesses, signed overflow, invalid enum loads and
other undefined behaviour turned into a failing exit status.
"""
import os
import re
import subprocess
import sys

import pytest

from tests import host_sanitizers

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


_LOG = []

# Kernels whose registers do not yet suffice (they spill to scratch memory): the
# d = 128 forward variants with half the exponentials on the polynomial (an option,
# not the default) and the d = 128 backward dQ kernel.
SCRATCH_ALLOWED = (re.compile(r"attn_fwd_kernelILi128ELi64ELb[01]ELb[01]ELi4E"),
                   re.compile(r"attn_bwd_dq_kernelILi128E"))


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    return host_sanitizers.build(str(tmp_path_factory.mktemp("san")), log=_LOG)


def test_kernels_keep_to_registers(sanitized_lib):
    # The same device code as the product build (sanitizers touch the host pass only):
    # every kernel fits its registers, so none keeps values in scratch memory, except
    # the listed variants. A lambda the compiler does not inline, for one, moves its
    # captured accumulators to scratch and slows the kernel several times over.
    res = host_sanitizers.kernel_resources(_LOG)
    kernels = {k: v for k, v in res.items() if "kernel" in k}
    assert len(kernels) > 100, len(kernels)
    bad = {k: v.get("ScratchSize") for k, v in kernels.items()
           if v.get("ScratchSize", -1) != 0 and not any(p.search(k) for p in SCRATCH_ALLOWED)}
    assert not bad, bad


def test_library_is_instrumented(sanitized_lib):
    undef = subprocess.run(["nm", "-D", "--undefined-only", sanitized_lib], capture_output=True, text=True,
                           check=True).stdout
    assert "__asan_report_load" in undef or "__asan_report_store" in undef
    assert "__ubsan_handle_" in undef


def test_abi_checks_pass_under_host_sanitizers(sanitized_lib):
    res = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "-q", "-p", "no:cacheprovider"],
                         cwd=ROOT, env=host_sanitizers.env(sanitized_lib), capture_output=True, text=True,
                         timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out and "failed" not in out, out[-2000:]
