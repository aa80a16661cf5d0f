"""Per-phase shader clocks of the bf16 forward kernel's ping-pong schedule.

    python -m exact_attention_22_amd.micro.phase_clocks build      # on any host with hipcc
    python -m exact_attention_22_amd.micro.phase_clocks run headline causal2k ...   # on the GPU
    python -m exact_attention_22_amd.micro.phase_clocks run --data random,k0,v0,q0 headline

`build` compiles the library with -DATTN_PHASE_CLOCKS into
_build/libattn_fwd_phase.so. In that build every wavefront of the forward kernel
sums the shader-clock cycles (s_memtime) of its softmax phases, of its waits at the
barriers that end them (none where the step ends without one), of its matrix
phases and of the waits after those, and
stores the sums in the rescale-count buffer instead of the counts. `run` loads that
library (the EXACT_ATTN_LIB variable, set for a child process), runs each named
workload three times and prints, for each group of wavefronts, the cycles per tile
of the four intervals, and the total cycles per wavefront. It then times 30 more
launches with events and prints the mean shader clock they ran at (a workgroup's
cycles over the launch time). With --data, each workload also runs on inputs
with one operand set to zero (k0, v0, q0) beside the seeded random inputs
(random): the instruction stream is the same, and the clock shows how the
matrix core's power draw, which depends on the operand values, sets it. The
instrumentation adds four clock reads per tile and eight one-lane stores per
wavefront at the end; the phases it times are otherwise the product kernel's.
"""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
LIB = os.path.join(ROOT, "_build", "libattn_fwd_phase.so")


def build() -> str:
    from exact_attention_22_amd import build as lib_build
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    return lib_build.build(LIB, extra=["-DATTN_PHASE_CLOCKS"])


DATA = ("random", "k0", "v0", "q0")


def measure(names, data=("random",)):
    import torch

    from exact_attention_22_amd import binding, inputs
    assert os.path.samefile(binding.LIB_PATH, LIB), binding.LIB_PATH
    dev = torch.device("cuda:0")
    for name in names:
        w = inputs.BY_NAME[name]
        if isinstance(w, inputs.VarlenWorkload):
            raise SystemExit(f"{name}: dense workloads only")
        q0, k0, v0 = (t.to(dev) for t in inputs.workload_inputs(w))
        for kind in data:
            q, k, v = (torch.zeros_like(t) if kind == z else t for t, z in ((q0, "q0"), (k0, "k0"), (v0, "v0")))
            label = name if kind == "random" else f"{name} ({kind})"
            report(label, w, q, k, v, torch, binding)


def report(name, w, q, k, v, torch, binding):
    for _ in range(3):
        o, lse, rec = binding.attention(q, k, v, causal=w.causal, scale=w.scale, rescale_count=True)
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = min(rec.numel() // 8, cus * 8)  # one record per wavefront of at most one workgroup per CU
    r = rec.flatten()[: n * 8].view(-1, 8).cpu().double()
    r = r[r[:, 4] > 0]
    slots = rec.flatten()[: n * 8].view(-1, 8, 8).cpu().double()  # [workgroup][wavefront][record]
    live = slots[:, :, 4].sum(1) > 0
    wg = slots[:, :, 5].max(1).values[live]  # a workgroup's cycles: its slowest wavefront
    ids = torch.arange(slots.shape[0])[live]
    xcd = [wg[ids % 8 == x].mean().item() for x in range(8)]
    print(f"{name} workgroups: {len(wg)}; cycles per workgroup min {wg.min():.0f}, median {wg.median():.0f}, "
          f"max {wg.max():.0f}, mean {wg.mean():.0f} (max / mean {wg.max() / wg.mean():.3f}); mean per XCD "
          f"{', '.join(f'{v:.0f}' for v in xcd)}", flush=True)
    for g in (0, 1):
        sel = r[r[:, 6] == g]
        t = sel[:, 4].sum()
        print(f"{name} group {'AB'[g]}: {len(sel)} wavefronts, {int(t)} tiles; cycles per tile: softmax "
              f"{sel[:, 0].sum() / t:.0f}, wait {sel[:, 1].sum() / t:.0f}, matrix {sel[:, 2].sum() / t:.0f}, "
              f"wait {sel[:, 3].sum() / t:.0f}; cycles per wavefront {sel[:, 5].mean():.0f} "
              f"({(sel[:, :4].sum(1)).mean():.0f} in tile steps)", flush=True)
    n_it = 30
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n_it):
        binding.attention(q, k, v, causal=w.causal, scale=w.scale, rescale_count=True)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n_it
    print(f"{name} launch {ms:.4f} ms; shader clock {wg.mean() / ms / 1e3:.0f} MHz (mean workgroup cycles "
          f"over the launch time)", flush=True)


def main(argv):
    if not argv or argv[0] not in ("build", "run"):
        raise SystemExit(__doc__)
    if argv[0] == "build":
        print(build())
        return 0
    args = argv[1:]
    data = ("random",)
    if args[:1] == ["--data"]:
        data = tuple(args[1].split(","))
        if not set(data) <= set(DATA):
            raise SystemExit(f"--data takes a comma-separated subset of {', '.join(DATA)}")
        args = args[2:]
    names = args or ["headline"]
    if os.environ.get("EXACT_ATTN_LIB") != LIB:
        env = dict(os.environ, EXACT_ATTN_LIB=LIB)
        return subprocess.run([sys.executable, "-m", "exact_attention_22_amd.micro.phase_clocks", "run", *argv[1:]],
                              cwd=ROOT, env=env).returncode
    measure(names, data)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
