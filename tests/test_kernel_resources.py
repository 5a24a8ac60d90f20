"""Occupancy of the hot kernels as the compiler reports it for the build's own
flags (CPU only: hipcc cross-compiles for gfx950, nothing is launched).

The single-launch stack runs two workgroups of four wavefronts per CU (two
wavefronts per SIMD) and the batched output kernel one workgroup of eight;
both sit close to the 256 registers that allow it (as does the
instrumented build of the stack, whose timelines are only representative at
the product's grid).  A change that pushes a
kernel past them does not fail any numerical test, it halves the kernel's
resident wavefronts (the stack's grid follows the occupancy query), so it
is checked here."""
import os
import re
import subprocess

import pytest

from rank_gated_memory_amd import build

CSRC = os.path.join(build.PKG, "csrc")


def resource_usage(source, flags=build.FLAGS):
    """{kernel name: {field: value}} from clang's resource-usage remarks."""
    cmd = ["/opt/rocm/bin/hipcc", *[f for f in flags if f not in ("-shared", "-fPIC")],
           "--cuda-device-only", "-c", os.path.join(CSRC, source), "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (-?\d+)", line)
        if m and name:
            kernels[name][m.group(1).strip()] = int(m.group(2))
    return kernels


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not installed")
@pytest.mark.parametrize("source,pattern,waves,flags", [
    ("gsi_kernels.hip", r"stack_kernel", 2, build.FLAGS),
    # the instrumented build must run the same grid for its timeline to hold
    ("gsi_kernels.hip", r"stack_kernel", 2, build.TRACE_FLAGS),
    ("gsi_batched.hip", r"bout_kernel", 2, build.FLAGS),
], ids=["stack", "stack-traced", "bout"])
def test_hot_kernels_keep_their_occupancy(source, pattern, waves, flags):
    usage = resource_usage(source, flags)
    hits = {k: v for k, v in usage.items() if re.search(pattern, k)}
    assert hits, f"no {pattern} in the remarks of {source}"
    for k, v in hits.items():
        assert v.get("Occupancy", 0) >= waves, f"{k}: {v}"
        assert v.get("VGPRs Spill", 0) == 0, f"{k} spills registers: {v}"
