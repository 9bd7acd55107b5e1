"""Audit of the compiled device code (hipcc, gfx950, no GPU needed).

The ring waits of the leaf/tree main loop are hand-written
`s_waitcnt vmcnt(n)` with n > 0: "at most n of this wave's memory operations
outstanding" proves the oldest ring stage landed only while every operation
in flight is a load (loads complete in order).  A register spill puts stores
in flight, and a store may complete before an older load.  So a kernel whose
code stores to scratch must not contain such a hand-written wait; those
kernels are built with the draining wait (vmcnt(0)) instead."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "parallelism_invariant_numerics_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not available")


def _asm(src, tmp_path):
    out = tmp_path / (src + ".s")
    subprocess.run([HIPCC, "-O3", "-std=c++20", "-I", os.path.join(ROOT, "include"),
                    "--offload-arch=gfx950", "-ffp-contract=off", "-fno-fast-math",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)],
                   check=True, capture_output=True)
    return out.read_text()


def _kernels(text):
    for part in re.split(r"\n(?=_Z[^\n]*:)", text):
        m = re.match(r"(_Z\S*):", part)
        if m:
            yield m.group(1), part


def _inline_asm(body):
    return "\n".join(re.findall(r";;#ASMSTART\n(.*?);;#ASMEND", body, flags=re.S))


@pytest.mark.parametrize("src", ["gemm.hip", "lmhead.hip", "moe.hip"])
def test_spilling_kernels_drain_their_ring_waits(src, tmp_path):
    text = _asm(src, tmp_path)
    checked = 0
    for name, body in _kernels(text):
        if "scratch_store" not in body:
            continue
        checked += 1
        waits = re.findall(r"s_waitcnt vmcnt\(([0-9]+)\)", _inline_asm(body))
        bad = [w for w in waits if int(w) > 0]
        assert not bad, f"{name}: spills and waits vmcnt({bad[0]}) in its ring"
    # the invariant GEMM itself must not spill at any depth
    if src == "gemm.hip":
        assert checked == 0, "a GEMM kernel spills"
