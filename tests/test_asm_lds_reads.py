"""The kernels' inline-assembly LDS reads against the compiler: in the gfx950
assembly of every device source, no instruction touches a register of an LDS
read written in inline assembly before the wait that retires the read (the
compiler treats such an output as written at once).  The scanner itself is
pinned first on small hand-written listings."""
import importlib.util
import os
import shutil
from concurrent.futures import ThreadPoolExecutor

import pytest

from asm_scan import scan_text

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _listing(*body):
    return "\n".join(["_Zkern:", *body, ".Lfunc_end0:"])


def test_scanner_flags_a_copy_before_the_wait():
    text = _listing(";;#ASMSTART", "ds_read_b32 v4, v2", ";;#ASMEND",
                    "v_accvgpr_write_b32 a1, v4", ";;#ASMSTART", "s_waitcnt lgkmcnt(0)", ";;#ASMEND")
    assert list(scan_text(text)) == ["_Zkern"]


def test_scanner_accepts_a_use_after_the_wait_and_counts_partial_waits():
    ok = _listing(";;#ASMSTART", "ds_read_b128 v[4:7], v2", "ds_read_b128 v[8:11], v2 offset:64",
                  "s_waitcnt lgkmcnt(1)", ";;#ASMEND", "v_mov_b32_e32 v20, v5",
                  ";;#ASMSTART", "s_waitcnt lgkmcnt(0)", ";;#ASMEND", "v_mov_b32_e32 v21, v9")
    assert scan_text(ok) == {}
    bad = _listing(";;#ASMSTART", "ds_read_b128 v[4:7], v2", "ds_read_b128 v[8:11], v2 offset:64",
                   "s_waitcnt lgkmcnt(1)", ";;#ASMEND", "v_mov_b32_e32 v20, v9")
    assert list(scan_text(bad)) == ["_Zkern"]


def test_scanner_follows_branches():
    # the read is still in flight on the taken path, retired on the other
    text = _listing(";;#ASMSTART", "ds_read_b32 v4, v2", ";;#ASMEND",
                    "s_cbranch_scc1 .LBB0_2", ";;#ASMSTART", "s_waitcnt lgkmcnt(0)", ";;#ASMEND",
                    "s_branch .LBB0_3", ".LBB0_2:", "v_add_u32_e32 v5, v4, v4", ".LBB0_3:", "s_endpgm")
    hits = scan_text(text)["_Zkern"]
    assert [h[2] for h in hits] == ["v_add_u32_e32 v5, v4, v4"]
    clean = text.replace("s_cbranch_scc1 .LBB0_2", "s_nop 0").replace("s_branch .LBB0_3", "s_endpgm")
    assert scan_text(clean) == {}


@pytest.mark.skipif(shutil.which("/opt/rocm/bin/hipcc") is None, reason="needs hipcc")
def test_kernels_never_touch_an_lds_read_in_flight(tmp_path):
    spec = importlib.util.spec_from_file_location(
        "_iso_build", os.path.join(ROOT, "parallelism_invariant_numerics_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    outs = [(s, str(tmp_path / (s + ".s"))) for s in b.DEVICE_SOURCES]
    with ThreadPoolExecutor(max_workers=6) as ex:
        for f in [ex.submit(b.device_asm, s, o) for s, o in outs]:
            f.result()
    report = {}
    for s, o in outs:
        for fn, hits in scan_text(open(o).read()).items():
            report[f"{s}: {fn}"] = hits[:3]
    assert report == {}, report
