"""The host code of the library (C ABI checks, identities, SHA-256; kernel
launchers stubbed) and the oracle, built with AddressSanitizer and
UndefinedBehaviorSanitizer, run the boundary, identity and oracle tests in a
child process.  Any sanitizer report fails the run (UBSan is built not to
recover, ASan aborts on its first error)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "parallelism_invariant_numerics_amd"))

TESTS = ["test_boundary.py", "test_identity.py", "test_oracle_gemm.py", "test_oracle_lmhead.py",
         "test_oracle_moe.py", "test_oracle_norm.py", "test_oracle_cpr.py"]


def _have(tool):
    return shutil.which(tool) is not None


@pytest.mark.skipif(not (_have("g++") and _have("gcc") and os.path.exists("/opt/rocm/include")),
                    reason="needs gcc, g++ and the ROCm headers")
def test_host_and_oracle_under_asan_ubsan(tmp_path):
    import build as libbuild  # parallelism_invariant_numerics_amd/build.py

    import oracle
    # a copy of the tree's Python parts with the sanitized libraries in place
    pkg = tmp_path / "parallelism_invariant_numerics_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "parallelism_invariant_numerics_amd", "__init__.py"), pkg)
    libbuild.build_host_sanitized(str(pkg / "libiso.so"))
    orc = tmp_path / "oracle"
    orc.mkdir()
    for f in ("__init__.py", "iso_oracle.c"):
        shutil.copy(os.path.join(ROOT, "oracle", f), orc)
    oracle.build_sanitized(str(orc / "liboracle.so"))
    shutil.copytree(os.path.join(ROOT, "iso_synth"), tmp_path / "iso_synth")
    shutil.copytree(os.path.join(ROOT, "include"), tmp_path / "include")
    tdir = tmp_path / "tests"
    shutil.copytree(os.path.join(ROOT, "tests"), tdir,
                    ignore=shutil.ignore_patterns("__pycache__", "test_gpu_*", "test_zz_*",
                                                  "test_sanitizers.py"))
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:detect_odr_violation=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["OMP_NUM_THREADS"] = "4"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "-k", "not bench_refuses", *[f"tests/{t}" for t in TESTS]],
                       cwd=tmp_path, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    # the child ran the sanitized builds of the copied tree
    probe = subprocess.run(
        [sys.executable, "-c", "import parallelism_invariant_numerics_amd as iso, oracle; "
         "oracle._load(); print(iso.LIB_PATH); print(oracle._LIB)"],
        cwd=tmp_path, env=env, capture_output=True, text=True, timeout=300)
    paths = probe.stdout.split()
    assert paths == [str(pkg / "libiso.so"), str(orc / "liboracle.so")], probe.stdout + probe.stderr
    for lib in paths:
        syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True,
                              text=True, check=True).stdout
        assert "__asan_" in syms and "__ubsan_" in syms, lib
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
