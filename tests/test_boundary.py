"""Host-side checks of the C ABI that need no GPU: the library loads and exports
every declared entry point, the contract identity is SHA-256 of the documented
canonical bytes, and every argument / shape / claim / workspace error is
returned before any launch (fake device addresses are never dereferenced)."""
import ctypes
import hashlib
import os
import re
import struct

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

iso = pytest.importorskip("parallelism_invariant_numerics_amd")

FAKE = 0x10000  # an aligned address the host checks accept; never dereferenced


def _declared():
    names = []
    inc = os.path.join(ROOT, "include")
    for f in sorted(os.listdir(inc)):
        if f.endswith(".h"):
            text = open(os.path.join(inc, f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"\b(iso_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert "iso_gemm" in names and "iso_lmhead_logprob" in names
    for n in names:
        assert hasattr(iso.lib, n), n


def test_version():
    assert "gfx950" in iso.version()


def _canonical(c):
    return struct.pack("<24s8I", b"iso.numerical_policy.v1\0", c.abi_version, c.in_dtype,
                       c.accum_dtype, c.leaf_count, c.leaf_size, c.tree, c.vocab_chunk,
                       c.schedule)


@pytest.mark.parametrize("L,m,chunk", [(4, 64, 0), (8, 256, 0), (8, 256, 128), (16, 256, 0),
                                       (4, 512, 0), (4, 128, 0), (1, 64, 0), (64, 65536, 0)])
def test_digest_is_sha256_of_canonical_bytes(L, m, chunk):
    c = iso.contract(L, m, chunk)
    assert len(_canonical(c)) == 56
    assert iso.digest(c) == hashlib.sha256(_canonical(c)).digest()


def test_digest_changes_with_every_field():
    base = iso.contract(8, 256, 0)
    d0 = iso.digest(base)
    for L, m, chunk in [(16, 256, 0), (8, 512, 0), (8, 256, 128), (4, 256, 0)]:
        assert iso.digest(iso.contract(L, m, chunk)) != d0
    iso.check_identity(base, d0)
    with pytest.raises(iso.IsoError) as e:
        iso.check_identity(base, iso.digest(iso.contract(4, 512, 0)))
    assert e.value.name == "ISO_ERR_IDENTITY"


def _raw(**kw):
    c = iso.Contract()
    iso.lib.iso_contract_init(ctypes.byref(c), 8, 256, 0)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value,code", [
    ("abi_version", 2, 8), ("in_dtype", 2, 3), ("accum_dtype", 1, 3), ("leaf_count", 3, 8),
    ("leaf_count", 128, 8), ("leaf_count", 0, 8), ("leaf_size", 96, 8), ("leaf_size", 0, 8),
    ("tree", 2, 8), ("schedule", 0, 8), ("vocab_chunk", 64, 8)])
def test_malformed_contract(field, value, code):
    c = _raw(**{field: value})
    assert iso.lib.iso_contract_validate(ctypes.byref(c)) == code
    out = ctypes.create_string_buffer(32)
    assert iso.lib.iso_contract_digest(ctypes.byref(c), out) == code


def _gemm(c, M=64, N=64, K=2048, P=1, A=FAKE, W=FAKE, C=FAKE, od=iso.F32, ws=None, wsb=0):
    return iso.lib.iso_gemm(ctypes.byref(c), A, W, C, od, M, N, K, P, ws, wsb, None)


def test_gemm_rejections_before_launch():
    c = iso.contract(8, 256, 0)
    assert _gemm(c, K=2047) == 2                      # K != L * m
    assert _gemm(c, M=-1) == 1
    assert _gemm(c, od=7) == 3
    for P in (3, 16, 0, -1):
        assert _gemm(c, P=P) == 4                      # outside the claim
    assert _gemm(iso.contract(4, 512, 0), P=8) == 4    # P must divide L
    assert _gemm(c, A=None) == 1
    assert _gemm(c, W=FAKE + 2) == 1                   # 16-byte alignment
    assert _gemm(c, P=2) == 6                          # workspace missing
    need = iso.gemm_workspace(c, 64, 64, 2)
    assert need == 2 * 64 * 64 * 4
    assert _gemm(c, P=2, ws=FAKE, wsb=need - 1) == 6
    assert _gemm(c, M=0) == 0 and _gemm(c, N=0) == 0   # empty: nothing launched
    assert _gemm(iso.contract(8, 256, 128)) == 8       # a logprob contract on a GEMM
    assert _gemm(c, K=1 << 23) == 2


def test_gemm_workspace_sizes():
    c16 = iso.contract(16, 256, 0)
    assert iso.gemm_workspace(c16, 10, 20, 1) == 0
    for P in (2, 4, 8):
        assert iso.gemm_workspace(c16, 10, 20, P) == P * 10 * 20 * 4
    # a partition deeper than the register tree is split further internally
    # (a few rows take the weight-streaming kernel, which holds the whole tree)
    assert iso.gemm_workspace(iso.contract(64, 64, 0), 10, 20, 1) == 0
    assert iso.gemm_workspace(iso.contract(64, 64, 0), 1000, 4096, 1) == 4 * 1000 * 4096 * 4
    assert iso.gemm_workspace(iso.contract(32, 64, 0), 1000, 4096, 1) == 2 * 1000 * 4096 * 4
    # one partition on too few 128 x 128 tiles to fill the chip: an optional
    # workspace lets the call split K into up to 8 subtrees (same bits)
    assert iso.gemm_workspace(c16, 64, 4096, 1) == 8 * 64 * 4096 * 4
    assert iso.gemm_workspace(c16, 128, 4096, 1) == 4 * 128 * 4096 * 4
    assert iso.gemm_workspace(iso.contract(8, 256, 0), 100, 2048, 1) == 4 * 100 * 2048 * 4
    assert iso.gemm_workspace(iso.contract(2, 1024, 0), 100, 2048, 1) == 2 * 100 * 2048 * 4
    assert iso.gemm_workspace(iso.contract(4, 512, 0), 300, 4096, 1) == 4 * 300 * 4096 * 4
    assert iso.gemm_workspace(c16, 4096, 4096, 1) == 0
    # the weight-streaming kernel takes up to 16 rows, and up to 32 on small layers
    assert iso.gemm_workspace(iso.contract(8, 256, 0), 32, 2048, 1) == 0
    assert iso.gemm_workspace(iso.contract(8, 256, 0), 64, 2048, 1) == 8 * 64 * 2048 * 4
    assert iso.gemm_workspace(c16, 16, 4096, 1) == 0
    assert iso.gemm_workspace(c16, 32, 4096, 1) == 8 * 32 * 4096 * 4
    with pytest.raises(iso.IsoError):
        iso.gemm_workspace(c16, 10, 20, 3)


def test_claims():
    c = iso.contract(4, 64, 0)
    for P in (1, 2, 4):
        iso.check_partitions(c, P)
    for P in (8, 3, 0):
        with pytest.raises(iso.IsoError) as e:
            iso.check_partitions(c, P)
        assert e.value.name == "ISO_ERR_CLAIM"


def test_baseline_rejections():
    f = iso.lib.iso_gemm_baseline
    assert f(FAKE, FAKE, FAKE, iso.F32, 4, 4, 100, None) == 2
    assert f(FAKE, FAKE, FAKE, 9, 4, 4, 128, None) == 3
    assert f(None, FAKE, FAKE, iso.F32, 4, 4, 128, None) == 1
    assert f(FAKE, FAKE, FAKE, iso.F32, 0, 4, 128, None) == 0


def _lm(c, M=8, V=512, K=256, P=1, ws=FAKE, wsb=1 << 40, H=FAKE, tok=FAKE):
    return iso.lib.iso_lmhead_logprob(ctypes.byref(c), H, FAKE, tok, FAKE, M, V, K, P, ws, wsb,
                                      None)


def test_lmhead_rejections_before_launch():
    c = iso.contract(4, 64, 128)
    assert _lm(iso.contract(4, 64, 0)) == 8           # not a logprob contract
    assert _lm(c, K=512) == 2
    assert _lm(c, V=0) == 2
    assert _lm(c, V=(1 << 20) + 1) == 2
    assert _lm(c, P=8) == 4
    assert _lm(c, H=None) == 1
    assert _lm(c, tok=None) == 1
    need = iso.lmhead_workspace(c, 8, 512, 1)
    assert need > 0
    assert _lm(c, ws=None) == 6
    assert _lm(c, wsb=need - 1) == 6
    assert _lm(c, M=0) == 0
    assert iso.lmhead_workspace(c, 8, 512, 2) >= need + 2 * 8 * 512 * 4


def _moe(T=16, H=256, E=8, I=128, k=4, gu=(4, 64), dn=(2, 64), X=FAKE, ws=FAKE, wsb=1 << 40):
    cg = iso.contract(*gu, 0)
    cd = iso.contract(*dn, 0)
    return iso.lib.iso_moe_combine(ctypes.byref(cg), ctypes.byref(cd), X, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, T, H, E, I, k, ws, wsb, None)


def test_moe_rejections_before_launch():
    assert _moe(E=0) == 1
    assert _moe(E=1025, k=4) == 2
    assert _moe(k=17, E=32) == 2
    assert _moe(k=9, E=8) == 2
    assert _moe(k=0) == 1
    assert _moe(gu=(8, 64)) == 2          # H != L * m
    assert _moe(dn=(4, 64)) == 2          # I != L * m
    assert _moe(H=2048, gu=(32, 64)) == 2  # too many leaves for the expert kernels
    assert _moe(T=0) == 0
    assert _moe(X=None) == 1
    need = iso.moe_workspace(16, 256, 8, 128, 4)
    assert _moe(wsb=need - 1) == 6
    assert _moe(ws=FAKE + 16) == 6        # workspace must be 256-byte aligned
    lay = iso.moe_layout(16, 256, 8, 128, 4)
    assert lay.idx < lay.gate < lay.h < lay.e < lay.total == need
    assert lay.e - lay.h >= 16 * 4 * 128 * 2 and lay.total - lay.e >= 16 * 4 * 256 * 4


def _norm(c, M=4, H=2048, x=FAKE, r=None, ro=None, w=FAKE + 0x100000, y=FAKE + 0x200000,
          od=iso.BF16, eps=1e-6):
    return iso.lib.iso_rmsnorm(ctypes.byref(c), x, r, ro, w, y, od, M, H, eps, None)


def test_rmsnorm_rejections_before_launch():
    c = iso.contract(64, 32, 0, iso.SCHED_SEQ)
    assert _norm(iso.contract(8, 256, 0)) == 8          # a matrix-product contract
    assert _norm(c, H=1024) == 2                        # H != L * m
    assert _norm(c, M=-1) == 1
    assert _norm(c, od=7) == 3
    assert _norm(c, eps=-1.0) == 1 and _norm(c, eps=float("nan")) == 1
    assert _norm(c, x=None) == 1 and _norm(c, w=None) == 1
    assert _norm(c, x=FAKE + 2) == 1                    # 16-byte alignment
    assert _norm(c, y=FAKE) == 1                        # y aliases x
    assert _norm(c, r=FAKE + 0x300000, ro=FAKE) == 1    # residual_out aliases x
    assert _norm(c, M=0) == 0                           # empty: nothing launched
    wide = iso.contract(64, 256, 0, iso.SCHED_SEQ)      # 256 elements per lane
    assert _norm(wide, H=16384) == 2
    many = iso.contract(4096, 1, 0, iso.SCHED_SEQ)      # 64 leaves per lane
    assert _norm(many, H=4096) == 2
    few = iso.contract(8, 4, 0, iso.SCHED_SEQ)          # 4 elements per lane
    assert _norm(few, H=32) == 2


def test_sequential_schedule_contracts():
    c = iso.contract(64, 32, 0, iso.SCHED_SEQ)
    assert iso.digest(c) == hashlib.sha256(_canonical(c)).digest()
    assert iso.digest(c) != iso.digest(iso.contract(64, 32 * 64, 0))
    for L, m, chunk in [(3, 32, 0), (8192, 1, 0), (64, 0, 0), (64, 32, 128)]:
        bad = _raw(leaf_count=L, leaf_size=m, vocab_chunk=chunk, schedule=iso.SCHED_SEQ)
        assert iso.lib.iso_contract_validate(ctypes.byref(bad)) == 8
    # the matrix products refuse a sequential-schedule contract
    assert _gemm(iso.contract(8, 256, 0, iso.SCHED_SEQ)) == 8


def _shard(c, M=4, V=1000, vb=0, ve=512, K=1024, H=FAKE, W=FAKE, tok=FAKE, st=FAKE, tg=FAKE):
    return iso.lib.iso_lmhead_shard_stats(ctypes.byref(c), H, W, tok, st, tg, M, V, vb, ve, K,
                                          None)


def test_lmhead_shard_rejections_before_launch():
    c = iso.contract(8, 128, 128)
    assert _shard(c, vb=100) == 2                  # shard start inside a chunk
    assert _shard(c, ve=600) == 2                  # shard end inside a chunk, not at V
    assert _shard(c, ve=1001) == 2                 # past the vocabulary
    assert _shard(c, vb=512, ve=512) == 2          # empty shard
    assert _shard(c, K=512) == 2                   # K != L * m
    assert _shard(iso.contract(8, 128, 0)) == 8    # not a logprob contract
    assert _shard(iso.contract(32, 64, 128), K=2048) == 4  # deeper than one register tree
    assert _shard(c, tok=None) == 1 and _shard(c, W=FAKE + 2) == 1
    assert _shard(c, vb=512, ve=1000, M=0) == 0    # empty: nothing launched
    fin = iso.lib.iso_lmhead_finish
    assert fin(FAKE, FAKE, FAKE, FAKE, -1, 100, None) == 1
    assert fin(FAKE, FAKE, FAKE, FAKE, 4, 0, None) == 1
    assert fin(FAKE, FAKE, FAKE, FAKE, 4, (1 << 20) + 1, None) == 2
    assert fin(None, FAKE, FAKE, FAKE, 4, 100, None) == 1
    assert fin(FAKE, FAKE, FAKE, FAKE, 0, 100, None) == 0


F2, F3, F4, F5, F6 = (FAKE * i for i in (2, 3, 4, 5, 6))  # distinct aligned fake addresses


def _cpr(c, T=64, H=2, q=FAKE, k=FAKE, v=FAKE, al=FAKE, be=FAKE, S0=None, o=F2, snap=F3, run=F4,
         ws=F5, wsb=1 << 40):
    return iso.lib.iso_cpr_prefill(ctypes.byref(c), q, k, v, al, be, S0, o, snap, run, T, H, ws,
                                   wsb, None)


def _cpr_dec(c, pos=20, H=2, o=F2, snap=F3, run=F4, ws=F5, wsb=1 << 40, q=FAKE):
    return iso.lib.iso_cpr_decode_step(ctypes.byref(c), q, FAKE, FAKE, FAKE, FAKE, pos, snap, run,
                                       o, H, ws, wsb, None)


def test_cpr_workspace_is_three_state_regions():
    """P_c and U_c for every closed chunk and the boundary states B_0..B_nb,
    each H * d * d FP32 (a multiple of 256 bytes, so no padding)."""
    c = iso.cpr_contract(16)
    state = 2 * 128 * 128 * 4
    for T in (0, 15, 16, 64, 70):
        nb = T // 16
        assert iso.cpr_workspace(c, 2, T) == (3 * nb + 1) * state
    with pytest.raises(iso.IsoError):
        iso.cpr_workspace(c, 0, 16)
    with pytest.raises(iso.IsoError):
        iso.cpr_workspace(iso.cpr_contract(16, head_size=64), 1, 16)


def test_cpr_contract_rules():
    with pytest.raises(iso.IsoError, match="ISO_ERR_CONTRACT"):
        iso.cpr_contract(0)
    with pytest.raises(iso.IsoError, match="ISO_ERR_CONTRACT"):
        iso.cpr_contract(65)                     # chunk at most 64 tokens
    with pytest.raises(iso.IsoError, match="ISO_ERR_CONTRACT"):
        iso.contract(128, 16, 128, iso.SCHED_CPR)  # no vocabulary chunk
    digests = {iso.digest(iso.cpr_contract(C)) for C in (1, 7, 64)}
    assert len(digests) == 3


def test_cpr_prefill_rejections_before_launch():
    c = iso.cpr_contract(16)
    assert _cpr(iso.contract(8, 256, 0)) == 8                 # not the CPR schedule
    assert _cpr(iso.cpr_contract(16, head_size=64)) == 2      # head size 128 only
    assert _cpr(c, H=0) == 1
    assert _cpr(c, H=65536) == 1
    assert _cpr(c, T=-1) == 1
    assert _cpr(c, T=16 * 65536) == 2                         # 65536 chunks
    assert _cpr(c, snap=None) == 1
    assert _cpr(c, run=F3) == 1                               # snap and run alias
    assert _cpr(c, snap=F3 + 4) == 1                          # 16-byte alignment
    assert _cpr(c, S0=F6 + 8) == 1
    assert _cpr(c, q=None) == 1
    assert _cpr(c, k=FAKE + 2) == 1
    assert _cpr(c, o=FAKE) == 1                               # o aliases an input
    assert _cpr(c, o=F3) == 1                                 # o aliases snap
    assert _cpr(c, S0=F6, o=F6) == 1                          # o aliases S0
    need = iso.cpr_workspace(c, 2, 64)
    assert _cpr(c, ws=None) == 6
    assert _cpr(c, wsb=need - 1) == 6
    assert _cpr(c, ws=F5 + 8) == 6


def test_cpr_decode_rejections_before_launch():
    c = iso.cpr_contract(16)
    assert _cpr_dec(iso.contract(8, 256, 0)) == 8
    assert _cpr_dec(c, H=0) == 1
    assert _cpr_dec(c, pos=-1) == 1
    assert _cpr_dec(c, pos=1 << 40) == 1
    assert _cpr_dec(c, run=F3) == 1
    assert _cpr_dec(c, o=F4) == 1
    assert _cpr_dec(c, o=FAKE) == 1
    assert _cpr_dec(c, q=None) == 1
    assert _cpr_dec(c, snap=F3 + 4) == 1
    need = iso.cpr_workspace(c, 2, 16)
    assert _cpr_dec(c, wsb=need - 1) == 6
    assert _cpr_dec(c, ws=None) == 6


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus 2 exits with status 2 and says so, before any GPU work."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr


def test_swiglu_rejections_before_launch():
    f = iso.lib.iso_swiglu
    assert f(FAKE, FAKE, None, FAKE, 0, None) == 0       # empty: nothing launched
    assert f(FAKE, FAKE, None, FAKE, -1, None) == 1      # negative size
    assert f(None, FAKE, None, FAKE, 8, None) == 1
    assert f(FAKE, None, FAKE, FAKE, 8, None) == 1
    assert f(FAKE, FAKE, FAKE, None, 8, None) == 1


def test_lmhead_noalloc_rejections_before_launch():
    f = iso.lib.iso_lmhead_logprob_noalloc
    c = iso.contract(8, 256, 128)
    cr = ctypes.byref(c)
    # the statistics of 3533 rows of a 151936-id vocabulary exceed the scratch
    assert f(cr, FAKE, FAKE, FAKE, FAKE, 3533, 151936, 2048, None) == 6
    assert f(cr, FAKE, FAKE, FAKE, FAKE, 10, 151936, 1024, None) == 2   # K != L * m
    assert f(cr, None, FAKE, FAKE, FAKE, 10, 151936, 2048, None) == 1
    assert f(cr, FAKE + 2, FAKE, FAKE, FAKE, 10, 151936, 2048, None) == 1  # unaligned
    assert f(cr, FAKE, FAKE, FAKE, FAKE, 0, 151936, 2048, None) == 0    # empty
    assert f(ctypes.byref(iso.contract(8, 256, 0)), FAKE, FAKE, FAKE, FAKE, 10, 1000, 2048,
             None) == 8                                                   # no vocab chunk
    assert iso.LMHEAD_NOALLOC_BYTES == 32 << 20
