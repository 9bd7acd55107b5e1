"""The identity part of the C ABI ([AGL] "Contract Structure and Enforcement":
regions, cases, composition, claims, SHA-256 identities named semantic,
numerical_policy and deployment; [KTB] section 6: checksums checked like a
lockfile).  Host only: incremental SHA-256 equals hashlib for any split, the
table identities equal SHA-256 of the documented bytes whatever the table's
order, each identity moves only with its own fields, and the per-call check
rejects a foreign policy or an unclaimed partition count."""
import ctypes
import hashlib
import random
import struct

import numpy as np
import pytest

iso = pytest.importorskip("parallelism_invariant_numerics_amd")


def _sha(parts):
    st = iso.Sha256State()
    assert iso.lib.iso_sha256_init(ctypes.byref(st)) == 0
    for p in parts:
        assert iso.lib.iso_sha256_update(ctypes.byref(st), p, len(p)) == 0
    out = ctypes.create_string_buffer(32)
    assert iso.lib.iso_sha256_final(ctypes.byref(st), out) == 0
    return out.raw


@pytest.mark.parametrize("n", [0, 1, 55, 56, 63, 64, 65, 119, 120, 127, 128, 1000, 4097])
def test_incremental_sha256_equals_hashlib(n):
    rng = random.Random(n)
    data = bytes(rng.randrange(256) for _ in range(n))
    for _ in range(5):
        cuts = sorted(rng.randrange(n + 1) for _ in range(rng.randrange(4)))
        parts = [data[a:b] for a, b in zip([0] + cuts, cuts + [n])]
        assert _sha(parts) == hashlib.sha256(data).digest()


def test_semantic_digest_of_weights_and_config():
    torch = pytest.importorskip("torch")
    w = np.arange(300, dtype=np.uint16).reshape(10, 30)
    t = torch.arange(7, dtype=torch.float32)
    cfg = '{"hidden": 2048, "vocab": 151936}'
    want = hashlib.sha256(w.tobytes() + t.numpy().tobytes() + cfg.encode()).digest()
    assert iso.semantic_digest([w, t, cfg]) == want
    assert iso.semantic_digest([w, t, cfg + " "]) != want


def _fields(c):
    return [c.abi_version, c.in_dtype, c.accum_dtype, c.leaf_count, c.leaf_size, c.tree,
            c.vocab_chunk, c.schedule]


def _documented(comps):
    """SHA-256 of the bytes the header documents, recomputed here."""
    items = sorted(comps.items())
    pol = b"iso.numerical_policy.table.v1\0" + struct.pack("<I", len(items))
    dep = (b"iso.deployment.v1\0" + iso.version().encode().ljust(32, b"\0") +
           struct.pack("<I", len(items)))
    for (region, case), (c, p, claims) in items:
        mask = sum(1 << (q.bit_length() - 1) for q in set(claims))
        names = region.encode().ljust(32, b"\0") + case.encode().ljust(32, b"\0")
        pol += names + struct.pack("<9I", *_fields(c), mask)
        dep += names + struct.pack("<I", p)
    return hashlib.sha256(pol).digest(), hashlib.sha256(dep).digest()


def _comps():
    return {
        ("dense_mlp", "engine_prefill"): (iso.contract(8, 256, 0), 1, [1, 2, 4, 8]),
        ("dense_mlp", "trainer_fwd"): (iso.contract(8, 256, 0), 8, [1, 2, 4, 8]),
        ("lm_head", "engine_prefill"): (iso.contract(8, 256, 128), 1, [1, 2, 4, 8]),
        ("lm_head", "trainer_fwd"): (iso.contract(8, 256, 128), 2, [1, 2, 4, 8]),
        ("final_norm", "engine_prefill"): (iso.contract(64, 32, 0, iso.SCHED_SEQ), 1, [1]),
        ("moe_down", "trainer_fwd"): (iso.contract(4, 128, 0), 4, [1, 2, 4]),
    }


def test_table_identities_are_the_documented_digests():
    comps = _comps()
    ec = iso.ExecutionContract(comps)
    pol, dep = _documented(comps)
    assert ec.numerical_policy == pol and ec.deployment == dep


def test_table_order_does_not_matter():
    comps = _comps()
    keys = list(comps)
    random.Random(3).shuffle(keys)
    table = (iso.Composition * len(keys))()
    for i, (region, case) in enumerate(keys):
        c, p, claims = comps[(region, case)]
        table[i].region, table[i].case_name = region.encode(), case.encode()
        table[i].policy, table[i].partitions = c, p
        table[i].claims = sum(1 << (q.bit_length() - 1) for q in claims)
    pol = ctypes.create_string_buffer(32)
    dep = ctypes.create_string_buffer(32)
    assert iso.lib.iso_table_digests(table, len(keys), pol, dep) == 0
    ec = iso.ExecutionContract(comps)
    assert pol.raw == ec.numerical_policy and dep.raw == ec.deployment


def test_each_identity_moves_only_with_its_own_fields():
    base = iso.ExecutionContract(_comps())
    # a different reduction decomposition: numerical policy changes
    c = _comps()
    c[("lm_head", "trainer_fwd")] = (iso.contract(16, 128, 128), 2, [1, 2, 4, 8])
    e = iso.ExecutionContract(c)
    assert e.numerical_policy != base.numerical_policy and e.deployment == base.deployment
    # a different claim: numerical policy changes
    c = _comps()
    c[("moe_down", "trainer_fwd")] = (iso.contract(4, 128, 0), 4, [1, 4])
    e = iso.ExecutionContract(c)
    assert e.numerical_policy != base.numerical_policy and e.deployment == base.deployment
    # a different partition count within the claims: only the deployment changes
    c = _comps()
    c[("dense_mlp", "trainer_fwd")] = (iso.contract(8, 256, 0), 4, [1, 2, 4, 8])
    e = iso.ExecutionContract(c)
    assert e.numerical_policy == base.numerical_policy and e.deployment != base.deployment


def _status(fn):
    with pytest.raises(iso.IsoError) as e:
        fn()
    return e.value.name


def test_table_errors():
    c = _comps()
    c[("dense_mlp", "trainer_fwd")] = (iso.contract(8, 256, 0), 2, [1, 4])     # 2 not claimed
    assert _status(lambda: iso.ExecutionContract(c)) == "ISO_ERR_CLAIM"
    c = _comps()
    c[("moe_down", "trainer_fwd")] = (iso.contract(4, 128, 0), 4, [1, 2, 4, 8])  # 8 does not divide 4
    assert _status(lambda: iso.ExecutionContract(c)) == "ISO_ERR_CLAIM"
    c = _comps()
    c[("final_norm", "trainer_fwd")] = (iso.contract(64, 32, 0, iso.SCHED_SEQ), 2, [1, 2])
    assert _status(lambda: iso.ExecutionContract(c)) == "ISO_ERR_CLAIM"      # no split of a row norm
    for bad in ("", "x" * 32):
        c = {(bad, "trainer_fwd"): (iso.contract(8, 256, 0), 1, [1])}
        assert _status(lambda: iso.ExecutionContract(c)) == "ISO_ERR_ARG"
    table = (iso.Composition * 2)()
    for t in table:
        t.region, t.case_name, t.policy, t.partitions, t.claims = b"a", b"b", iso.contract(8, 256, 0), 1, 1
    pol = ctypes.create_string_buffer(32)
    assert iso.lib.iso_table_digests(table, 2, pol, pol) == 1                # repeated (region, case)
    table[1].policy.leaf_count = 3
    table[1].case_name = b"c"
    assert iso.lib.iso_table_digests(table, 2, pol, pol) == 8                # malformed policy


def test_per_call_check():
    ec = iso.ExecutionContract(_comps())
    ec.check("lm_head", "trainer_fwd", iso.contract(8, 256, 128), 8)
    ec.check("final_norm", "engine_prefill", iso.contract(64, 32, 0, iso.SCHED_SEQ), 1)
    assert _status(lambda: ec.check("lm_head", "trainer_fwd", iso.contract(4, 512, 128), 2)) \
        == "ISO_ERR_IDENTITY"
    assert _status(lambda: ec.check("moe_down", "trainer_fwd", iso.contract(4, 128, 0), 8)) \
        == "ISO_ERR_CLAIM"
    assert _status(lambda: ec.check("moe_down", "trainer_fwd", iso.contract(4, 128, 0), 3)) \
        == "ISO_ERR_CLAIM"
    assert _status(lambda: ec.check("attention", "trainer_fwd", iso.contract(8, 256, 0), 1)) \
        == "ISO_ERR_ARG"
