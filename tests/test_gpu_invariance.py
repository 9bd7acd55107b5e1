"""The invariance sweep: W [4096 x 4096] (16 leaves of 256); 64 seeded probe
rows evaluated alone (batch 1), inside batches of 8, 64 and 4096 seeded filler
rows at seeded positions (including tile edges 0, 127, 128, 4095), at extra
batch sizes with ragged tiles, and with the leaves spread over 1, 2, 4 and 8
partitions.  Every probe output must have the same bits in every variant;
the reference variant is batch 1 with one partition."""
import numpy as np
import pytest

import oracle
from gpu_util import absdot, check_gemm_tol, dev, host, note, torch, u32
from iso_synth import make_config

pytestmark = pytest.mark.gpu

iso = pytest.importorskip("parallelism_invariant_numerics_amd")


@pytest.fixture(scope="module")
def sweep():
    cfg = make_config("sweep")
    c = iso.contract(cfg["leaves"], cfg["K"] // cfg["leaves"], 0)
    return cfg, c, dev(cfg["Wt"])


def _gemm(c, dW, rows_bits, P):
    out = iso.gemm(dev(rows_bits), dW, c, partitions=P)
    torch().cuda.synchronize()
    return u32(host(out))


def _layouts(cfg):
    """(batch, list of (probe ids, positions)) for every embedding variant."""
    rng = np.random.default_rng(cfg["placement_seed"])
    n = cfg["probes"]
    out = []
    for b in range(8):  # batch 8: eight probes each, at seeded slots
        out.append((8, np.arange(8 * b, 8 * b + 8), rng.permutation(8)))
    out.append((64, np.arange(n), np.arange(n)))
    out.append((64, np.arange(n), np.arange(n)[::-1].copy()))
    for _ in range(2):
        out.append((64, np.arange(n), rng.permutation(64)))
    for _ in range(2):
        pos = np.concatenate([[0, 127, 128, 4095], rng.choice(np.arange(1, 4095), n - 4, replace=False)])
        pos = np.unique(pos)
        while pos.size < n:
            pos = np.unique(np.concatenate([pos, rng.integers(1, 4095, n - pos.size)]))
        out.append((4096, np.arange(n), rng.permutation(pos)))
    for b in (65, 129, 1000):
        out.append((b, np.arange(n), rng.choice(b, n, replace=False)))
    return out


def test_invariance_sweep(sweep):
    cfg, c, dW = sweep
    probes, filler = cfg["probe_rows"], cfg["filler"]
    note("sweep reference: batch 1, P=1")
    ref = np.stack([_gemm(c, dW, probes[i:i + 1], 1)[0] for i in range(cfg["probes"])])
    # the reference itself against the oracle, on sampled columns
    rng = np.random.default_rng(11)
    rows = np.repeat(np.arange(cfg["probes"]), 16)
    cols = rng.integers(0, cfg["N"], rows.size)
    want = oracle.gemm_elems(probes, cfg["Wt"], cfg["leaves"], rows, cols)
    check_gemm_tol(ref.view(np.float32)[rows, cols], want, absdot(probes, cfg["Wt"], rows, cols),
                   "sweep reference")
    checked = 0
    for P in (1, 2, 4, 8):
        if P > 1:
            note(f"batch 1, P={P}")
            for i in range(0, cfg["probes"], 16):
                assert np.array_equal(_gemm(c, dW, probes[i:i + 1], P)[0], ref[i]), (i, P)
                checked += 1
        for batch, ids, pos in _layouts(cfg):
            note(f"batch {batch}, P={P}")
            X = filler[:batch].copy()
            X[pos] = probes[ids]
            C = _gemm(c, dW, X, P)
            for i, p in zip(ids, pos):
                assert np.array_equal(C[p], ref[i]), (batch, P, int(i), int(p))
                checked += 1
    assert checked > 1000
