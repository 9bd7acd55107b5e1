"""GPU parity of the CPR gated delta rule with the oracle, bit for bit (every
step is a correctly rounded FP32 multiply or add in the definition's order,
every dot product the balanced tree over the 128 products): prefill outputs
and final states over chunk lengths, ragged and short sequences, zero and
given initial states; decode steps (with the re-sync at every chunk end)
continuing a prefill give the prefill's bits; a head's bits do not depend on
the other heads; the full 16-head, 4096-token layer against the oracle on
sampled heads; and the argument checks."""
import numpy as np
import pytest

import oracle
from gpu_util import dev, host, note, torch
from iso_synth import cpr_inputs, normal_f32

pytestmark = pytest.mark.gpu

iso = pytest.importorskip("parallelism_invariant_numerics_amd")

D = 128


def _dev_inputs(x):
    t = torch()
    return (dev(x["q"]), dev(x["k"]), dev(x["v"]), t.from_numpy(x["alpha"]).to("cuda"),
            t.from_numpy(x["beta"]).to("cuda"))


def _s0(H, seed):
    return (normal_f32(seed, (H, D, D)) * np.float32(0.05)).astype(np.float32)


def _same(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32),
                          np.asarray(b, np.float32).view(np.uint32))


@pytest.mark.parametrize("T,H,C,init", [(64, 2, 16, False), (100, 3, 32, True), (7, 1, 64, True),
                                        (128, 2, 64, True), (33, 2, 1, False), (96, 1, 48, True),
                                        (0, 2, 16, True)])
def test_prefill_matches_oracle_bitwise(T, H, C, init):
    t = torch()
    note(f"cpr prefill T={T} H={H} C={C} init={init}")
    x = cpr_inputs(max(T, 1), H, D, seed=701 + T)
    x = {k: v[:T] for k, v in x.items()}
    S0 = _s0(H, 711) if init else None
    c = iso.cpr_contract(C)
    o, snap, run = iso.cpr_prefill(*_dev_inputs(x), c,
                                   S0=None if S0 is None else t.from_numpy(S0).to("cuda"))
    t.cuda.synchronize()
    oe, snape, rune = oracle.cpr_prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], C, S0=S0)
    assert _same(host(o), oe)
    assert _same(host(snap), snape)
    assert _same(host(run), rune)


@pytest.mark.parametrize("T0", [0, 37, 64, 65])
def test_decode_continues_prefill_bitwise(T0):
    t = torch()
    T, H, C = 160, 2, 32
    note(f"cpr decode from T0={T0} to T={T}")
    x = cpr_inputs(T, H, D, seed=721)
    c = iso.cpr_contract(C)
    q, k, v, al, be = _dev_inputs(x)
    o_all, snap_all, run_all = iso.cpr_prefill(q, k, v, al, be, c)
    if T0 > 0:
        _, snap, run = iso.cpr_prefill(q[:T0], k[:T0], v[:T0], al[:T0], be[:T0], c)
    else:
        snap = t.zeros((H, D, D), dtype=t.float32, device="cuda")
        run = t.zeros((H, D, D), dtype=t.float32, device="cuda")
    outs = []
    for p in range(T0, T):
        outs.append(iso.cpr_decode_step(q, k, v, al, be, p, snap, run, c).clone())
    t.cuda.synchronize()
    o_all = host(o_all)
    for i, p in enumerate(range(T0, T)):
        assert _same(host(outs[i]), o_all[p]), f"token {p}"
    assert _same(host(snap), host(snap_all))
    assert _same(host(run), host(run_all))
    # and the decode path agrees with the oracle's decode
    oe, snape, rune = oracle.cpr_prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], C)
    assert _same(o_all, oe)


def test_heads_are_independent():
    t = torch()
    T, H, C = 96, 4, 32
    x = cpr_inputs(T, H, D, seed=731)
    c = iso.cpr_contract(C)
    o4, s4, r4 = iso.cpr_prefill(*_dev_inputs(x), c)
    one = {k: np.ascontiguousarray(v[:, 2:3]) for k, v in x.items()}
    o1, s1, r1 = iso.cpr_prefill(*_dev_inputs(one), c)
    t.cuda.synchronize()
    assert _same(host(o4)[:, 2:3], host(o1))
    assert _same(host(s4)[2:3], host(s1))
    assert _same(host(r4)[2:3], host(r1))


def test_full_layer_against_oracle_on_sampled_heads():
    """The benchmarked layer: 16 heads of 128, 4096 tokens, chunk 64.  The
    oracle recomputes heads 0 and 11 in full (a head's bits depend only on
    its own inputs)."""
    t = torch()
    T, H, C = 4096, 16, 64
    note("cpr full layer 16 x 4096")
    x = cpr_inputs(T, H, D, seed=601)
    c = iso.cpr_contract(C)
    o, snap, run = iso.cpr_prefill(*_dev_inputs(x), c)
    t.cuda.synchronize()
    o, snap, run = host(o), host(snap), host(run)
    heads = [0, 11]
    sub = {k: np.ascontiguousarray(v[:, heads]) for k, v in x.items()}
    oe, snape, rune = oracle.cpr_prefill(sub["q"], sub["k"], sub["v"], sub["alpha"], sub["beta"], C)
    assert _same(o[:, heads], oe)
    assert _same(snap[heads], snape)
    assert _same(run[heads], rune)
    assert np.isfinite(o).all()


def test_rejections():
    t = torch()
    x = cpr_inputs(8, 1, D, seed=741)
    q, k, v, al, be = _dev_inputs(x)
    c = iso.cpr_contract(4)
    with pytest.raises(iso.IsoError, match="ISO_ERR_CONTRACT"):
        iso.cpr_contract(65)
    ws = t.empty(iso.cpr_workspace(c, 1, 8), dtype=t.uint8, device="cuda")
    with pytest.raises(iso.IsoError, match="ISO_ERR_SHAPE"):
        iso.cpr_prefill(q, k, v, al, be, iso.cpr_contract(4, head_size=64), workspace=ws)
    with pytest.raises(iso.IsoError):  # the workspace query rejects it too
        iso.cpr_workspace(iso.cpr_contract(4, head_size=64), 1, 8)
    same = t.zeros((1, D, D), dtype=t.float32, device="cuda")
    with pytest.raises(iso.IsoError, match="ISO_ERR_ARG"):
        iso.cpr_prefill(q, k, v, al, be, c, snap=same, run=same)
    small = t.empty(16, dtype=t.uint8, device="cuda")
    with pytest.raises(iso.IsoError, match="ISO_ERR_WORKSPACE"):
        iso.cpr_prefill(q, k, v, al, be, c, workspace=small)
    with pytest.raises(iso.IsoError, match="ISO_ERR_CONTRACT"):
        iso.cpr_prefill(q, k, v, al, be, iso.contract(8, 16, 0, iso.SCHED_SEQ), workspace=ws)
    with pytest.raises(ValueError):
        iso.cpr_decode_step(q, k, v, al, be, 8, same, same.clone(), c)  # pos past the arrays
