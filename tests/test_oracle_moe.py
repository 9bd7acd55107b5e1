"""Pins of the oracle's MoE routing, SwiGLU FFN and fixed-order combine."""
import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
from pins import moe_combine_pins
from iso_synth import bf16_bits_to_f32, f32_to_bf16_bits, normal_bf16, normal_f32


def _small(T=16, Hd=128, E=8, I=64, seed=0):
    X = normal_bf16(seed + 1, (T, Hd), 1.0)
    lg = normal_f32(seed + 2, (T, E))
    Wg = normal_bf16(seed + 3, (E, I, Hd), 0.05)
    Wu = normal_bf16(seed + 4, (E, I, Hd), 0.05)
    Wd = normal_bf16(seed + 5, (E, Hd, I), 0.05)
    return X, lg, Wg, Wu, Wd


def test_routing_matches_lexsort_with_ties():
    T, E, k = 64, 32, 8
    lg = normal_f32(1, (T, E))
    lg[::3, 5] = lg[::3, 9]            # planted ties: id 5 must precede id 9
    lg[1::4, :] = np.round(lg[1::4, :])  # many ties per row
    idx, gate = oracle.moe_route(lg, k)
    for t in range(T):
        order = np.lexsort((np.arange(E), -lg[t]))  # primary: logit desc; then id asc
        assert np.array_equal(idx[t], order[:k])
    assert np.allclose(gate.sum(1), 1.0, rtol=0, atol=8 * 2.0 ** -53 * 8)


def test_gates_are_softmax_over_selected():
    # renormalising the full softmax over the selected experts equals a softmax
    # over the selected logits (the full denominator cancels)
    T, E, k = 32, 128, 8
    lg = normal_f32(2, (T, E))
    idx, gate = oracle.moe_route(lg, k)
    sel = np.take_along_axis(lg.astype(np.float64), idx.astype(np.int64), axis=1)
    assert np.allclose(gate, softmax(sel, axis=1), rtol=1e-14, atol=0)
    assert np.all(np.diff(sel, axis=1) <= 0)


def test_swiglu_stage_against_float64_formula():
    X, lg, Wg, Wu, Wd = _small()
    idx, _ = oracle.moe_route(lg, 4)
    act, h = oracle.moe_gate_up(X, Wg, Wu, idx, 2)
    x = bf16_bits_to_f32(X).astype(np.float64)
    for t in (0, 7, 15):
        for s in range(4):
            e = idx[t, s]
            g = x[t] @ bf16_bits_to_f32(Wg[e]).astype(np.float64).T
            u = x[t] @ bf16_bits_to_f32(Wu[e]).astype(np.float64).T
            want = g * expit(g) * u
            assert np.allclose(act[t, s], want, rtol=1e-5, atol=1e-6)
    assert np.array_equal(h, f32_to_bf16_bits(act))


def test_top1_combine_is_expert_output():
    X, lg, Wg, Wu, Wd = _small()
    r = oracle.moe(X, lg, Wg, Wu, Wd, 1, 2, 2)
    assert np.all(r["gate"] == 1.0)
    assert np.array_equal(r["y"], r["e"][:, 0, :].astype(np.float64))


def test_identical_experts():
    X, lg, Wg, Wu, Wd = _small(E=4)
    Wg[:] = Wg[0]
    Wu[:] = Wu[0]
    Wd[:] = Wd[0]
    r = oracle.moe(X, lg, Wg, Wu, Wd, 4, 2, 2)
    e = r["e"]
    for s in range(1, 4):
        assert np.array_equal(e[:, s], e[:, 0])
    assert np.allclose(r["y"], e[:, 0].astype(np.float64), rtol=4 * 2.0 ** -52, atol=1e-300)


def test_integer_down_projection_exact():
    # h integer-valued in bf16 and integer weights: every partial sum is exact
    T, Hd, E, I, k = 4, 32, 3, 64, 2
    rng = np.random.default_rng(3)
    idx = np.array([[0, 2], [1, 0], [2, 1], [0, 1]], np.int32)
    hi = rng.integers(-8, 9, size=(T, k, I))
    wi = rng.integers(-8, 9, size=(E, Hd, I))
    e = oracle.moe_down(f32_to_bf16_bits(hi.astype(np.float32)),
                        f32_to_bf16_bits(wi.astype(np.float32)), idx, 4)
    for t in range(T):
        for s in range(k):
            assert np.array_equal(e[t, s].astype(np.int64), wi[idx[t, s]] @ hi[t, s])


def test_combine_pairing_pins():
    # hand-worked outputs (tests/golden/moe_combine_pins.txt): distinct dyadic
    # gates against unit-vector expert rows, so gate k must meet slot k's row
    pins = moe_combine_pins()
    assert len(pins) == 4
    for p in pins:
        k = p["top_k"]
        gate = np.array([p["gates"]], dtype=np.float64)
        e = np.array([p["e"]], dtype=np.float32)
        assert gate.shape == (1, k) and e.shape[:2] == (1, k)
        y = oracle.moe_combine(gate, e)
        assert np.array_equal(y[0], np.array(p["y"])), (k, y[0], p["y"])
        # several tokens at once: each token pairs its own gates and rows
        g2 = np.concatenate([gate, gate[:, ::-1]])
        e2 = np.concatenate([e, e])
        y2 = oracle.moe_combine(g2, e2)
        assert np.array_equal(y2[0], y[0])
        assert np.array_equal(y2[1], (g2[1][:, None] * e2[1].astype(np.float64)).sum(0))


def test_combine_distinct_experts_float64():
    # the whole block with distinct experts: y is the gate-weighted sum of the
    # expert outputs of the same slot (a float64 product-sum of the oracle's own
    # gates and expert outputs; every term is exact in float64 up to one
    # rounding per add)
    X, lg, Wg, Wu, Wd = _small(T=12, E=16)
    r = oracle.moe(X, lg, Wg, Wu, Wd, 4, 2, 2)
    want = np.einsum("tk,tkh->th", r["gate"], r["e"].astype(np.float64))
    assert np.allclose(r["y"], want, rtol=4 * 2.0 ** -52, atol=1e-300)
    # the slots hold different experts, so a permuted pairing is far off
    swapped = np.einsum("tk,tkh->th", r["gate"][:, ::-1], r["e"].astype(np.float64))
    assert np.max(np.abs(swapped - r["y"])) > 1e-3


def test_routing_order_closed_form():
    # expert logits ln 3, ln 8, -30, ln 5: routing order (1, 3, 0) and gates
    # 8/16, 5/16, 3/16 (the full softmax's denominator cancels in the
    # renormalisation; exp(-30) only enters through it)
    lg = np.log(np.array([[3.0, 8.0, np.exp(-30.0), 5.0]])).astype(np.float32)
    lg[0, 2] = -30.0
    idx, gate = oracle.moe_route(lg, 3)
    assert idx.tolist() == [[1, 3, 0]]
    p = np.exp(lg[0, [1, 3, 0]].astype(np.float64))
    assert np.allclose(gate[0], p / p.sum(), rtol=1e-15, atol=0)
    assert np.allclose(gate[0], [0.5, 0.3125, 0.1875], rtol=1e-6, atol=0)


def test_token_permutation_equivariance():
    X, lg, Wg, Wu, Wd = _small(T=24)
    r = oracle.moe(X, lg, Wg, Wu, Wd, 4, 2, 2)
    perm = np.random.default_rng(4).permutation(24)
    r2 = oracle.moe(X[perm], lg[perm], Wg, Wu, Wd, 4, 2, 2)
    assert np.array_equal(r2["idx"], r["idx"][perm])
    assert np.array_equal(r2["h"], r["h"][perm])
    assert np.array_equal(r2["y"].view(np.uint64), r["y"][perm].view(np.uint64))


def test_bad_args_rejected():
    with pytest.raises(ValueError):
        oracle.moe_route(normal_f32(1, (4, 8)), 9)
