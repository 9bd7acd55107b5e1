"""Pins of the oracle's CPR gated delta rule (chunkwise-parallel recurrent
evaluation with a state re-sync every chunk): a hand-worked three-token
example (tests/golden/cpr_pins.txt), closed forms for pure decay (beta = 0)
and for basis keys and queries (each write replaces one state column), a
float64 evaluation of the matrix recurrence within an FP32 error bound, and
the decode-equals-prefill property the chunk re-sync exists for."""
import numpy as np
import pytest

import oracle
from iso_synth import bf16_bits_to_f32, cpr_inputs, f32_to_bf16_bits
from pins import cpr_pins

PINS = cpr_pins()


def _bits(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _golden_inputs():
    toks = PINS["tok"]
    T, d = len(toks), 2
    q = _bits([[t["q"]] for t in toks]).reshape(T, 1, d)
    k = _bits([[t["k"]] for t in toks]).reshape(T, 1, d)
    v = _bits([[t["v"]] for t in toks]).reshape(T, 1, d)
    alpha = np.array([[t["alpha"]] for t in toks], dtype=np.float32)
    beta = np.array([[t["beta"]] for t in toks], dtype=np.float32)
    S0 = np.array(PINS["B0"], dtype=np.float32).reshape(1, d, d)
    return q, k, v, alpha, beta, S0


def test_hand_worked_example():
    q, k, v, alpha, beta, S0 = _golden_inputs()
    o, snap, run = oracle.cpr_prefill(q, k, v, alpha, beta, 2, S0=S0)
    assert np.array_equal(o[:, 0, :], np.array(PINS["o"], dtype=np.float32))
    assert np.array_equal(snap[0].ravel(), np.array(PINS["snap"], dtype=np.float32))
    assert np.array_equal(run[0].ravel(), np.array(PINS["run"], dtype=np.float32))
    P, U = oracle.cpr_transition(k[:2, 0], v[:2, 0], alpha[:2, 0], beta[:2, 0])
    assert np.array_equal(P.ravel(), np.array(PINS["P"], dtype=np.float32))
    assert np.array_equal(U.ravel(), np.array(PINS["U"], dtype=np.float32))


def test_hand_worked_example_by_decode_steps():
    q, k, v, alpha, beta, S0 = _golden_inputs()
    snap = S0.copy()
    run = S0.copy()
    for t in range(3):
        o, snap, run = oracle.cpr_decode_step(q, k, v, alpha, beta, 2, t, snap, run)
        assert np.array_equal(o[0], np.array(PINS["o"][t], dtype=np.float32))
    assert np.array_equal(snap[0].ravel(), np.array(PINS["snap"], dtype=np.float32))
    assert np.array_equal(run[0].ravel(), np.array(PINS["run"], dtype=np.float32))


@pytest.mark.parametrize("T,C", [(12, 4), (13, 4), (7, 16)])
def test_pure_decay_is_a_power_of_two_scaling(T, C):
    """beta = 0, alpha = 1/2: S_t = 2^-t S_0, so o_t = 2^-(t+1) S_0 q_t.  Small
    integer states and queries keep every tree sum exact in FP32."""
    rng = np.random.default_rng(7)
    H, d = 2, 8
    S0 = rng.integers(-4, 5, size=(H, d, d)).astype(np.float32)
    qf = rng.integers(-2, 3, size=(T, H, d)).astype(np.float32)
    kf = rng.standard_normal((T, H, d)).astype(np.float32)
    vf = rng.standard_normal((T, H, d)).astype(np.float32)
    alpha = np.full((T, H), 0.5, dtype=np.float32)
    beta = np.zeros((T, H), dtype=np.float32)
    o, snap, run = oracle.cpr_prefill(_bits(qf), _bits(kf), _bits(vf), alpha, beta, C, S0=S0)
    for t in range(T):
        want = np.einsum("hij,hj->hi", S0.astype(np.float64), qf[t].astype(np.float64)) * 2.0 ** -(t + 1)
        assert np.array_equal(o[t].astype(np.float64), want)
    assert np.array_equal(snap.astype(np.float64), S0 * 2.0 ** -((T // C) * C))
    assert np.array_equal(run.astype(np.float64), S0 * 2.0 ** -T)


@pytest.mark.parametrize("T,C", [(16, 4), (13, 4), (9, 8), (5, 16)])
def test_basis_keys_replace_columns(T, C):
    """alpha = beta = 1 with k_t = e_{j_t}: the step replaces column j_t of S by
    v_t.  With q_t = e_{i_t} the output is column i_t of the new state, i.e.
    the latest v written there (or S_0's column).  Values in +-[1/2, 2) keep
    v - s exact, so the replacement is exact; the chunk form (projections,
    entries 0 or 1) is exact too."""
    rng = np.random.default_rng(11)
    H, d = 2, 8
    S0 = (rng.choice([-1, 1], size=(H, d, d)) * rng.uniform(0.5, 2.0, size=(H, d, d)))
    S0 = bf16_bits_to_f32(_bits(S0))
    vf = rng.choice([-1, 1], size=(T, H, d)) * rng.uniform(0.5, 2.0, size=(T, H, d))
    v = _bits(vf)
    kj = rng.integers(0, d, size=(T, H))
    qi = rng.integers(0, d, size=(T, H))
    eye = np.eye(d, dtype=np.float32)
    k = _bits(eye[kj])
    q = _bits(eye[qi])
    ones = np.ones((T, H), dtype=np.float32)
    o, snap, run = oracle.cpr_prefill(q, k, v, ones, ones, C, S0=S0)
    state = S0.astype(np.float64).copy()
    vv = bf16_bits_to_f32(v).astype(np.float64)
    for t in range(T):
        for h in range(H):
            state[h][:, kj[t, h]] = vv[t, h]
            assert np.array_equal(o[t, h].astype(np.float64), state[h][:, qi[t, h]])
    assert np.array_equal(run.astype(np.float64), state)
    if T % C == 0:
        assert np.array_equal(snap, run)


def _recurrence_f64(q, k, v, alpha, beta, S0):
    """S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = S_t q_t, in float64 matrix form."""
    qf, kf, vf = (bf16_bits_to_f32(x).astype(np.float64) for x in (q, k, v))
    T, H, d = qf.shape
    S = S0.astype(np.float64).copy()
    o = np.empty((T, H, d))
    eye = np.eye(d)
    for t in range(T):
        for h in range(H):
            kk = kf[t, h]
            A = alpha[t, h] * (eye - beta[t, h] * np.outer(kk, kk))
            S[h] = S[h] @ A + beta[t, h] * np.outer(vf[t, h], kk)
            o[t, h] = S[h] @ qf[t, h]
    return o, S


@pytest.mark.parametrize("T,C", [(96, 16), (70, 32), (40, 64)])
def test_close_to_the_float64_recurrence(T, C):
    """Each output is within an FP32 bound of the exact recurrence: per token
    a state entry takes ~d rounding errors of relative size 2^-24 in the tree
    sums and updates, and the map is a contraction (alpha <= 1, unit keys,
    beta <= 1), so the error grows at most linearly in T."""
    H, d = 2, 16
    x = cpr_inputs(T, H, d, seed=611)
    S0 = np.zeros((H, d, d), dtype=np.float32)
    o, _, run = oracle.cpr_prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], C, S0=S0)
    o64, S64 = _recurrence_f64(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0)
    bound = 4.0 * T * d * 2.0 ** -24 * max(1.0, np.abs(o64).max())
    assert np.abs(o - o64).max() <= bound
    if T % C != 0:
        assert np.abs(run - S64).max() <= 4.0 * T * d * 2.0 ** -24 * max(1.0, np.abs(S64).max())


def test_single_chunk_needs_no_transition():
    """With C >= T no chunk closes: outputs and the running state are the
    stepped recurrence alone, so any larger C gives the same bits."""
    x = cpr_inputs(24, 2, 16, seed=621)
    a = oracle.cpr_prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], 32)
    b = oracle.cpr_prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], 64)
    for u, w in zip(a, b):
        assert np.array_equal(u, w)


def test_resync_changes_the_state_bits():
    """The chunk form and the stepped state agree to rounding but not bit for
    bit: the re-sync is what makes prefill and decode share one boundary."""
    T, C = 32, 16
    x = cpr_inputs(T, 2, 16, seed=631)
    _, snap, run = oracle.cpr_prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], C)
    o_big, _, run_big = oracle.cpr_prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], 64)
    assert np.array_equal(snap, run)  # T is a multiple of C: run is the boundary
    assert not np.array_equal(run, run_big)
    assert np.abs(run - run_big).max() < 1e-4


@pytest.mark.parametrize("T0", [0, 5, 16, 21])
def test_decode_continues_prefill_bitwise(T0):
    """Prefill of T0 tokens, then one decode step per token up to T: outputs
    and final states equal a prefill of all T tokens, bit for bit."""
    T, C, H, d = 40, 16, 3, 16
    x = cpr_inputs(T, H, d, seed=641)
    S0 = np.zeros((H, d, d), dtype=np.float32)
    o_all, snap_all, run_all = oracle.cpr_prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], C,
                                                  S0=S0)
    if T0 > 0:
        part = {k: v[:T0] for k, v in x.items()}
        o0, snap, run = oracle.cpr_prefill(part["q"], part["k"], part["v"], part["alpha"],
                                           part["beta"], C, S0=S0)
        assert np.array_equal(o0, o_all[:T0])
    else:
        snap, run = S0.copy(), S0.copy()
    for t in range(T0, T):
        o, snap, run = oracle.cpr_decode_step(x["q"], x["k"], x["v"], x["alpha"], x["beta"], C, t,
                                              snap, run)
        assert np.array_equal(o, o_all[t])
    assert np.array_equal(snap, snap_all)
    assert np.array_equal(run, run_all)


def test_boundaries_chain_through_the_chunk_form():
    """Every boundary state is U_c + B_c P_c of the previous one, with (P_c,
    U_c) from the chunk alone."""
    T, C, H, d = 48, 16, 1, 8
    x = cpr_inputs(T, H, d, seed=651)
    _, _, _, bounds = oracle.cpr_prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], C,
                                         bounds=True)
    assert bounds.shape == (T // C + 1, H, d, d)
    assert not bounds[0].any()
    for c in range(T // C):
        sl = slice(c * C, (c + 1) * C)
        P, U = oracle.cpr_transition(x["k"][sl, 0], x["v"][sl, 0], x["alpha"][sl, 0], x["beta"][sl, 0])
        want = U.astype(np.float64) + bounds[c, 0].astype(np.float64) @ P.astype(np.float64)
        assert np.abs(bounds[c + 1, 0] - want).max() <= 8 * d * 2.0 ** -24 * max(1.0, np.abs(want).max())


def test_rejects_bad_arguments():
    x = cpr_inputs(4, 1, 6, seed=661)  # d = 6 is not a power of two
    with pytest.raises(ValueError):
        oracle.cpr_prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], 2)
    y = cpr_inputs(4, 1, 8, seed=662)
    with pytest.raises(ValueError):
        oracle.cpr_prefill(y["q"], y["k"][:3], y["v"], y["alpha"], y["beta"], 2)
    with pytest.raises(ValueError):
        oracle.cpr_prefill(y["q"], y["k"], y["v"], y["alpha"], y["beta"], 0)


def test_dot_products_are_balanced_trees():
    """The output dot product of one token with beta = 0, alpha = 1 (the state
    is unchanged) over the products [2^24, 1, 1, -2^24]: the balanced tree
    gives (2^24 + 1) + (1 - 2^24) = 2^24 + (1 - 2^24) = 1 in FP32 (2^24 + 1
    rounds to 2^24), a left-to-right sum gives 0 and a right-to-left sum 2.
    Every CPR dot product (step, chunk form, pass) is this one tree."""
    d = 4
    S0 = np.zeros((1, d, d), dtype=np.float32)
    S0[0, 0] = [2.0 ** 24, 1.0, 1.0, -(2.0 ** 24)]
    S0[0, 1] = [-(2.0 ** 24), 1.0, 1.0, 2.0 ** 24]  # tree 1, left-to-right 2, right-to-left 0
    q = _bits(np.ones((1, 1, d)))
    k = _bits(np.full((1, 1, d), 0.5))
    v = _bits(np.zeros((1, 1, d)))
    one = np.ones((1, 1), dtype=np.float32)
    zero = np.zeros((1, 1), dtype=np.float32)
    o, _, run = oracle.cpr_prefill(q, k, v, one, zero, 4, S0=S0)
    assert o[0, 0, 0] == 1.0
    assert o[0, 0, 1] == 1.0
    assert np.array_equal(run, S0)
