"""Pins of the oracle's sampled-token logprob against closed forms,
scipy's log_softmax and vocabulary-permutation equivariance."""
import numpy as np
import pytest
from scipy.special import log_softmax

import oracle
from iso_synth import f32_to_bf16_bits, normal_bf16, uniform_tokens
from pins import logsoftmax_forms


def _forms():
    return {(f["V"], f["case"]): f["expected"] for f in logsoftmax_forms()}


@pytest.mark.parametrize("V", [512, 151936])
def test_uniform_logits_give_minus_log_v(V):
    K = 64
    H = normal_bf16(1, (3, K), 1.0)
    Wvt = np.zeros((V, K), np.uint16)  # W = 0: every logit is exactly 0
    tok = np.array([0, V - 1, V // 3], np.int32)
    lp, zt, _ = oracle.lmhead_logprob(H, Wvt, tok, 2)
    want = _forms()[(V, "uniform")]
    assert np.all(zt == 0.0)
    assert np.allclose(lp, want, rtol=0, atol=1e-13)


def test_single_spike():
    V, K = 151936, 64
    H = np.zeros((2, K), np.uint16)
    H[:, 5] = f32_to_bf16_bits(np.float32([4.0]))[0]
    Wvt = np.zeros((V, K), np.uint16)
    j0 = 12345
    Wvt[j0, 5] = f32_to_bf16_bits(np.float32([5.0]))[0]  # z[j0] = 20 exactly
    tok = np.array([j0, 7], np.int32)
    lp, zt, _ = oracle.lmhead_logprob(H, Wvt, tok, 2)
    f = _forms()
    assert zt[0] == 20.0 and zt[1] == 0.0
    # float64 sequential sum of V terms near 1: error at most V * 2^-53 per step
    tol = V * 2.0 ** -52
    assert abs(lp[0] - f[(V, "spike20_t")]) < tol
    assert abs(lp[1] - f[(V, "spike20_o")]) < tol


@pytest.mark.parametrize("M,V,K,L", [(8, 512, 256, 4), (4, 1000, 512, 8), (3, 4099, 256, 2)])
def test_against_scipy_log_softmax(M, V, K, L):
    H = normal_bf16(3, (M, K), 1.0)
    Wvt = normal_bf16(4, (V, K), 0.05)
    tok = uniform_tokens(5, M, V)
    lp, zt, lse = oracle.lmhead_logprob(H, Wvt, tok, L)
    z = oracle.gemm(H, Wvt, L).astype(np.float64)
    ref = log_softmax(z, axis=1)[np.arange(M), tok]
    assert np.allclose(lp, ref, rtol=0, atol=1e-12)
    assert np.array_equal(zt, z[np.arange(M), tok].astype(np.float32))


def test_vocab_permutation_equivariance():
    M, V, K = 5, 700, 256
    H = normal_bf16(6, (M, K), 1.0)
    Wvt = normal_bf16(7, (V, K), 0.05)
    tok = uniform_tokens(8, M, V)
    lp, _, _ = oracle.lmhead_logprob(H, Wvt, tok, 4)
    perm = np.random.default_rng(9).permutation(V)   # new row q holds old row perm[q]
    inv = np.argsort(perm)
    lp2, _, _ = oracle.lmhead_logprob(H, Wvt[perm], inv[tok].astype(np.int32), 4)
    # only the order of the float64 exp-sum changes
    assert np.allclose(lp, lp2, rtol=0, atol=1e-12)


def test_bad_token_gives_nan():
    H = normal_bf16(10, (3, 64), 1.0)
    Wvt = normal_bf16(11, (32, 64), 0.05)
    lp, _, _ = oracle.lmhead_logprob(H, Wvt, np.array([-1, 32, 3], np.int32), 1)
    assert np.isnan(lp[0]) and np.isnan(lp[1]) and np.isfinite(lp[2])
