"""GPU parity of iso_lmhead_logprob with the oracle (|diff| <= 1e-5 per
logprob), closed forms, ragged vocabularies and rows, invariance of each row's
bits across batch size, row position and partitions, and the LM-head workload
at full size (8192 x 2048 hidden, 151936 vocabulary) on sampled rows."""
import math

import numpy as np
import pytest

import oracle
from gpu_util import LOGPROB_ATOL, dev, dev_i32, host, note, torch, u32
from iso_synth import make_config, normal_bf16, uniform_tokens

pytestmark = pytest.mark.gpu

iso = pytest.importorskip("parallelism_invariant_numerics_amd")


def _lp(H, Wvt, tok, L, P=1, dWvt=None):
    c = iso.contract(L, H.shape[1] // L, 128)
    out = iso.lmhead_logprob(dev(H), dWvt if dWvt is not None else dev(Wvt), dev_i32(tok), c,
                             partitions=P)
    torch().cuda.synchronize()
    return host(out)


def test_tiny_workload_parity():
    cfg = make_config("tiny")
    note("tiny logprob")
    got = _lp(cfg["A"], cfg["Wt"], cfg["tok"], cfg["leaves"])
    want, _, _ = oracle.lmhead_logprob(cfg["A"], cfg["Wt"], cfg["tok"], cfg["leaves"])
    assert np.max(np.abs(got - want)) <= LOGPROB_ATOL


@pytest.mark.parametrize("V", [512, 151936])
def test_uniform_logits(V):
    K = 128
    H = normal_bf16(1, (4, K), 1.0)
    Wvt = np.zeros((V, K), np.uint16)
    tok = np.array([0, V - 1, 5, V // 2], np.int32)
    note(f"uniform logits V={V}")
    got = _lp(H, Wvt, tok, 2)
    assert np.max(np.abs(got.astype(np.float64) + math.log(V))) <= 4e-6


@pytest.mark.parametrize("M,V,K,L", [(1, 1000, 256, 4), (130, 4099, 512, 8), (3, 127, 256, 2),
                                     (257, 129, 1024, 16), (5, 2000, 2048, 32), (9, 300, 256, 1)])
def test_ragged_parity(M, V, K, L):
    H = normal_bf16(M + 3, (M, K), 1.0)
    Wvt = normal_bf16(V + 4, (V, K), 0.05)
    tok = uniform_tokens(M + V, M, V)
    note(f"ragged logprob M={M} V={V} K={K} L={L}")
    got = _lp(H, Wvt, tok, L)
    want, _, _ = oracle.lmhead_logprob(H, Wvt, tok, L)
    assert np.max(np.abs(got - want)) <= LOGPROB_ATOL


def test_bad_tokens_give_nan():
    H = normal_bf16(2, (3, 256), 1.0)
    Wvt = normal_bf16(3, (300, 256), 0.05)
    note("bad token ids")
    got = _lp(H, Wvt, np.array([-1, 300, 7], np.int32), 4)
    assert np.isnan(got[0]) and np.isnan(got[1]) and np.isfinite(got[2])


def test_row_invariance_batches_and_partitions():
    K, V, L = 2048, 5000, 8
    probes = normal_bf16(21, (64, K), 1.0)
    filler = normal_bf16(22, (300, K), 1.0)
    Wvt = normal_bf16(23, (V, K), 0.02)
    tok = uniform_tokens(24, 64, V)
    dW = dev(Wvt)
    note("logprob reference: batch 1")
    ref = np.array([_lp(probes[i:i + 1], None, tok[i:i + 1], L, 1, dW)[0] for i in range(64)],
                   np.float32)
    want, _, _ = oracle.lmhead_logprob(probes, Wvt, tok, L)
    assert np.max(np.abs(ref - want)) <= LOGPROB_ATOL
    rng = np.random.default_rng(25)
    ftok = uniform_tokens(26, 300, V)
    for P in (1, 2, 4, 8):
        note(f"logprob batch 64 P={P}")
        assert np.array_equal(u32(_lp(probes, None, tok, L, P, dW)), u32(ref)), P
        for batch in (8, 130, 300):
            pos = rng.choice(batch, 8, replace=False)
            ids = rng.choice(64, 8, replace=False)
            X = filler[:batch].copy()
            t = ftok[:batch].copy()
            X[pos] = probes[ids]
            t[pos] = tok[ids]
            note(f"logprob batch {batch} P={P}")
            got = _lp(X, None, t, L, P, dW)
            assert np.array_equal(u32(got[pos]), u32(ref[ids])), (batch, P)


def test_lmhead_full_size_sampled():
    cfg = make_config("lmhead")
    H, Wvt, tok, L = cfg["H"], cfg["Wvt"], cfg["tok"], cfg["leaves"]
    note("lmhead full size 8192 x 2048 x 151936")
    dW = dev(Wvt)
    got = _lp(H, None, tok, L, 1, dW)
    rows = np.array([0, 127, 128, 4095, 8191, 777, 5000, 6001])
    want, _, _ = oracle.lmhead_logprob(H[rows], Wvt, tok[rows], L)
    assert np.max(np.abs(got[rows] - want)) <= LOGPROB_ATOL
    note("lmhead full-size rows re-evaluated as a batch of 8")
    small = _lp(H[rows], None, tok[rows], L, 1, dW)
    assert np.array_equal(u32(small), u32(got[rows]))
    assert np.all(np.isfinite(got)) and np.all(got <= 0)


@pytest.mark.parametrize("K,L,V", [(256, 4, 1000), (512, 4, 77), (512, 8, 1200), (1024, 8, 300),
                                   (2048, 8, 5000), (4096, 8, 700)])
def test_decode_rows_match_batch(K, L, V):
    """One to 16 rows take the decode kernel (weights streamed to registers, one workgroup per
    CU); the same rows inside a batch of 40 take the fused kernel.  Same bits, ragged and
    sub-chunk vocabularies, bad token ids, and leaf sizes the decode kernel does not take."""
    H = normal_bf16(K + V, (40, K), 1.0)
    Wvt = normal_bf16(K + V + 1, (V, K), 0.05)
    tok = uniform_tokens(K + 2, 40, V)
    tok[3], tok[5], tok[21] = V - 1, -1, V
    dW = dev(Wvt)
    note(f"decode rows vs batch K={K} L={L} V={V}")
    big = _lp(H, None, tok, L, 1, dW)
    for m in (1, 7, 16):
        for start in (0, 20):
            small = _lp(H[start:start + m], None, tok[start:start + m], L, 1, dW)
            assert np.array_equal(u32(small), u32(big[start:start + m])), (m, start)
    want, _, _ = oracle.lmhead_logprob(H[:16], Wvt, tok[:16], L)
    ok = np.isfinite(want)
    assert np.array_equal(ok, np.isfinite(big[:16]))
    assert np.max(np.abs(big[:16][ok] - want[ok])) <= LOGPROB_ATOL
