"""The vocabulary-sharded LM-head (iso_lmhead_shard_stats + iso_lmhead_finish)
gives the bits of the single fused call for every shard count, shard order
and ragged vocabulary, and agrees with the oracle within 1e-5; a decode loop
(one row per call) gives the bits of the prefill call over the same rows and
agrees with the oracle at every step.  Stand-in for a vocabulary-parallel
LM-head whose ranks exchange only per-chunk (max, sum) pairs and the target
logit ("IsoExec: Eliminating Trainer-Inference Mismatch in SkyRL", section
"Achieving Parallelism Invariance": partials combine by the fixed tree
whatever the layout)."""
import numpy as np
import pytest

import oracle
from gpu_util import LOGPROB_ATOL, dev, dev_i32, host, note, torch
from iso_synth import make_config, normal_bf16, uniform_tokens

pytestmark = pytest.mark.gpu

iso = pytest.importorskip("parallelism_invariant_numerics_amd")


def _shard_bounds(V, S):
    """S contiguous shards of whole 128-id chunks (the last may be ragged)."""
    nchunk = (V + 127) // 128
    cuts = [round(i * nchunk / S) * 128 for i in range(S)] + [V]
    return [(cuts[i], min(cuts[i + 1], V)) for i in range(S) if cuts[i] < min(cuts[i + 1], V)]


def _sharded(dH, dW, dtok, c, V, S=None, reverse=False, bounds=None):
    t = torch()
    M = dH.shape[0]
    nchunk = (V + 127) // 128
    stats = t.empty((M, nchunk, 2), dtype=t.float32, device="cuda")
    target = t.empty(M, dtype=t.float32, device="cuda")
    bounds = bounds or _shard_bounds(V, S)
    for vb, ve in (reversed(bounds) if reverse else bounds):
        iso.lmhead_shard_stats(dH, dW[vb:ve], dtok, c, V, vb, stats, target)
    out = iso.lmhead_finish(stats, target, dtok, V)
    t.cuda.synchronize()
    return host(out)


def _check_oracle(got, want, what):
    bad = np.isnan(want)
    assert np.array_equal(np.isnan(got), bad), what
    assert np.max(np.abs(got[~bad] - want[~bad]), initial=0.0) <= LOGPROB_ATOL, what


@pytest.mark.parametrize("V", [5000, 4096, 130])
def test_shard_counts_give_the_fused_bits(V):
    M, K, L = 300, 512, 4
    note(f"vocab shards V={V}")
    H = normal_bf16(71, (M, K), 1.0)
    W = normal_bf16(72, (V, K), 0.05)
    tok = uniform_tokens(73, M, V)
    tok[::37] = -1          # bad ids: NaN either way
    tok[5] = V
    c = iso.contract(L, K // L, 128)
    dH, dW, dtok = dev(H), dev(W), dev_i32(tok)
    ref = host(iso.lmhead_logprob(dH, dW, dtok, c))
    assert np.isnan(ref[::37]).all() and np.isnan(ref[5])
    want, _, _ = oracle.lmhead_logprob(H, W, tok, L)
    _check_oracle(ref, want, "fused")
    for S in (1, 2, 3, 4, 8):
        if S > (V + 127) // 128:
            continue
        got = _sharded(dH, dW, dtok, c, V, S, reverse=(S % 2 == 0))
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), S
        _check_oracle(got, want, f"{S} shards")


def test_ragged_shards_and_boundary_tokens():
    # unequal shards (one chunk, many chunks, a ragged last chunk), sampled
    # tokens on both sides of every shard boundary and in the ragged tail
    M, K, L, V = 96, 256, 4, 3000
    H = normal_bf16(91, (M, K), 1.0)
    W = normal_bf16(92, (V, K), 0.05)
    bounds = [(0, 128), (128, 1280), (1280, 1408), (1408, 2944), (2944, V)]
    tok = uniform_tokens(93, M, V)
    edges = [b for b, _ in bounds[1:]] + [e - 1 for _, e in bounds]
    tok[:len(edges)] = edges
    tok[len(edges)] = V - 1
    tok[len(edges) + 1] = 2944
    tok[-1] = V + 7          # out of range: NaN
    tok[-2] = -2
    note("vocab shards: ragged cuts, boundary tokens")
    c = iso.contract(L, K // L, 128)
    dH, dW, dtok = dev(H), dev(W), dev_i32(tok)
    want, _, _ = oracle.lmhead_logprob(H, W, tok, L)
    ref = host(iso.lmhead_logprob(dH, dW, dtok, c))
    for rev in (False, True):
        got = _sharded(dH, dW, dtok, c, V, bounds=bounds, reverse=rev)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), rev
        _check_oracle(got, want, f"ragged shards reverse={rev}")
    assert np.isnan(ref[-1]) and np.isnan(ref[-2])


def test_decode_loop_matches_prefill():
    # one row per call (a decode step) against one call over all the rows,
    # and every step against the oracle
    M, K, V, L = 32, 1024, 3000, 8
    H = normal_bf16(81, (M, K), 1.0)
    W = normal_bf16(82, (V, K), 0.02)
    tok = uniform_tokens(83, M, V)
    tok[3] = 2944            # first id of the ragged last chunk
    tok[4] = V - 1
    c = iso.contract(L, K // L, 128)
    dH, dW, dtok = dev(H), dev(W), dev_i32(tok)
    note("decode loop: prefill call")
    prefill = host(iso.lmhead_logprob(dH, dW, dtok, c))
    want, _, _ = oracle.lmhead_logprob(H, W, tok, L)
    _check_oracle(prefill, want, "prefill")
    for i in range(M):
        step = host(iso.lmhead_logprob(dH[i:i + 1].contiguous(), dW, dtok[i:i + 1].contiguous(), c))
        assert step.view(np.uint32)[0] == prefill.view(np.uint32)[i]
        assert abs(float(step[0]) - want[i]) <= LOGPROB_ATOL, i
        shard = _sharded(dH[i:i + 1].contiguous(), dW, dtok[i:i + 1].contiguous(), c, V, 4)
        assert shard.view(np.uint32)[0] == prefill.view(np.uint32)[i]
        assert abs(float(shard[0]) - want[i]) <= LOGPROB_ATOL, i


def test_full_size_eight_vocabulary_shards():
    lm = make_config("lmhead")
    note("vocab shards full size (8 shards of the 151936 vocabulary)")
    dH, dW = dev(lm["H"]), dev(lm["Wvt"])
    dtok = dev_i32(lm["tok"])
    c = iso.contract(lm["leaves"], lm["K"] // lm["leaves"], 128)
    ref = host(iso.lmhead_logprob(dH, dW, dtok, c))
    got = _sharded(dH, dW, dtok, c, lm["V"], 8)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # sampled rows against the oracle (every row costs 0.6 GFLOP on the host)
    rows = np.array([0, 1, 4095, 8191, 2222, 6000])
    want, _, _ = oracle.lmhead_logprob(lm["H"][rows], lm["Wvt"], lm["tok"][rows], lm["leaves"])
    _check_oracle(got[rows], want, "full size, 8 shards")
