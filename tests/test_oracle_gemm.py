"""Pins of the oracle's leaf/tree GEMM against facts fixed outside the oracle.

* hand-derived tree-order bit patterns (tests/golden/tree_order_pins.txt);
* integer-valued inputs, whose every partial sum is exact in FP32, against
  numpy's int64 product;
* random inputs against a float64 product, within the rigorous FP32 bound
  gamma_{m-1+log2 L} * sum|a*b| of a sequential leaf sum plus the tree levels;
* the oracle's own batch- and partition-invariance.
"""
import math

import numpy as np
import pytest

import oracle
from iso_synth import bf16_bits_to_f32, f32_to_bf16_bits, normal_bf16
from pins import f32_bits, tree_case_inputs, tree_pins


def _fold(vals, order):
    """Reference folds in float32 used only to show a pin discriminates."""
    v = [np.float32(x) for x in vals]
    if order == "sequential":
        s = v[0]
        for x in v[1:]:
            s = np.float32(s + x)
        return s
    if order == "reverse":
        s = v[-1]
        for x in reversed(v[:-1]):
            s = np.float32(s + x)
        return s
    if order == "interleaved":  # pairs (i, i + n/2) at every level
        while len(v) > 1:
            h = len(v) // 2
            v = [np.float32(v[i] + v[i + h]) for i in range(h)]
        return v[0]
    raise ValueError(order)


@pytest.mark.parametrize("pin", tree_pins(), ids=lambda p: f"{p['kind']}-L{p['leaves']}")
def test_tree_order_pins(pin):
    # the pin must tell the orders apart (or be documented as not doing so)
    assert int(f32_bits(_fold(pin["values"], "sequential"))) == pin["sequential"]
    assert int(f32_bits(_fold(pin["values"], pin["other_name"]))) == pin["other"]
    leaf_size = 64
    A, Wt = tree_case_inputs(pin, leaf_size, rows=3, cols=5)
    L = pin["leaves"] if pin["kind"] == "tree" else 1
    C = oracle.gemm(A, Wt, L)
    want = pin["balanced"] if pin["kind"] == "tree" else pin["sequential"]
    assert np.all(f32_bits(C) == want), hex(int(f32_bits(C)[0, 0]))


@pytest.mark.parametrize("P", [1, 2, 4])
def test_tree_pins_under_partitions(P):
    for pin in tree_pins():
        if pin["kind"] != "tree" or pin["leaves"] % P:
            continue
        A, Wt = tree_case_inputs(pin, 32, rows=2, cols=2)
        C = oracle.gemm_partitioned(A, Wt, pin["leaves"], P)
        assert np.all(f32_bits(C) == pin["balanced"])


@pytest.mark.parametrize("M,N,K,L", [(5, 7, 256, 4), (3, 33, 2048, 8), (2, 4, 4096, 16), (1, 1, 32, 1)])
def test_integer_inputs_exact(M, N, K, L):
    rng = np.random.default_rng(7 + K)
    ai = rng.integers(-8, 9, size=(M, K))
    wi = rng.integers(-8, 9, size=(N, K))
    A = f32_to_bf16_bits(ai.astype(np.float32))
    Wt = f32_to_bf16_bits(wi.astype(np.float32))
    C = oracle.gemm(A, Wt, L)
    exact = ai.astype(np.int64) @ wi.astype(np.int64).T
    assert np.array_equal(C.astype(np.int64), exact)
    assert np.array_equal(C, exact.astype(np.float32))


def _gamma(n):
    u = 2.0 ** -24
    return n * u / (1 - n * u)


@pytest.mark.parametrize("M,N,K,L,sa,sw", [
    (8, 64, 256, 4, 1.0, 0.05),     # the tiny workload's shape family
    (4, 16, 2048, 8, 1.0, 0.02),    # prefill / LM-head leaf structure
    (2, 8, 4096, 16, 1.0, 0.02),    # invariance-sweep leaf structure
    (3, 5, 2048, 4, 1.0, 0.02),     # MoE gate/up leaf structure
])
def test_random_against_float64(M, N, K, L, sa, sw):
    A = normal_bf16(11 + M, (M, K), sa)
    Wt = normal_bf16(12 + N, (N, K), sw)
    C = oracle.gemm(A, Wt, L).astype(np.float64)
    a = bf16_bits_to_f32(A).astype(np.float64)
    w = bf16_bits_to_f32(Wt).astype(np.float64)
    exact = a @ w.T
    absdot = np.abs(a) @ np.abs(w).T
    m = K // L
    bound = _gamma(m - 1 + int(math.log2(L))) * absdot
    err = np.abs(C - exact)
    assert np.all(err <= bound)
    # the random case is not degenerate: the 1e-5 tolerance is well above the error
    assert np.all(err <= 1e-5 * absdot)


def test_transpose_mistake_is_caught():
    # A non-square case where using W instead of W^T would index wrongly.
    A = normal_bf16(21, (3, 128), 1.0)
    Wt = normal_bf16(22, (5, 128), 0.05)
    C = oracle.gemm(A, Wt, 4)
    exact = bf16_bits_to_f32(A).astype(np.float64) @ bf16_bits_to_f32(Wt).astype(np.float64).T
    assert C.shape == (3, 5)
    assert np.allclose(C, exact, rtol=0, atol=1e-4)


def test_batch_embedding_invariance():
    K, N, L = 1024, 48, 8
    Wt = normal_bf16(31, (N, K), 0.02)
    probes = normal_bf16(32, (4, K), 1.0)
    filler = normal_bf16(33, (64, K), 1.0)
    alone = np.stack([oracle.gemm(probes[i:i + 1], Wt, L)[0] for i in range(4)])
    for batch in (8, 64):
        X = filler[:batch].copy()
        pos = [0, batch - 1, batch // 2, 1]
        for i, p in enumerate(pos):
            X[p] = probes[i]
        C = oracle.gemm(X, Wt, L)
        for i, p in enumerate(pos):
            assert np.array_equal(f32_bits(C[p]), f32_bits(alone[i]))


@pytest.mark.parametrize("L", [8, 16])
def test_partition_invariance(L):
    K = 64 * L
    A = normal_bf16(41, (6, K), 1.0)
    Wt = normal_bf16(42, (10, K), 0.02)
    base = f32_bits(oracle.gemm(A, Wt, L))
    for P in (1, 2, 4, 8):
        assert np.array_equal(f32_bits(oracle.gemm_partitioned(A, Wt, L, P)), base)


def test_elems_match_full():
    A = normal_bf16(51, (9, 512), 1.0)
    Wt = normal_bf16(52, (17, 512), 0.05)
    C = oracle.gemm(A, Wt, 4)
    rows = np.array([0, 8, 3, 3, 7])
    cols = np.array([0, 16, 5, 6, 0])
    assert np.array_equal(f32_bits(oracle.gemm_elems(A, Wt, 4, rows, cols)), f32_bits(C[rows, cols]))


def test_leaf_order_changes_bits():
    """Guard against a silently order-free oracle: a different leaf count over
    the same data must change some bits on random data."""
    A = normal_bf16(61, (16, 2048), 1.0)
    Wt = normal_bf16(62, (64, 2048), 0.02)
    c8 = f32_bits(oracle.gemm(A, Wt, 8))
    c1 = f32_bits(oracle.gemm(A, Wt, 1))
    assert np.count_nonzero(c8 != c1) > 0


@pytest.mark.parametrize("args", [(4, 3), (5, 1)])
def test_bad_shapes_rejected(args):
    K, L = 257, args[0]
    A = np.zeros((1, K), np.uint16)
    Wt = np.zeros((1, K), np.uint16)
    with pytest.raises(ValueError):
        oracle.gemm(A, Wt, L)
