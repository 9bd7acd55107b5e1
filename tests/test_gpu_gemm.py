"""GPU parity of iso_gemm with the CPU oracle, through the C ABI.

* exact cases (tree-order pins, integer inputs): bit for bit;
* random cases: |gpu - oracle| <= 1e-5 * sum_k |a_k b_k| per element;
* partitions P = 1, 2, 4, 8: identical bits;
* bf16 output: the FP32 root rounded to nearest-even, bit for bit;
* the prefill workload at full size (4096 x 2048 x 2048, 8 leaves of 256):
  sampled elements against the oracle, all elements across P and output dtypes.
"""
import ctypes

import numpy as np
import pytest

import oracle
from gpu_util import absdot, check_gemm_tol, dev, host, note, torch, u32
from iso_synth import f32_to_bf16_bits, make_config, normal_bf16
from pins import tree_case_inputs, tree_pins

pytestmark = pytest.mark.gpu

iso = pytest.importorskip("parallelism_invariant_numerics_amd")


def _run(A, Wt, L, P=1, out_dtype=None):
    K = A.shape[1]
    c = iso.contract(L, K // L, 0)
    out = iso.gemm(dev(A), dev(Wt), c, partitions=P, out_dtype=out_dtype or iso.F32)
    torch().cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("P", [1, 2, 4])
def test_tree_order_pins_bitwise(P):
    for pin in tree_pins():
        if pin["kind"] != "tree" or pin["leaves"] % P:
            continue
        note(f"tree pin L={pin['leaves']} P={P}")
        A, Wt = tree_case_inputs(pin, 64, rows=3, cols=5)
        C = _run(A, Wt, pin["leaves"], P)
        assert np.all(u32(C) == pin["balanced"]), hex(int(u32(C)[0, 0]))


@pytest.mark.parametrize("M,N,K,L", [(1, 1, 64, 1), (65, 129, 256, 4), (300, 200, 2048, 8),
                                     (128, 128, 4096, 16), (7, 300, 512, 2), (129, 17, 1024, 16)])
def test_integer_inputs_exact(M, N, K, L):
    note(f"integer exact M={M} N={N} K={K} L={L}")
    rng = np.random.default_rng(M * 7 + N)
    ai = rng.integers(-8, 9, size=(M, K))
    wi = rng.integers(-8, 9, size=(N, K))
    C = _run(f32_to_bf16_bits(ai.astype(np.float32)), f32_to_bf16_bits(wi.astype(np.float32)), L)
    assert np.array_equal(C.astype(np.int64), ai @ wi.T)


def test_tiny_workload_parity():
    cfg = make_config("tiny")
    note("tiny workload 8x256x512, 4 leaves of 64")
    C = _run(cfg["A"], cfg["Wt"], cfg["leaves"])
    ref = oracle.gemm(cfg["A"], cfg["Wt"], cfg["leaves"])
    check_gemm_tol(C, ref, absdot(cfg["A"], cfg["Wt"]), "tiny")


@pytest.mark.parametrize("M,N,K,L", [(257, 383, 1024, 8), (33, 640, 512, 2), (1, 130, 2048, 8),
                                     (130, 1, 256, 4), (200, 300, 4096, 16), (64, 64, 2048, 32),
                                     (40, 72, 4096, 64)])
def test_random_ragged_parity(M, N, K, L):
    note(f"random ragged M={M} N={N} K={K} L={L}")
    A = normal_bf16(M + 1, (M, K), 1.0)
    Wt = normal_bf16(N + 2, (N, K), 0.02)
    C = _run(A, Wt, L)
    check_gemm_tol(C, oracle.gemm(A, Wt, L), absdot(A, Wt), f"{M}x{N}x{K}/L{L}")


@pytest.mark.parametrize("L", [8, 16])
def test_partitions_bitwise(L):
    M, N, K = 200, 300, 256 * L
    A = normal_bf16(5, (M, K), 1.0)
    Wt = normal_bf16(6, (N, K), 0.02)
    note(f"partitions L={L}")
    base = u32(_run(A, Wt, L, 1))
    for P in (2, 4, 8):
        assert np.array_equal(u32(_run(A, Wt, L, P)), base), P
    bf = _run(A, Wt, L, 1, iso.BF16)
    assert np.array_equal(bf, f32_to_bf16_bits(base.view(np.float32)))


def test_half_empty_tiles_bitwise():
    """Row tiles with at most 64 rows (the lower waves of the tile then only keep the
    stage ring going) under every partition count, FP32 and bf16: the same bits as the
    same rows inside a batch of 600, and the oracle's values within tolerance."""
    K, N, L = 2048, 384, 8
    A = normal_bf16(31, (600, K), 1.0)
    Wt = normal_bf16(32, (N, K), 0.02)
    note("half-empty tiles")
    big = u32(_run(A, Wt, L))
    bigb = _run(A, Wt, L, 1, iso.BF16)
    for m in (64, 129, 192):  # one 64-row tile; 128 + 1; 128 + 64
        for P in (1, 2, 4, 8):
            assert np.array_equal(u32(_run(A[:m], Wt, L, P)), big[:m]), (m, P)
            assert np.array_equal(_run(A[:m], Wt, L, P, iso.BF16), bigb[:m]), (m, P, "bf16")
    rows = np.array([0, 63, 128, 191])
    check_gemm_tol(big[rows].view(np.float32), oracle.gemm(A[rows], Wt, L), absdot(A[rows], Wt),
                   "half-empty tiles")


def test_run_to_run_determinism():
    A = normal_bf16(7, (513, 2048), 1.0)
    Wt = normal_bf16(8, (257, 2048), 0.02)
    note("determinism x3")
    runs = [u32(_run(A, Wt, 8)) for _ in range(3)]
    assert np.array_equal(runs[0], runs[1]) and np.array_equal(runs[0], runs[2])


def test_bits_across_streams_and_launch_order():
    # the same GEMM enqueued on two streams (default priority) that run at
    # the same time, each behind other work, in both launch orders, and with
    # its partitions' roots on a third: every result has the bits of a lone
    # call on the current stream (no float atomics, no order from timing)
    t = torch()
    A = normal_bf16(17, (1100, 2048), 1.0)
    Wt = normal_bf16(18, (700, 2048), 0.02)
    A2 = normal_bf16(19, (3000, 2048), 1.0)
    c = iso.contract(8, 256, 0)
    dA, dW, dA2 = dev(A), dev(Wt), dev(A2)
    note("streams: reference call")
    ref = u32(host(iso.gemm(dA, dW, c)))
    t.cuda.synchronize()
    s1, s2, s3 = t.cuda.Stream(), t.cuda.Stream(), t.cuda.Stream()
    outs = []
    for order in range(2):
        note(f"streams: concurrent calls, order {order}")
        o = [t.empty((1100, 700), dtype=t.float32, device="cuda") for _ in range(3)]
        f = [t.empty((3000, 700), dtype=t.float32, device="cuda") for _ in range(2)]
        ws = t.empty(iso.gemm_workspace(c, 1100, 700, 4), dtype=t.uint8, device="cuda")
        t.cuda.synchronize()
        first, second = (s1, s2) if order == 0 else (s2, s1)
        with t.cuda.stream(first):
            iso.gemm(dA2, dW, c, out=f[0])       # other work ahead of the call
            iso.gemm(dA, dW, c, out=o[0])
        with t.cuda.stream(second):
            iso.gemm(dA, dW, c, out=o[1])
            iso.gemm(dA2, dW, c, out=f[1])
        with t.cuda.stream(s3):
            iso.gemm(dA, dW, c, out=o[2], partitions=4, workspace=ws)
        t.cuda.synchronize()
        outs += [u32(host(x)) for x in o]
    for i, x in enumerate(outs):
        assert np.array_equal(x, ref), i


def test_empty_problem():
    c = iso.contract(4, 64, 0)
    t = torch()
    A = t.empty((0, 256), dtype=t.bfloat16, device="cuda")
    Wt = t.zeros((8, 256), dtype=t.bfloat16, device="cuda")
    out = iso.gemm(A, Wt, c)
    assert out.shape == (0, 8)


def test_prefill_full_size():
    cfg = make_config("prefill")
    A, Wt, L = cfg["A"], cfg["Wt"], cfg["leaves"]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    c = iso.contract(L, K // L, 0)
    t = torch()
    dA, dW = dev(A), dev(Wt)
    note("prefill full size P=1 fp32")
    base = iso.gemm(dA, dW, c)
    t.cuda.synchronize()
    C = host(base)
    rng = np.random.default_rng(2024)
    rows = np.concatenate([[0, 0, M - 1, M - 1, 127, 128], rng.integers(0, M, 1500)])
    cols = np.concatenate([[0, N - 1, 0, N - 1, 127, 128], rng.integers(0, N, 1500)])
    ref = oracle.gemm_elems(A, Wt, L, rows, cols)
    check_gemm_tol(C[rows, cols], ref, absdot(A, Wt, rows, cols), "prefill sampled")
    for P in (2, 4, 8):
        note(f"prefill full size P={P}")
        out = iso.gemm(dA, dW, c, partitions=P)
        t.cuda.synchronize()
        assert np.array_equal(u32(host(out)), u32(C)), P
    note("prefill full size bf16 out")
    bf = host(iso.gemm(dA, dW, c, out_dtype=iso.BF16))
    assert np.array_equal(bf, f32_to_bf16_bits(C))


@pytest.mark.parametrize("M,N,K,L", [(4100, 2100, 2048, 4), (2048, 4000, 2048, 2), (4000, 2304, 1024, 1)])
def test_wide_tile_ragged(M, N, K, L):
    """Shapes that take the 128 x 256 tile kernel (at most four leaves per workgroup, at least
    16 stages, a tile per CU), with ragged M and N: sampled elements (edges and the 256-column
    tile boundaries included) against the oracle; every element equal across partitions (P = 2
    also wide, P = 4 and 8 on the 128 x 128 kernels), bf16 output, and the last 70 rows alone
    (a small batch on other kernels)."""
    t = torch()
    A = normal_bf16(M + L, (M, K), 1.0)
    Wt = normal_bf16(N + L, (N, K), 0.02)
    c = iso.contract(L, K // L, 0)
    dA, dW = dev(A), dev(Wt)
    note(f"wide tile M={M} N={N} K={K} L={L}")
    C = host(iso.gemm(dA, dW, c))
    rng = np.random.default_rng(M + N)
    rows = np.concatenate([[0, M - 1, M - 1, 127, 128, M - 1], rng.integers(0, M, 600)])
    cols = np.concatenate([[N - 1, 0, 255, 256, 255, N - 1 - (N - 1) % 256], rng.integers(0, N, 600)])
    check_gemm_tol(C[rows, cols], oracle.gemm_elems(A, Wt, L, rows, cols),
                   absdot(A, Wt, rows, cols), "wide sampled")
    for P in (2, 4, 8):
        if L % P:
            continue
        note(f"wide tile P={P}")
        assert np.array_equal(u32(host(iso.gemm(dA, dW, c, partitions=P))), u32(C)), P
    note("wide tile bf16 out")
    assert np.array_equal(host(iso.gemm(dA, dW, c, out_dtype=iso.BF16)), f32_to_bf16_bits(C))
    note("wide tile last 70 rows alone")
    tail = host(iso.gemm(dev(A[M - 70:]), dW, c))
    assert np.array_equal(u32(tail), u32(C[M - 70:]))


def test_baseline_accuracy():
    M, N, K = 129, 257, 2048
    A = normal_bf16(9, (M, K), 1.0)
    Wt = normal_bf16(10, (N, K), 0.02)
    note("baseline accuracy")
    out = iso.gemm_baseline(dev(A), dev(Wt))
    torch().cuda.synchronize()
    check_gemm_tol(host(out), oracle.gemm(A, Wt, 8), absdot(A, Wt), "baseline")


@pytest.mark.parametrize("M,N", [(65, 257), (64, 256), (3, 5)])
def test_partition_combine_shapes(M, N):
    """The combine of the partition roots on odd, aligned and tiny M N gives the P = 1 bits,
    FP32 and bf16 (the P = 8 workspace of these shapes included)."""
    K, L = 2048, 8
    A = normal_bf16(M + 31, (M, K), 1.0)
    Wt = normal_bf16(N + 32, (N, K), 0.02)
    note(f"partition combine shapes M={M} N={N}")
    base = u32(_run(A, Wt, L, 1))
    for P in (2, 4, 8):
        assert np.array_equal(u32(_run(A, Wt, L, P)), base), P
        bf = _run(A, Wt, L, P, iso.BF16)
        assert np.array_equal(bf, f32_to_bf16_bits(base.view(np.float32))), P


@pytest.mark.parametrize("K,L,N", [(256, 4, 300), (512, 4, 128), (2048, 8, 2048), (1024, 8, 77),
                                   (4096, 16, 4096), (2048, 32, 130), (4096, 64, 96),
                                   (4096, 8, 256), (4096, 4, 256), (1024, 2, 200)])
def test_few_rows_match_batch(K, L, N):
    """Up to 256 rows may take the weight-streaming kernel (one workgroup per 16 output
    columns, eight subtrees of leaves per column block, row groups of 16 double-buffered), or,
    with a workspace on a shape of few 128 x 128 tiles, the tile kernel split into up to 8
    partitions of whole subtrees; the same rows inside a batch of 600 take the tile kernel.
    Same bits for every plan, FP32 and bf16, ragged N; 4 leaves of 1024 and 2 leaves are
    shapes the weight-streaming kernel leaves to the tile kernels."""
    t = torch()
    A = normal_bf16(K + N, (600, K), 1.0)
    Wt = normal_bf16(K + N + 1, (N, K), 0.02)
    note(f"few rows vs batch K={K} L={L} N={N}")
    big = u32(_run(A, Wt, L))
    bigb = _run(A, Wt, L, 1, iso.BF16)
    c = iso.contract(L, K // L, 0)
    dW = dev(Wt)
    for m in (1, 5, 16, 17, 32, 33, 48, 64, 65, 96, 130, 256):
        for start in (0, 150):
            a = dev(A[start:start + m])
            assert np.array_equal(u32(_run(A[start:start + m], Wt, L)), big[start:start + m]), (m, start)
            assert np.array_equal(_run(A[start:start + m], Wt, L, 1, iso.BF16),
                                  bigb[start:start + m]), (m, start)
            # without a workspace (no split plan) the bits are the same
            o = t.empty((m, N), dtype=t.float32, device="cuda")
            st = iso.lib.iso_gemm(ctypes.byref(c), a.data_ptr(), dW.data_ptr(), o.data_ptr(), iso.F32,
                                  m, N, K, 1, None, 0, t.cuda.current_stream().cuda_stream)
            if st == 6:  # more than 16 leaves outside the weight-streaming kernel need one
                assert L > 16, (m, start)
                continue
            assert st == 0, (m, start, st)
            t.cuda.synchronize()
            assert np.array_equal(u32(host(o)), big[start:start + m]), (m, start, "no workspace")
    check_gemm_tol(big[:16].view(np.float32), oracle.gemm(A[:16], Wt, L), absdot(A[:16], Wt),
                   f"few rows {K}/{L}")


@pytest.mark.parametrize("K,L,M,N", [(4096, 16, 64, 4096), (4096, 16, 33, 130), (2048, 8, 128, 2048),
                                     (4096, 64, 40, 1000), (1024, 4, 100, 203), (2048, 8, 72, 1024),
                                     (2048, 8, 72, 1022)])
def test_split_workspace_contents_and_graph_replays(K, L, M, N):
    """A one-partition call on few output tiles with a workspace splits K into partitions of
    whole subtrees (roots in the workspace, then the fold).  Its bits equal the rows' bits in a
    batch of 600 whatever the workspace held before (random bytes, all ones, the previous
    call's roots), for FP32 and for bf16 at an odd element offset of the output, and across
    graph replays with eager calls on the same workspace in between.  The fold runs tile by tile
    (2048 x 2048, 2048 x 1024: at most 16 MiB of weights on a multiple of 8 tiles) or in element
    order (the rest; N = 1022 is not a multiple of 4, and a bf16 output at an odd offset is not
    8-byte aligned)."""
    t = torch()
    A = normal_bf16(K + M, (600, K), 1.0)
    Wt = normal_bf16(K + N + 7, (N, K), 0.02)
    note(f"split workspace contents K={K} L={L} M={M} N={N}")
    big = u32(_run(A, Wt, L))
    want = big[100:100 + M]
    wantb = f32_to_bf16_bits(want.view(np.float32))
    c = iso.contract(L, K // L, 0)
    a, dW = dev(A[100:100 + M]), dev(Wt)
    need = iso.gemm_workspace(c, M, N, 1)
    assert need > 0  # these shapes take the split
    ws = t.randint(0, 256, (need,), dtype=t.uint8, device="cuda")
    o = t.empty((M, N), dtype=t.float32, device="cuda")
    ob = t.empty((M * N + 1,), dtype=t.bfloat16, device="cuda")
    st = t.cuda.current_stream().cuda_stream

    def call(out, dtype, stream=st):
        return iso.lib.iso_gemm(ctypes.byref(c), a.data_ptr(), dW.data_ptr(), out, dtype, M, N, K,
                                1, ws.data_ptr(), need, stream)

    for fill in ("random", "again", "ones", "again"):
        if fill == "ones":
            ws.fill_(255)
        o.fill_(float("nan"))
        assert call(o.data_ptr(), iso.F32) == 0
        t.cuda.synchronize()
        assert np.array_equal(u32(host(o)), want), fill
        assert call(ob.data_ptr() + 2, iso.BF16) == 0
        t.cuda.synchronize()
        assert np.array_equal(host(ob)[1:].view(np.uint16).reshape(M, N), wantb), fill

    g = t.cuda.CUDAGraph()
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):
        with t.cuda.graph(g, stream=s):
            assert call(o.data_ptr(), iso.F32, stream=s.cuda_stream) == 0
    t.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        o.fill_(float("nan"))
        g.replay()
        t.cuda.synchronize()
        assert np.array_equal(u32(host(o)), want), ("replay", rep)
        assert call(ob.data_ptr() + 2, iso.BF16) == 0  # an eager call in between
        t.cuda.synchronize()
        assert np.array_equal(host(ob)[1:].view(np.uint16).reshape(M, N), wantb), ("eager", rep)
