"""GPU parity of iso_rmsnorm with the oracle, bit for bit (every step is a
correctly rounded FP32 operation in the contract's order), over leaf shapes,
ragged batches, with and without the residual add, in place, FP32 and bf16
outputs, the hand-derived tree pins, each row's bits across batch size and
row position, and the normalization in front of the LM-head at full size
(8192 rows x 2048 hidden)."""
import numpy as np
import pytest

import oracle
from gpu_util import dev, host, note, torch
from iso_synth import normal_bf16
from pins import rmsnorm_pins

pytestmark = pytest.mark.gpu

iso = pytest.importorskip("parallelism_invariant_numerics_amd")


def _gpu(x, w, L, eps, residual=None, out_bf16=True, in_place=False):
    t = torch()
    H = x.shape[1]
    c = iso.contract(L, H // L, 0, iso.SCHED_SEQ)
    dx = dev(x)
    dr = None if residual is None else dev(residual)
    dro = dr if in_place else (None if residual is None else t.empty_like(dr))
    y = iso.rmsnorm(dx, dev(w), c, residual=dr, residual_out=dro, eps=eps,
                    out_dtype=iso.BF16 if out_bf16 else iso.F32)
    t.cuda.synchronize()
    return host(y), (None if dro is None else host(dro))


def _check(x, w, L, eps, residual=None, out_bf16=True, in_place=False):
    y, h = _gpu(x, w, L, eps, residual, out_bf16, in_place)
    ye, he, _ = oracle.rmsnorm(x, w, L, eps, residual=residual, out_bf16=out_bf16)
    if out_bf16:
        assert np.array_equal(y, ye)
    else:
        assert np.array_equal(y.view(np.uint32), ye.view(np.uint32))
    if residual is not None:
        assert np.array_equal(h, he)


# (M, H, L): one leaf per lane; fewer leaves than lanes; 2, 4 and 8 leaves per
# lane; the smallest and largest lane spans
SHAPES = [(8, 2048, 64), (1000, 2048, 64), (3, 2048, 16), (5, 2048, 128), (7, 2048, 256),
          (9, 2048, 512), (11, 512, 64), (4, 8192, 64), (6, 1024, 8), (2, 64, 8)]


@pytest.mark.parametrize("M,H,L", SHAPES)
@pytest.mark.parametrize("residual", [False, True])
def test_bitwise_parity(M, H, L, residual):
    note(f"rmsnorm M={M} H={H} L={L} residual={residual}")
    x = normal_bf16(31, (M, H), 1.0)
    r = normal_bf16(32, (M, H), 0.5) if residual else None
    w = normal_bf16(33, (H,), 1.0)
    _check(x, w, L, 1e-6, residual=r)
    _check(x, w, L, 0.25, residual=r, out_bf16=False)


def test_in_place_residual():
    x = normal_bf16(41, (64, 2048), 1.0)
    r = normal_bf16(42, (64, 2048), 1.0)
    w = normal_bf16(43, (2048,), 1.0)
    _check(x, w, 64, 1e-6, residual=r, in_place=True)


def test_tree_order_pins_on_gpu():
    # the golden sum-of-squares rows placed one value per leaf of 8 in a
    # 512-element row (64 leaves): the GPU must follow the balanced tree
    pins = [p for p in rmsnorm_pins()["ss"] if p["L"] == 4]
    w = np.full(512, 0x3F80, dtype=np.uint16)
    for p in pins:
        x = np.zeros((1, 512), dtype=np.uint16)
        for i, v in enumerate(p["h"]):
            x[0, 8 * i] = v
        _, _, ss = oracle.rmsnorm(x, w, 64, 0.0)
        assert int(ss.view(np.uint32)[0]) == p["expected"]
        _check(x, w, 64, 0.0, out_bf16=False)


def test_closed_form_rows_on_gpu():
    for p in rmsnorm_pins()["y"]:
        H, L = p["H"], p["L"]
        if H < 64 or H // min(L, 64) < 8:
            continue  # the kernel's lane span starts at 8 elements
        x = np.full((3, H), p["h"], dtype=np.uint16)
        w = np.full(H, p["w"], dtype=np.uint16)
        y, _ = _gpu(x, w, L, p["eps"])
        assert np.all(y == p["y_bf16"])


def test_row_bits_do_not_depend_on_the_batch():
    H = 2048
    probe = normal_bf16(51, (16, H), 1.0)
    rprobe = normal_bf16(52, (16, H), 1.0)
    w = normal_bf16(53, (H,), 1.0)
    ref, href = _gpu(probe[:1], w, 64, 1e-6, residual=rprobe[:1])
    for M in (1, 8, 64, 4096):
        x = normal_bf16(54 + M, (M, H), 1.0)
        r = normal_bf16(55 + M, (M, H), 1.0)
        for pos in {0, M // 2, M - 1}:
            x[pos] = probe[0]
            r[pos] = rprobe[0]
            y, h = _gpu(x, w, 64, 1e-6, residual=r)
            assert np.array_equal(y[pos], ref[0]) and np.array_equal(h[pos], href[0])


def test_full_size_in_front_of_the_lmhead():
    # the LM-head workload's hidden states: 8192 rows x 2048, residual add
    M, H = 8192, 2048
    note("rmsnorm full size 8192 x 2048")
    x = normal_bf16(61, (M, H), 1.0)
    r = normal_bf16(62, (M, H), 1.0)
    w = normal_bf16(63, (H,), 1.0)
    _check(x, w, 64, 1e-6, residual=r)


def test_empty_batch():
    t = torch()
    c = iso.contract(64, 32, 0, iso.SCHED_SEQ)
    x = t.empty((0, 2048), dtype=t.bfloat16, device="cuda")
    w = t.ones(2048, dtype=t.bfloat16, device="cuda")
    y = iso.rmsnorm(x, w, c)
    assert y.shape == (0, 2048)
