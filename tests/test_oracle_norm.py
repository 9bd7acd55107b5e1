"""Pins of the oracle's RMSNorm: the sum-of-squares tree order, the residual
add rounding and closed-form rows (tests/golden/rmsnorm_pins.txt, derived by
hand), plus a float64 brute force on random rows within the FP32 error
bound of the evaluation order."""
import numpy as np
import pytest

import oracle
from iso_synth import bf16_bits_to_f32, normal_bf16
from pins import rmsnorm_pins

PINS = rmsnorm_pins()
ONE = 0x3F80


@pytest.mark.parametrize("pin", PINS["ss"], ids=lambda p: f"H{p['H']}L{p['L']}")
def test_sum_of_squares_follows_the_leaf_tree(pin):
    x = np.zeros((1, pin["H"]), dtype=np.uint16)
    x[0, :len(pin["h"])] = pin["h"]
    w = np.full(pin["H"], ONE, dtype=np.uint16)
    _, h, ss = oracle.rmsnorm(x, w, pin["L"], 0.0)
    assert np.array_equal(h, x)  # no residual: h is x
    assert int(ss.view(np.uint32)[0]) == pin["expected"]


@pytest.mark.parametrize("pin", PINS["add"], ids=lambda p: f"{p['x']:04x}+{p['r']:04x}")
def test_residual_add_rounds_to_bf16(pin):
    H = 8
    x = np.full((1, H), pin["x"], dtype=np.uint16)
    r = np.full((1, H), pin["r"], dtype=np.uint16)
    w = np.full(H, ONE, dtype=np.uint16)
    _, h, _ = oracle.rmsnorm(x, w, 8, 1e-6, residual=r)
    assert np.all(h == pin["h"])


@pytest.mark.parametrize("pin", PINS["y"], ids=lambda p: f"H{p['H']}L{p['L']}h{p['h']:04x}")
def test_closed_form_rows(pin):
    x = np.full((3, pin["H"]), pin["h"], dtype=np.uint16)
    w = np.full(pin["H"], pin["w"], dtype=np.uint16)
    y, _, _ = oracle.rmsnorm(x, w, pin["L"], pin["eps"], out_bf16=True)
    assert np.all(y == pin["y_bf16"])
    yf, _, _ = oracle.rmsnorm(x, w, pin["L"], pin["eps"], out_bf16=False)
    assert np.all(yf.view(np.uint32) == pin["y_f32"])


@pytest.mark.parametrize("pin", PINS["row"], ids=lambda p: f"H{p['H']}L{p['L']}")
def test_hand_worked_rows(pin):
    """FP32 outputs of hand-derived rows: fixes where eps sits and the
    association (h * r) * w of the last step."""
    x = np.array([pin["h"]], dtype=np.uint16)
    w = np.array(pin["w"], dtype=np.uint16)
    yf, _, _ = oracle.rmsnorm(x, w, pin["L"], pin["eps"], out_bf16=False)
    assert np.array_equal(yf.view(np.uint32)[0], np.array(pin["y_f32"], dtype=np.uint32))


@pytest.mark.parametrize("H,L,eps", [(2048, 64, 1e-6), (2048, 1, 1e-6), (2048, 2048, 1e-6),
                                     (512, 16, 0.25), (4096, 256, 1e-6), (256, 32, 3.0)])
def test_against_float64_definition(H, L, eps):
    # a large eps makes its place in the formula visible (under the root)
    M = 32
    x = normal_bf16(11, (M, H), 1.0)
    r = normal_bf16(12, (M, H), 0.5)
    w = normal_bf16(13, (H,), 1.0)
    y, h, ss = oracle.rmsnorm(x, w, L, eps, residual=r, out_bf16=False)
    # h: the bf16 rounding of the exact sum
    hx = bf16_bits_to_f32(x).astype(np.float64) + bf16_bits_to_f32(r).astype(np.float64)
    hf = bf16_bits_to_f32(h).astype(np.float64)
    assert np.all(np.abs(hf - hx) <= np.abs(hx) * 2.0 ** -8 + 1e-300)
    # sum of squares: FP32 error bound of L sequential leaves of m plus log2(L) levels
    m = H // L
    ss64 = (hf * hf).sum(axis=1)
    bound = (m + np.log2(L) + 1) * 2.0 ** -24 * ss64
    assert np.all(np.abs(ss.astype(np.float64) - ss64) <= bound)
    # y against the float64 formula on the same h: a few FP32 roundings after ss
    y64 = hf / np.sqrt(ss64 / H + eps)[:, None] * bf16_bits_to_f32(w).astype(np.float64)
    rel = (m + np.log2(L) + 8) * 2.0 ** -24
    assert np.all(np.abs(y - y64) <= rel * np.abs(y64) + 1e-30)


def test_rows_are_independent():
    H = 1024
    x = normal_bf16(21, (64, H), 1.0)
    w = normal_bf16(22, (H,), 1.0)
    y, _, _ = oracle.rmsnorm(x, w, 64, 1e-5)
    for i in (0, 17, 63):
        yi, _, _ = oracle.rmsnorm(x[i:i + 1], w, 64, 1e-5)
        assert np.array_equal(yi[0], y[i])


def test_bad_arguments():
    x = np.zeros((2, 64), dtype=np.uint16)
    w = np.zeros(64, dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.rmsnorm(x, w, 3, 1e-6)    # not a power of two
    with pytest.raises(ValueError):
        oracle.rmsnorm(x, w, 128, 1e-6)  # more leaves than elements
