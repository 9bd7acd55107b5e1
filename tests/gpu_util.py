"""Helpers for the GPU tests: device upload of bf16 bit patterns, bit views
and the per-element GEMM tolerance 1e-5 * sum_k |a_k b_k|."""
from __future__ import annotations

import sys

import numpy as np

from iso_synth import bf16_bits_to_f32

GEMM_RTOL = 1e-5      # |gpu - oracle| <= GEMM_RTOL * sum_k |a_k * b_k|
LOGPROB_ATOL = 1e-5   # |gpu - oracle| on a logprob


def torch():
    import torch as t
    return t


def dev(bits: np.ndarray):
    """uint16 bf16 bits -> a torch.bfloat16 device tensor with the same bits."""
    t = torch()
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return t.from_numpy(a).to("cuda").view(t.bfloat16)


def dev_i32(x: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to("cuda")


def host(t) -> np.ndarray:
    import torch as _t
    if t.dtype == _t.bfloat16:
        return t.view(_t.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def u32(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def absdot(A_bits, Wt_bits, rows=None, cols=None) -> np.ndarray:
    """sum_k |a_ik w_jk| in float64, for all (i, j) or for listed pairs."""
    a = np.abs(bf16_bits_to_f32(A_bits).astype(np.float64))
    w = np.abs(bf16_bits_to_f32(Wt_bits).astype(np.float64))
    if rows is None:
        return a @ w.T
    return np.einsum("ik,ik->i", a[rows], w[cols])


def check_gemm_tol(got, want, ad, what=""):
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    tol = GEMM_RTOL * ad
    ratio = float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0
    bad = err > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} elements over tolerance, max err/tol {ratio:.3g}"
    return ratio


def note(msg: str):
    """Name the case before a GPU step, flushed, so a crash log says where."""
    sys.stdout.write(f"[case] {msg}\n")
    sys.stdout.flush()
