"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU oracle.

This module holds no arithmetic of the method itself: it only draws random
numbers (numpy PCG64) and stores them as the bit patterns the library consumes.

* bf16 tensors are raw ``uint16`` bit patterns.  A draw is made in float64,
  scaled by sigma, cast to float32 and rounded to bf16 with round-to-nearest-
  even on the float32 bit pattern (finite values only).
* Weight matrices are returned in the library's storage order: for a matrix
  W of shape [K x N] (K = contraction), the stored array is W^T, shaped
  [N][K], so every output column's K weights are contiguous (the storage of a
  linear layer's ``out_features x in_features`` weight).  Drawing order is the
  stored order, so the seed fixes the stored bits.
* Large tensors are drawn in row blocks to bound host memory; the stream of
  random numbers is identical to one big draw.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "normal_bf16",
    "uniform_tokens",
    "normal_f32",
    "CONFIGS",
    "make_config",
    "unit_rows_bf16",
    "uniform_f32",
    "cpr_inputs",
]

_BLOCK = 1 << 24  # elements per draw block


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even) and return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(seed: int, shape, sigma: float) -> np.ndarray:
    """N(0, sigma^2) samples rounded to bf16, as uint16 bits of the given shape."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    rng = np.random.default_rng(seed)
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _BLOCK):
        e = min(n, s + _BLOCK)
        x = (rng.standard_normal(e - s) * sigma).astype(np.float32)
        out[s:e] = f32_to_bf16_bits(x)
    return out.reshape(shape)


def normal_f32(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    """N(0, sigma^2) float32 samples (router logits)."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(tuple(shape)) * sigma).astype(np.float32)


def uniform_tokens(seed: int, m: int, v: int) -> np.ndarray:
    """m token ids drawn uniformly from {0, ..., v-1}, as int32."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, v, size=int(m)).astype(np.int32)


# Workload recipes (shapes, distributions, leaf structure, seeds).  Weight
# shapes are the stored [N][K] arrays described above.
CONFIGS = {
    "tiny": dict(M=8, K=256, N=512, leaves=4, sigma_a=1.0, sigma_w=0.05,
                 seeds=(101, 102, 103)),
    "prefill": dict(M=4096, K=2048, N=2048, leaves=8, sigma_a=1.0, sigma_w=0.02,
                    seeds=(201, 202)),
    "lmhead": dict(M=8192, K=2048, V=151936, leaves=8, sigma_a=1.0, sigma_w=0.02,
                   seeds=(301, 302, 303)),
    "sweep": dict(K=4096, N=4096, leaves=16, sigma_a=1.0, sigma_w=0.02, probes=64,
                  seeds=(401, 402, 403, 404)),
    "moe": dict(T=4096, H=2048, E=128, I=512, top_k=8, leaves_gate_up=4, leaves_down=4,
                sigma_x=1.0, sigma_w=0.02, seeds=(501, 502, 503, 504, 505, 506)),
}


def make_config(name: str, rows: int | None = None) -> dict:
    """Arrays for one workload.  ``rows`` truncates the activation rows (the
    weights are unchanged), which keeps the same seeded bits for the rows kept."""
    c = CONFIGS[name]
    out = dict(c)
    if name in ("tiny", "prefill"):
        s_a, s_w = c["seeds"][0], c["seeds"][1]
        M = c["M"] if rows is None else rows
        a = normal_bf16(s_a, (c["M"], c["K"]), c["sigma_a"])[:M]
        out.update(A=np.ascontiguousarray(a), Wt=normal_bf16(s_w, (c["N"], c["K"]), c["sigma_w"]), M=M)
        if name == "tiny":
            out["tok"] = uniform_tokens(c["seeds"][2], c["M"], c["N"])[:M]
        return out
    if name == "lmhead":
        M = c["M"] if rows is None else rows
        a = normal_bf16(c["seeds"][0], (c["M"], c["K"]), c["sigma_a"])[:M]
        out.update(H=np.ascontiguousarray(a),
                   Wvt=normal_bf16(c["seeds"][1], (c["V"], c["K"]), c["sigma_w"]),
                   tok=uniform_tokens(c["seeds"][2], c["M"], c["V"])[:M], M=M)
        return out
    if name == "sweep":
        out.update(Wt=normal_bf16(c["seeds"][0], (c["N"], c["K"]), c["sigma_w"]),
                   probe_rows=normal_bf16(c["seeds"][1], (c["probes"], c["K"]), c["sigma_a"]),
                   filler=normal_bf16(c["seeds"][2], (4096, c["K"]), c["sigma_a"]),
                   placement_seed=c["seeds"][3])
        return out
    if name == "moe":
        T = c["T"] if rows is None else rows
        s = c["seeds"]
        x = normal_bf16(s[0], (c["T"], c["H"]), c["sigma_x"])[:T]
        lg = normal_f32(s[1], (c["T"], c["E"]), 1.0)[:T]
        out.update(X=np.ascontiguousarray(x), logits=np.ascontiguousarray(lg), T=T,
                   Wg=normal_bf16(s[2], (c["E"], c["I"], c["H"]), c["sigma_w"]),
                   Wu=normal_bf16(s[3], (c["E"], c["I"], c["H"]), c["sigma_w"]),
                   Wd=normal_bf16(s[4], (c["E"], c["H"], c["I"]), c["sigma_w"]),
                   ordering_seed=s[5])
        return out
    raise KeyError(name)


def unit_rows_bf16(seed: int, shape) -> np.ndarray:
    """N(0, 1) draws, each last-axis row scaled to unit L2 norm in float64,
    then rounded to bf16 (the normalised query/key rows a linear-attention
    layer feeds its recurrence)."""
    shape = tuple(int(s) for s in shape)
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape)
    x = x / np.linalg.norm(x, axis=-1, keepdims=True)
    return f32_to_bf16_bits(x.astype(np.float32))


def uniform_f32(seed: int, shape, lo: float, hi: float) -> np.ndarray:
    """U[lo, hi) float32 samples."""
    rng = np.random.default_rng(seed)
    return rng.uniform(lo, hi, size=tuple(int(s) for s in shape)).astype(np.float32)


def cpr_inputs(T: int, H: int, d: int, seed: int = 601) -> dict:
    """One gated-delta-rule layer's per-token inputs for T tokens and H heads of
    size d: q, k unit rows [T][H][d] (bf16 bits), v ~ N(0, 1) [T][H][d] (bf16
    bits), decay gate alpha ~ U[0.9, 1) and write strength beta ~ U[0, 1)
    [T][H] float32.  Seeds seed .. seed + 4."""
    return {
        "q": unit_rows_bf16(seed, (T, H, d)),
        "k": unit_rows_bf16(seed + 1, (T, H, d)),
        "v": normal_bf16(seed + 2, (T, H, d), 1.0),
        "alpha": uniform_f32(seed + 3, (T, H), 0.9, 1.0),
        "beta": uniform_f32(seed + 4, (T, H), 0.0, 1.0),
    }
