"""Readers for the golden pin files and builders of the exact-input cases.

These helpers only parse text and place values into input arrays; they hold
none of the method's arithmetic.
"""
from __future__ import annotations

import os

import numpy as np

from iso_synth import f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _value(tok: str) -> float:
    tok = tok.strip()
    neg = tok.startswith("-")
    if neg:
        tok = tok[1:]
    if tok.startswith("2^"):
        v = 2.0 ** int(tok[2:])
    else:
        v = float(int(tok))
    return -v if neg else v


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield [c.strip() for c in line.split("|")]


def tree_pins():
    """Rows of tree_order_pins.txt as dicts."""
    out = []
    for kind, leaves, vals, bal, seq, other in _lines("tree_order_pins.txt"):
        name, bits = other.split("=")
        out.append(dict(kind=kind, leaves=int(leaves), values=[_value(v) for v in vals.split()],
                        balanced=int(bal, 16), sequential=int(seq, 16),
                        other_name=name, other=int(bits, 16)))
    return out


def logsoftmax_forms():
    return [dict(V=int(v), case=c, expected=float(e))
            for v, c, e in _lines("logsoftmax_closed_forms.txt")]


def product_factors(v: float):
    """Two bf16-exact factors whose product is exactly v (v in {0, +-1, +-2^-2j})."""
    if v == 0.0:
        return 0.0, 0.0
    mant, exp = np.frexp(abs(v))  # v = mant * 2^exp, mant = 0.5 for powers of two
    assert mant == 0.5, "pins use powers of two"
    e = int(exp) - 1
    assert e % 2 == 0
    return float(np.copysign(2.0 ** (e // 2), v)), 2.0 ** (e // 2)


def tree_case_inputs(pin, leaf_size: int, rows: int = 1, cols: int = 1, kind=None):
    """A [rows][K] and Wt [cols][K] bf16 bits such that every output element
    has, for a "tree" pin, exactly one product per leaf equal to the pin's leaf
    value; for an "inleaf" pin, the values sit in consecutive k of leaf 0."""
    kind = kind or pin["kind"]
    L = pin["leaves"]
    K = L * leaf_size
    a = np.zeros(K, dtype=np.float32)
    w = np.zeros(K, dtype=np.float32)
    for i, v in enumerate(pin["values"]):
        k = i * leaf_size + (i * 7) % leaf_size if kind == "tree" else i
        fa, fw = product_factors(v)
        a[k], w[k] = fa, fw
    A = np.tile(f32_to_bf16_bits(a), (rows, 1))
    Wt = np.tile(f32_to_bf16_bits(w), (cols, 1))
    return A, Wt


def f32_bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def rmsnorm_pins():
    """Rows of rmsnorm_pins.txt grouped by kind."""
    out = {"ss": [], "add": [], "y": [], "row": []}
    for row in _lines("rmsnorm_pins.txt"):
        kind = row[0]
        if kind == "ss":
            out["ss"].append(dict(H=int(row[1]), L=int(row[2]),
                                  h=[int(v, 16) for v in row[3].split()],
                                  expected=int(row[4], 16)))
        elif kind == "add":
            out["add"].append(dict(x=int(row[1], 16), r=int(row[2], 16), h=int(row[3], 16)))
        elif kind == "y":
            out["y"].append(dict(H=int(row[1]), L=int(row[2]), h=int(row[3], 16),
                                 w=int(row[4], 16), eps=float(row[5]),
                                 y_bf16=int(row[6], 16), y_f32=int(row[7], 16)))
        elif kind == "row":
            out["row"].append(dict(H=int(row[1]), L=int(row[2]), eps=float(row[3]),
                                   h=[int(v, 16) for v in row[4].split()],
                                   w=[int(v, 16) for v in row[5].split()],
                                   y_f32=[int(v, 16) for v in row[6].split()]))
    return out


def cpr_pins():
    """The hand-worked CPR example of cpr_pins.txt: B0 [2][2], tokens as
    (k, v, q, alpha, beta), outputs o [3][2], the chunk form (P, U) of the
    first chunk, and the final snap / run states."""
    out = {"tok": [], "o": None}
    for row in _lines("cpr_pins.txt"):
        kind = row[0]
        nums = [[float(x) for x in f.split()] for f in row[1:]]
        if kind == "tok":
            out["tok"].append(dict(k=nums[0], v=nums[1], q=nums[2], alpha=nums[3][0], beta=nums[4][0]))
        elif kind == "o":
            out["o"] = nums
        else:
            out[kind] = nums[0]
    return out


def moe_combine_pins():
    """Rows of moe_combine_pins.txt: top_k, gates [k], expert rows [k][H], y [H]."""
    out = []
    for k, gates, rows, y in _lines("moe_combine_pins.txt"):
        e = [[float(v) for v in r.split()] for r in rows.split(";")]
        out.append(dict(top_k=int(k), gates=[float(v) for v in gates.split()], e=e,
                        y=[float(v) for v in y.split()]))
    return out
