"""CPU oracle for the invariant numerics path -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  The product library never does: the two share
no code, and meet only in the seeded input bit patterns of ``iso_synth``.

The arithmetic lives in ``iso_oracle.c`` (plain C, one loop per definition);
this module builds it with gcc and wraps it with ctypes.  Every function
returns numpy arrays and raises ``ValueError`` when the C side rejects its
arguments.  Citations for each computation are in the C file's header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "iso_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
          "-std=c11", "-Wall", "-Wextra"]

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle into ``oracle/liboracle.so`` with gcc."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(out_path: str) -> str:
    """The oracle under AddressSanitizer and UndefinedBehaviorSanitizer
    (same arithmetic flags), for the CPU sanitizer run of the tests."""
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-g"]
    flags = [f for f in CFLAGS if f != "-O2"] + ["-O1"]
    subprocess.run(["gcc", *flags, *san, _SRC, "-o", out_path, "-lm"], check=True)
    return out_path


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        sigs = {
            "oracle_threads": ([], I),
            "oracle_set_threads": ([I], I),
            "oracle_gemm": ([P, P, I64, I64, I64, I, P], I),
            "oracle_gemm_elems": ([P, P, I64, I, P, P, I64, P], I),
            "oracle_gemm_partitioned": ([P, P, I64, I64, I64, I, I, P], I),
            "oracle_lmhead_logprob": ([P, P, P, I64, I64, I64, I, P, P, P], I),
            "oracle_moe_route": ([P, I64, I64, I, P, P], I),
            "oracle_moe_gate_up": ([P, P, P, P, I64, I64, I64, I64, I, I, P, P], I),
            "oracle_moe_down": ([P, P, P, I64, I64, I64, I64, I, I, P], I),
            "oracle_moe_combine": ([P, P, I64, I64, I, P], I),
            "oracle_rmsnorm": ([P, P, P, I64, I64, I, ctypes.c_float, I, P, P, P], I),
            "oracle_cpr_prefill": ([P, P, P, P, P, P, I64, I64, I, I, P, P, P, P], I),
            "oracle_cpr_decode_step": ([P, P, P, P, P, I64, I64, I, I, P, P, P], I),
            "oracle_cpr_transition": ([P, P, P, P, I, I, P, P], I),
        }
        for name, (args, res) in sigs.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 inputs are uint16 bit patterns")
    return a


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle rejected arguments of {what}")


def threads() -> int:
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    """Threads of the following calls (they split independent outputs only,
    so no result changes)."""
    _check(_load().oracle_set_threads(int(n)), "set_threads")


def gemm(A, Wt, leaves: int) -> np.ndarray:
    """FP32 C [M][N] of A [M][K] times the matrix stored as Wt [N][K]."""
    A, Wt = _u16(A), _u16(Wt)
    M, K = A.shape
    N = Wt.shape[0]
    if Wt.shape[1] != K:
        raise ValueError("K mismatch")
    C = np.empty((M, N), dtype=np.float32)
    _check(_load().oracle_gemm(_p(A), _p(Wt), M, N, K, leaves, _p(C)), "gemm")
    return C


def gemm_elems(A, Wt, leaves: int, rows, cols) -> np.ndarray:
    A, Wt = _u16(A), _u16(Wt)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows/cols shape mismatch")
    if rows.size and (rows.min() < 0 or rows.max() >= A.shape[0] or cols.min() < 0
                      or cols.max() >= Wt.shape[0]):
        raise ValueError("element index out of range")
    out = np.empty(rows.shape, dtype=np.float32)
    _check(_load().oracle_gemm_elems(_p(A), _p(Wt), A.shape[1], leaves, _p(rows), _p(cols),
                                     rows.size, _p(out)), "gemm_elems")
    return out


def gemm_partitioned(A, Wt, leaves: int, partitions: int) -> np.ndarray:
    A, Wt = _u16(A), _u16(Wt)
    M, K = A.shape
    N = Wt.shape[0]
    C = np.empty((M, N), dtype=np.float32)
    _check(_load().oracle_gemm_partitioned(_p(A), _p(Wt), M, N, K, leaves, partitions, _p(C)),
           "gemm_partitioned")
    return C


def lmhead_logprob(H, Wvt, tok, leaves: int):
    """Returns (logprob float64 [M], target logit float32 [M], logsumexp float64 [M])."""
    H, Wvt = _u16(H), _u16(Wvt)
    tok = np.ascontiguousarray(tok, dtype=np.int32)
    M, K = H.shape
    V = Wvt.shape[0]
    lp = np.empty(M, dtype=np.float64)
    zt = np.empty(M, dtype=np.float32)
    lse = np.empty(M, dtype=np.float64)
    _check(_load().oracle_lmhead_logprob(_p(H), _p(Wvt), _p(tok), M, V, K, leaves, _p(lp),
                                         _p(zt), _p(lse)), "lmhead_logprob")
    return lp, zt, lse


def moe_route(logits, top_k: int):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    idx = np.empty((T, top_k), dtype=np.int32)
    gate = np.empty((T, top_k), dtype=np.float64)
    _check(_load().oracle_moe_route(_p(logits), T, E, top_k, _p(idx), _p(gate)), "moe_route")
    return idx, gate


def moe_gate_up(X, Wg, Wu, idx, leaves: int):
    """Returns (act float32 [T][k][I], h bf16 bits [T][k][I])."""
    X, Wg, Wu = _u16(X), _u16(Wg), _u16(Wu)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, Hd = X.shape
    E, I, _ = Wg.shape
    k = idx.shape[1]
    act = np.empty((T, k, I), dtype=np.float32)
    h = np.empty((T, k, I), dtype=np.uint16)
    _check(_load().oracle_moe_gate_up(_p(X), _p(Wg), _p(Wu), _p(idx), T, Hd, E, I, k, leaves,
                                      _p(act), _p(h)), "moe_gate_up")
    return act, h


def moe_down(h, Wd, idx, leaves: int):
    h, Wd = _u16(h), _u16(Wd)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k, I = h.shape
    E, Hd, _ = Wd.shape
    e = np.empty((T, k, Hd), dtype=np.float32)
    _check(_load().oracle_moe_down(_p(h), _p(Wd), _p(idx), T, Hd, E, I, k, leaves, _p(e)),
           "moe_down")
    return e


def moe_combine(gate, e):
    gate = np.ascontiguousarray(gate, dtype=np.float64)
    e = np.ascontiguousarray(e, dtype=np.float32)
    T, k, Hd = e.shape
    y = np.empty((T, Hd), dtype=np.float64)
    _check(_load().oracle_moe_combine(_p(gate), _p(e), T, Hd, k, _p(y)), "moe_combine")
    return y


def moe(X, logits, Wg, Wu, Wd, top_k: int, leaves_gate_up: int, leaves_down: int):
    """Whole MoE FFN block; returns a dict with every stage's output."""
    idx, gate = moe_route(logits, top_k)
    act, h = moe_gate_up(X, Wg, Wu, idx, leaves_gate_up)
    e = moe_down(h, Wd, idx, leaves_down)
    y = moe_combine(gate, e)
    return dict(idx=idx, gate=gate, act=act, h=h, e=e, y=y)


def rmsnorm(x, w, leaves: int, eps: float, residual=None, out_bf16: bool = True):
    """RMSNorm of x [M][H] (bf16 bits) with weight w [H]: returns (y, h, ss)
    with y as bf16 bits (out_bf16) or float32, h = bf16(x + residual) bits
    (x itself without a residual) and the per-row FP32 sum of squares."""
    x, w = _u16(x), _u16(w)
    M, H = x.shape
    if w.shape != (H,):
        raise ValueError("w must be [H]")
    r = None if residual is None else _u16(residual)
    if r is not None and r.shape != (M, H):
        raise ValueError("residual must be [M][H]")
    h = np.empty((M, H), dtype=np.uint16)
    y = np.empty((M, H), dtype=np.uint16 if out_bf16 else np.float32)
    ss = np.empty(M, dtype=np.float32)
    _check(_load().oracle_rmsnorm(_p(x), _p(r), _p(w), M, H, leaves, float(eps),
                                  1 if out_bf16 else 0, _p(h), _p(y), _p(ss)), "rmsnorm")
    return y, h, ss


def _f32(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.float32:
        raise TypeError("expected float32")
    return a


def _cpr_inputs(q, k, v, alpha, beta):
    q, k, v = _u16(q), _u16(k), _u16(v)
    alpha, beta = _f32(alpha), _f32(beta)
    if q.ndim != 3 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must be [T][H][d]")
    T, H, d = q.shape
    if alpha.shape != (T, H) or beta.shape != (T, H):
        raise ValueError("alpha, beta must be [T][H]")
    return q, k, v, alpha, beta, T, H, d


def cpr_prefill(q, k, v, alpha, beta, chunk: int, S0=None, bounds: bool = False):
    """CPR Gated DeltaNet prefill of q, k, v [T][H][d] (bf16 bits), alpha,
    beta [T][H] float32, from boundary state S0 [H][d][d] (zeros if None).
    Returns (o [T][H][d], snap [H][d][d], run [H][d][d]) and, with
    bounds=True, every boundary state [T//chunk + 1][H][d][d] as well."""
    q, k, v, alpha, beta, T, H, d = _cpr_inputs(q, k, v, alpha, beta)
    if S0 is not None:
        S0 = _f32(S0)
        if S0.shape != (H, d, d):
            raise ValueError("S0 must be [H][d][d]")
    o = np.empty((T, H, d), np.float32)
    snap = np.empty((H, d, d), np.float32)
    run = np.empty((H, d, d), np.float32)
    bnd = np.empty((T // chunk + 1, H, d, d), np.float32) if bounds else None
    _check(_load().oracle_cpr_prefill(_p(q), _p(k), _p(v), _p(alpha), _p(beta), _p(S0), T, H, d,
                                      chunk, _p(o), _p(snap), _p(run), _p(bnd)), "cpr_prefill")
    return (o, snap, run, bnd) if bounds else (o, snap, run)


def cpr_decode_step(q, k, v, alpha, beta, chunk: int, pos: int, snap, run):
    """One CPR decode step for token `pos` of the [T][H][d] history arrays;
    returns (o [H][d], snap, run) with the states updated (copies)."""
    q, k, v, alpha, beta, T, H, d = _cpr_inputs(q, k, v, alpha, beta)
    if not 0 <= pos < T:
        raise ValueError("pos outside the history")
    snap = _f32(snap).copy()
    run = _f32(run).copy()
    o = np.empty((H, d), np.float32)
    _check(_load().oracle_cpr_decode_step(_p(q), _p(k), _p(v), _p(alpha), _p(beta), pos, H, d,
                                          chunk, _p(snap), _p(run), _p(o)), "cpr_decode_step")
    return o, snap, run


def cpr_transition(k, v, alpha, beta):
    """Chunk form (P, U) [d][d] of n tokens of one head: k, v [n][d] bf16
    bits, alpha, beta [n] float32."""
    k, v = _u16(k), _u16(v)
    alpha, beta = _f32(alpha), _f32(beta)
    n, d = k.shape
    P = np.empty((d, d), np.float32)
    U = np.empty((d, d), np.float32)
    _check(_load().oracle_cpr_transition(_p(k), _p(v), _p(alpha), _p(beta), n, d, _p(P), _p(U)),
           "cpr_transition")
    return P, U
