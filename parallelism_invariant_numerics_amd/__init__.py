"""Python binding of libiso -- parallelism- and batch-invariant matmul and
token-logprob kernels for AMD MI355X (gfx950).

Argument marshalling only: every computation runs in the HIP kernels behind
the C ABI declared in ``include/iso.h``.  PyTorch provides device memory and
the current HIP stream.  bf16 operands are ``torch.bfloat16`` (or 16-bit
integer tensors holding bf16 bit patterns); weights are stored k-contiguous,
``Wt[N][K]`` for a K x N matrix.

If ``libiso.so`` has not been built, importing this package raises
``ImportError``; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

# PyTorch bundles its own HIP runtime (SONAME libamdhip64.so.7).  Importing it
# first makes libiso.so bind to that same runtime, so device pointers and
# streams from torch are valid in the library; loading libiso.so first would
# bring up a second runtime instance in the process.
import torch  # noqa: F401  (load order matters)

__all__ = [
    "IsoError", "Contract", "contract", "digest", "check_identity", "check_partitions",
    "gemm_workspace", "gemm", "gemm_baseline", "lmhead_workspace", "lmhead_logprob",
    "lmhead_logprob_noalloc", "LMHEAD_NOALLOC_BYTES",
    "moe_workspace", "moe_layout", "moe_combine", "moe_stages", "swiglu",
    "cpr_contract", "cpr_workspace", "cpr_prefill", "cpr_decode_step",
    "lib", "LIB_PATH", "F32", "BF16", "VOCAB_CHUNK", "version",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libiso.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python parallelism_invariant_numerics_amd/build.py` "
        "(the library has no non-HIP fallback)")

lib = ctypes.CDLL(LIB_PATH)

BF16 = 1
F32 = 2
VOCAB_CHUNK = 128
SCHED_MFMA = 1   # bf16 MFMA 16x16x32 leaves (matrix products)
SCHED_SEQ = 2    # one term at a time, ascending (RMSNorm)
SCHED_CPR = 3    # CPR gated delta rule: leaf_count = head size, leaf_size = chunk
_STATUS = {0: "ISO_OK", 1: "ISO_ERR_ARG", 2: "ISO_ERR_SHAPE", 3: "ISO_ERR_DTYPE",
           4: "ISO_ERR_CLAIM", 5: "ISO_ERR_IDENTITY", 6: "ISO_ERR_WORKSPACE",
           7: "ISO_ERR_LAUNCH", 8: "ISO_ERR_CONTRACT"}


class Contract(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in (
        "abi_version", "in_dtype", "accum_dtype", "leaf_count", "leaf_size", "tree",
        "vocab_chunk", "schedule")]

    def __repr__(self):
        return "Contract(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class IsoError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = _STATUS.get(status, str(status))
        msg = lib.iso_status_str(status).decode()
        if self.name == "ISO_ERR_LAUNCH":
            msg += ": " + lib.iso_last_launch_error().decode()
        super().__init__(f"{where}: {self.name} ({msg})")


class Sha256State(ctypes.Structure):
    _fields_ = [("h", ctypes.c_uint32 * 8), ("nbytes", ctypes.c_uint64),
                ("buf", ctypes.c_uint8 * 64), ("nbuf", ctypes.c_uint32)]


class Composition(ctypes.Structure):
    """One (region, case) composition of an execution contract."""
    _fields_ = [("region", ctypes.c_char * 32), ("case_name", ctypes.c_char * 32),
                ("policy", Contract), ("partitions", ctypes.c_uint32),
                ("claims", ctypes.c_uint32)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_U32 = ctypes.c_uint32
_CP = ctypes.POINTER(Contract)
_SIGS = {
    "iso_contract_init": ([_CP, _U32, _U32, _U32], _I),
    "iso_contract_validate": ([_CP], _I),
    "iso_contract_digest": ([_CP, ctypes.c_char_p], _I),
    "iso_contract_check": ([_CP, ctypes.c_char_p], _I),
    "iso_check_partitions": ([_CP, _I], _I),
    "iso_gemm_workspace": ([_CP, _I64, _I64, _I], ctypes.c_size_t),
    "iso_gemm": ([_CP, _P, _P, _P, _U32, _I64, _I64, _I64, _I, _P, ctypes.c_size_t, _P], _I),
    "iso_gemm_baseline": ([_P, _P, _P, _U32, _I64, _I64, _I64, _P], _I),
    "iso_lmhead_workspace": ([_CP, _I64, _I64, _I], ctypes.c_size_t),
    "iso_lmhead_logprob": ([_CP, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, ctypes.c_size_t, _P],
                           _I),
    "iso_lmhead_logprob_noalloc": ([_CP, _P, _P, _P, _P, _I64, _I64, _I64, _P], _I),
    "iso_moe_layout_of": ([_I64, _I64, _I64, _I64, _I, _P], _I),
    "iso_moe_workspace": ([_I64, _I64, _I64, _I64, _I], ctypes.c_size_t),
    "iso_moe_combine": ([_CP, _CP, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I, _P,
                         ctypes.c_size_t, _P], _I),
    "iso_rmsnorm": ([_CP, _P, _P, _P, _P, _P, _U32, _I64, _I64, ctypes.c_float, _P], _I),
    "iso_cpr_workspace": ([_CP, _I64, _I64], ctypes.c_size_t),
    "iso_cpr_prefill": ([_CP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _P, ctypes.c_size_t,
                         _P], _I),
    "iso_cpr_decode_step": ([_CP, _P, _P, _P, _P, _P, _I64, _P, _P, _P, _I64, _P,
                             ctypes.c_size_t, _P], _I),
    "iso_lmhead_shard_stats": ([_CP, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P], _I),
    "iso_lmhead_finish": ([_P, _P, _P, _P, _I64, _I64, _P], _I),
    "iso_sha256_init": ([ctypes.POINTER(Sha256State)], _I),
    "iso_sha256_update": ([ctypes.POINTER(Sha256State), _P, ctypes.c_size_t], _I),
    "iso_sha256_final": ([ctypes.POINTER(Sha256State), ctypes.c_char_p], _I),
    "iso_table_digests": ([ctypes.POINTER(Composition), ctypes.c_size_t, ctypes.c_char_p,
                           ctypes.c_char_p], _I),
    "iso_table_check": ([ctypes.POINTER(Composition), ctypes.c_size_t, ctypes.c_char_p,
                         ctypes.c_char_p, _CP, _I], _I),
    "iso_swiglu": ([_P, _P, _P, _P, _I64, _P], _I),
    "iso_status_str": ([_I], ctypes.c_char_p),
    "iso_version": ([], ctypes.c_char_p),
    "iso_last_launch_error": ([], ctypes.c_char_p),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

_BAD_SIZE = ctypes.c_size_t(-1).value


def version() -> str:
    return lib.iso_version().decode()


def _ok(status: int, where: str):
    if status != 0:
        raise IsoError(status, where)


def contract(leaf_count: int, leaf_size: int, vocab_chunk: int = 0,
             schedule: int = SCHED_MFMA) -> Contract:
    """A validated contract with the library defaults (bf16 in, FP32
    accumulation, balanced tree) and the given in-leaf schedule (MFMA for
    the matrix products, SCHED_SEQ for rmsnorm)."""
    c = Contract()
    _ok(lib.iso_contract_init(ctypes.byref(c), leaf_count, leaf_size, vocab_chunk),
        "iso_contract_init")
    c.schedule = schedule
    _ok(lib.iso_contract_validate(ctypes.byref(c)), "iso_contract_validate")
    return c


def digest(c: Contract) -> bytes:
    """numerical_policy identity (SHA-256) of a contract."""
    out = ctypes.create_string_buffer(32)
    _ok(lib.iso_contract_digest(ctypes.byref(c), out), "iso_contract_digest")
    return out.raw


def check_identity(c: Contract, want: bytes) -> None:
    if len(want) != 32:
        raise ValueError("a digest is 32 bytes")
    _ok(lib.iso_contract_check(ctypes.byref(c), want), "iso_contract_check")


def check_partitions(c: Contract, partitions: int) -> None:
    _ok(lib.iso_check_partitions(ctypes.byref(c), partitions), "iso_check_partitions")


# ---------------------------------------------------------------- tensors

def _torch():
    import torch
    return torch


def _bf16_ptr(t, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold bf16 (bfloat16 or 16-bit integer bit patterns)")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _dev_ptr(t, name, dtype):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.dtype != dtype:
        raise TypeError(f"{name} must be a torch tensor of {dtype}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _workspace(nbytes, device, ws):
    torch = _torch()
    if nbytes == 0:
        return ws, (0 if ws is None else ws.numel() * ws.element_size())
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def gemm_workspace(c: Contract, M: int, N: int, partitions: int = 1) -> int:
    n = lib.iso_gemm_workspace(ctypes.byref(c), M, N, partitions)
    if n == _BAD_SIZE:
        raise IsoError(1, "iso_gemm_workspace")
    return n


def gemm(A, Wt, c: Contract, *, out=None, out_dtype: int = F32, partitions: int = 1,
         workspace=None, stream=None):
    """C = A @ Wt.T with the contract's leaves and tree.  Returns C."""
    torch = _torch()
    M, K = A.shape
    N = Wt.shape[0]
    if Wt.dim() != 2 or Wt.shape[1] != K:
        raise ValueError("Wt must be [N][K]")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32 if out_dtype == F32 else torch.bfloat16,
                          device=A.device)
    optr = _dev_ptr(out, "out", torch.float32 if out_dtype == F32 else out.dtype)
    if out_dtype == BF16 and out.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError("bf16 output tensor expected")
    if out.shape != (M, N):
        raise ValueError("out must be [M][N]")
    need = gemm_workspace(c, M, N, partitions)
    ws, wsb = _workspace(need, A.device, workspace)
    _ok(lib.iso_gemm(ctypes.byref(c), _bf16_ptr(A, "A"), _bf16_ptr(Wt, "Wt"), optr, out_dtype,
                     M, N, K, partitions, None if ws is None else ws.data_ptr(), wsb,
                     _stream(stream)), "iso_gemm")
    return out


def gemm_baseline(A, Wt, *, out=None, out_dtype: int = F32, stream=None):
    """Non-invariant comparison GEMM (one accumulator over all of K)."""
    torch = _torch()
    M, K = A.shape
    N = Wt.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32 if out_dtype == F32 else torch.bfloat16,
                          device=A.device)
    _ok(lib.iso_gemm_baseline(_bf16_ptr(A, "A"), _bf16_ptr(Wt, "Wt"), out.data_ptr(), out_dtype,
                              M, N, K, _stream(stream)), "iso_gemm_baseline")
    return out


def lmhead_workspace(c: Contract, M: int, V: int, partitions: int = 1) -> int:
    n = lib.iso_lmhead_workspace(ctypes.byref(c), M, V, partitions)
    if n == _BAD_SIZE:
        raise IsoError(1, "iso_lmhead_workspace")
    return n


def lmhead_logprob(H, Wvt, tok, c: Contract, *, out=None, partitions: int = 1,
                   workspace=None, stream=None):
    """logprob[i] = log softmax(H[i] @ Wvt.T)[tok[i]] (FP32)."""
    torch = _torch()
    M, K = H.shape
    V = Wvt.shape[0]
    if Wvt.dim() != 2 or Wvt.shape[1] != K:
        raise ValueError("Wvt must be [V][K]")
    if tok.shape != (M,):
        raise ValueError("tok must be [M]")
    if out is None:
        out = torch.empty(M, dtype=torch.float32, device=H.device)
    need = lmhead_workspace(c, M, V, partitions)
    ws, wsb = _workspace(need, H.device, workspace)
    _ok(lib.iso_lmhead_logprob(ctypes.byref(c), _bf16_ptr(H, "H"), _bf16_ptr(Wvt, "Wvt"),
                               _dev_ptr(tok, "tok", torch.int32),
                               _dev_ptr(out, "out", torch.float32), M, V, K, partitions,
                               None if ws is None else ws.data_ptr(), wsb, _stream(stream)),
        "iso_lmhead_logprob")
    return out


LMHEAD_NOALLOC_BYTES = 32 << 20  # ISO_LMHEAD_NOALLOC_BYTES


def lmhead_logprob_noalloc(H, Wvt, tok, c: Contract, *, out=None, stream=None):
    """lmhead_logprob (one partition) with the library's static device
    scratch as the workspace: the library call allocates nothing (``out`` is
    allocated here when not given).  Calls that overlap on one GPU race."""
    torch = _torch()
    M, K = H.shape
    V = Wvt.shape[0]
    if Wvt.dim() != 2 or Wvt.shape[1] != K:
        raise ValueError("Wvt must be [V][K]")
    if tok.shape != (M,):
        raise ValueError("tok must be [M]")
    if out is None:
        out = torch.empty(M, dtype=torch.float32, device=H.device)
    _ok(lib.iso_lmhead_logprob_noalloc(ctypes.byref(c), _bf16_ptr(H, "H"), _bf16_ptr(Wvt, "Wvt"),
                                       _dev_ptr(tok, "tok", torch.int32),
                                       _dev_ptr(out, "out", torch.float32), M, V, K,
                                       _stream(stream)), "iso_lmhead_logprob_noalloc")
    return out


class MoeLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("idx", "gate", "h", "e", "total")]


def lmhead_shard_stats(H, Wvt_shard, tok, c: Contract, V: int, v_begin: int, stats, target, *,
                       stream=None):
    """Chunk statistics of the vocabulary shard [v_begin, v_begin + rows of
    Wvt_shard) into the shared stats [M][ceil(V/128)][2] and target [M]
    buffers (float32 device tensors)."""
    torch = _torch()
    M, K = H.shape
    v_end = v_begin + Wvt_shard.shape[0]
    _ok(lib.iso_lmhead_shard_stats(ctypes.byref(c), _bf16_ptr(H, "H"),
                                   _bf16_ptr(Wvt_shard, "Wvt_shard"),
                                   _dev_ptr(tok, "tok", torch.int32),
                                   _dev_ptr(stats, "stats", torch.float32),
                                   _dev_ptr(target, "target", torch.float32), M, V, v_begin,
                                   v_end, K, _stream(stream)), "iso_lmhead_shard_stats")


def lmhead_finish(stats, target, tok, V: int, *, out=None, stream=None):
    """logprob [M] from the gathered chunk statistics of every shard."""
    torch = _torch()
    M = tok.shape[0]
    if out is None:
        out = torch.empty(M, dtype=torch.float32, device=tok.device)
    _ok(lib.iso_lmhead_finish(_dev_ptr(stats, "stats", torch.float32),
                              _dev_ptr(target, "target", torch.float32),
                              _dev_ptr(tok, "tok", torch.int32),
                              _dev_ptr(out, "out", torch.float32), M, V, _stream(stream)),
        "iso_lmhead_finish")
    return out


def rmsnorm(x, weight, c: Contract, *, residual=None, residual_out=None, eps: float = 1e-6,
            out=None, out_dtype: int = BF16, stream=None):
    """y = RMSNorm(x [+ residual]) * weight with the contract's fixed leaf
    tree over each row.  residual_out (may be `residual` itself) receives
    bf16(x + residual).  Returns y."""
    torch = _torch()
    if x.dim() != 2:
        raise ValueError("x must be [M][H]")
    M, H = x.shape
    if weight.dim() != 1 or weight.shape[0] != H:
        raise ValueError("weight must be [H]")
    for t, name in ((residual, "residual"), (residual_out, "residual_out")):
        if t is not None and tuple(t.shape) != (M, H):
            raise ValueError(f"{name} must be [M][H]")
    if out is None:
        out = torch.empty((M, H), dtype=torch.float32 if out_dtype == F32 else torch.bfloat16,
                          device=x.device)
    if out_dtype == F32:
        optr = _dev_ptr(out, "out", torch.float32)
    else:
        optr = _bf16_ptr(out, "out")
    if tuple(out.shape) != (M, H):
        raise ValueError("out must be [M][H]")
    _ok(lib.iso_rmsnorm(ctypes.byref(c), _bf16_ptr(x, "x"),
                        None if residual is None else _bf16_ptr(residual, "residual"),
                        None if residual_out is None else _bf16_ptr(residual_out, "residual_out"),
                        _bf16_ptr(weight, "weight"), optr, out_dtype, M, H, float(eps),
                        _stream(stream)), "iso_rmsnorm")
    return out


def cpr_contract(chunk: int, head_size: int = 128) -> Contract:
    """Contract of the CPR gated delta rule: head size d (tree leaves of the
    dot products) and chunk length C (the state re-sync interval)."""
    return contract(head_size, chunk, 0, SCHED_CPR)


def cpr_workspace(c: Contract, H: int, T: int) -> int:
    n = lib.iso_cpr_workspace(ctypes.byref(c), H, T)
    if n == _BAD_SIZE:
        raise IsoError(1, "iso_cpr_workspace")
    return n


def _cpr_seq(q, k, v, alpha, beta):
    if q.dim() != 3 or tuple(k.shape) != tuple(q.shape) or tuple(v.shape) != tuple(q.shape):
        raise ValueError("q, k, v must be [T][H][d]")
    T, H, _ = q.shape
    if tuple(alpha.shape) != (T, H) or tuple(beta.shape) != (T, H):
        raise ValueError("alpha, beta must be [T][H]")
    return T, H


def cpr_prefill(q, k, v, alpha, beta, c: Contract, *, S0=None, out=None, snap=None, run=None,
                workspace=None, stream=None):
    """CPR prefill of q, k, v [T][H][d] (bf16), alpha, beta [T][H] (float32)
    from the boundary state S0 [H][d][d] (zeros if None).  Returns
    (o [T][H][d], snap [H][d][d], run [H][d][d]) as float32 tensors."""
    torch = _torch()
    T, H = _cpr_seq(q, k, v, alpha, beta)
    d = q.shape[2]
    dev = q.device
    if S0 is not None and tuple(S0.shape) != (H, d, d):
        raise ValueError("S0 must be [H][d][d]")
    if out is None:
        out = torch.empty((T, H, d), dtype=torch.float32, device=dev)
    if snap is None:
        snap = torch.empty((H, d, d), dtype=torch.float32, device=dev)
    if run is None:
        run = torch.empty((H, d, d), dtype=torch.float32, device=dev)
    if workspace is None:
        ws, wsb = _workspace(cpr_workspace(c, H, T), dev, None)
    else:  # the entry point checks its size
        ws, wsb = workspace, workspace.numel() * workspace.element_size()
    _ok(lib.iso_cpr_prefill(ctypes.byref(c), _bf16_ptr(q, "q"), _bf16_ptr(k, "k"),
                            _bf16_ptr(v, "v"), _dev_ptr(alpha, "alpha", torch.float32),
                            _dev_ptr(beta, "beta", torch.float32),
                            None if S0 is None else _dev_ptr(S0, "S0", torch.float32),
                            _dev_ptr(out, "out", torch.float32),
                            _dev_ptr(snap, "snap", torch.float32),
                            _dev_ptr(run, "run", torch.float32), T, H,
                            None if ws is None else ws.data_ptr(), wsb, _stream(stream)),
        "iso_cpr_prefill")
    return out, snap, run


def cpr_decode_step(q, k, v, alpha, beta, pos: int, snap, run, c: Contract, *, out=None,
                    workspace=None, stream=None):
    """One CPR decode step of token `pos` of the sequence arrays (tokens
    0..pos present); snap and run [H][d][d] are updated in place.  Returns
    o [H][d]."""
    torch = _torch()
    T, H = _cpr_seq(q, k, v, alpha, beta)
    if not 0 <= pos < T:
        raise ValueError("pos must index a token of the sequence arrays")
    d = q.shape[2]
    if tuple(snap.shape) != (H, d, d) or tuple(run.shape) != (H, d, d):
        raise ValueError("snap, run must be [H][d][d]")
    if out is None:
        out = torch.empty((H, d), dtype=torch.float32, device=q.device)
    if workspace is None:
        ws, wsb = _workspace(cpr_workspace(c, H, c.leaf_size), q.device, None)
    else:
        ws, wsb = workspace, workspace.numel() * workspace.element_size()
    _ok(lib.iso_cpr_decode_step(ctypes.byref(c), _bf16_ptr(q, "q"), _bf16_ptr(k, "k"),
                                _bf16_ptr(v, "v"), _dev_ptr(alpha, "alpha", torch.float32),
                                _dev_ptr(beta, "beta", torch.float32), pos,
                                _dev_ptr(snap, "snap", torch.float32),
                                _dev_ptr(run, "run", torch.float32),
                                _dev_ptr(out, "out", torch.float32), H,
                                None if ws is None else ws.data_ptr(), wsb, _stream(stream)),
        "iso_cpr_decode_step")
    return out


def moe_layout(T: int, H: int, E: int, I: int, top_k: int) -> MoeLayout:
    out = MoeLayout()
    _ok(lib.iso_moe_layout_of(T, H, E, I, top_k, ctypes.byref(out)), "iso_moe_layout_of")
    return out


def moe_workspace(T: int, H: int, E: int, I: int, top_k: int) -> int:
    n = lib.iso_moe_workspace(T, H, E, I, top_k)
    if n == _BAD_SIZE:
        raise IsoError(1, "iso_moe_workspace")
    return n


def moe_combine(X, router_logits, Wg, Wu, Wd, top_k: int, gate_up: Contract, down: Contract, *,
                out=None, workspace=None, stream=None):
    """MoE FFN with the fixed routing-order combine.  X [T][H] bf16, logits
    [T][E] fp32, Wg/Wu [E][I][H], Wd [E][H][I] bf16.  Returns Y [T][H] fp32."""
    torch = _torch()
    T, H = X.shape
    E, I, H2 = Wg.shape
    if H2 != H or tuple(Wu.shape) != (E, I, H) or tuple(Wd.shape) != (E, H, I):
        raise ValueError("weight shapes must be Wg/Wu [E][I][H], Wd [E][H][I]")
    if tuple(router_logits.shape) != (T, E):
        raise ValueError("router logits must be [T][E]")
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=X.device)
    need = moe_workspace(T, H, E, I, top_k)
    ws, wsb = _workspace(need, X.device, workspace)
    _ok(lib.iso_moe_combine(ctypes.byref(gate_up), ctypes.byref(down), _bf16_ptr(X, "X"),
                            _dev_ptr(router_logits, "router_logits", torch.float32),
                            _bf16_ptr(Wg, "Wg"), _bf16_ptr(Wu, "Wu"), _bf16_ptr(Wd, "Wd"),
                            _dev_ptr(out, "out", torch.float32), T, H, E, I, top_k,
                            None if ws is None else ws.data_ptr(), wsb, _stream(stream)),
        "iso_moe_combine")
    return out


def swiglu(G, U, *, act=True, stream=None):
    """h = bf16(silu(G) * U) element by element (G, U float32 device tensors
    of one shape), with the MoE gate/up stage's device function.  Returns h
    (bfloat16), or (act, h) with the FP32 activation before rounding when
    act is True."""
    torch = _torch()
    if tuple(G.shape) != tuple(U.shape):
        raise ValueError("G and U must have one shape")
    gp = _dev_ptr(G, "G", torch.float32)
    up = _dev_ptr(U, "U", torch.float32)
    h = torch.empty(G.shape, dtype=torch.bfloat16, device=G.device)
    a = torch.empty(G.shape, dtype=torch.float32, device=G.device) if act else None
    _ok(lib.iso_swiglu(gp, up, None if a is None else a.data_ptr(), h.data_ptr(), G.numel(),
                       _stream(stream)), "iso_swiglu")
    return (a, h) if act else h


def moe_stages(workspace, T: int, H: int, E: int, I: int, top_k: int) -> dict:
    """Views of the stage outputs left in a MoE workspace: idx [T][k] int32,
    gate [T][k] fp32, h [T][k][I] bf16, e [T][k][H] fp32."""
    torch = _torch()
    lay = moe_layout(T, H, E, I, top_k)
    b = workspace.view(torch.uint8)
    tk = T * top_k

    def view(off, n, dt, shape):
        return b[off:off + n * torch.tensor([], dtype=dt).element_size()].view(dt).view(*shape)

    return dict(idx=view(lay.idx, tk, torch.int32, (T, top_k)),
                gate=view(lay.gate, tk, torch.float32, (T, top_k)),
                h=view(lay.h, tk * I, torch.bfloat16, (T, top_k, I)),
                e=view(lay.e, tk * H, torch.float32, (T, top_k, H)))


# ------------------------------------------------------------------ identities

def semantic_digest(items) -> bytes:
    """SHA-256 over the bytes of `items` in order: numpy arrays and torch
    tensors (copied to the host, contiguous, raw element bytes), bytes, or
    str (UTF-8, e.g. a model configuration as canonical JSON)."""
    import numpy as np
    st = Sha256State()
    _ok(lib.iso_sha256_init(ctypes.byref(st)), "iso_sha256_init")
    for it in items:
        if isinstance(it, str):
            buf = it.encode()
        elif isinstance(it, (bytes, bytearray)):
            buf = bytes(it)
        elif hasattr(it, "detach"):  # torch tensor
            t = it.detach().contiguous().cpu()
            buf = t.view(_torch().uint8).numpy().tobytes() if t.numel() else b""
        else:
            buf = np.ascontiguousarray(it).tobytes()
        _ok(lib.iso_sha256_update(ctypes.byref(st), buf, len(buf)), "iso_sha256_update")
    out = ctypes.create_string_buffer(32)
    _ok(lib.iso_sha256_final(ctypes.byref(st), out), "iso_sha256_final")
    return out.raw


class ExecutionContract:
    """Regions x cases compositions with their identities, and the per-call
    check.  compositions: {(region, case): (contract, partitions, claims)}
    where claims is an iterable of partition counts."""

    def __init__(self, compositions: dict, semantic: bytes = b""):
        self._table = (Composition * len(compositions))()
        for i, ((region, case), (c, p, claims)) in enumerate(sorted(compositions.items())):
            e = self._table[i]
            e.region = region.encode()
            e.case_name = case.encode()
            e.policy = c
            e.partitions = p
            e.claims = sum(1 << (int(q).bit_length() - 1) for q in set(claims))
        self.semantic = semantic
        pol = ctypes.create_string_buffer(32)
        dep = ctypes.create_string_buffer(32)
        _ok(lib.iso_table_digests(self._table, len(compositions), pol, dep), "iso_table_digests")
        self.numerical_policy = pol.raw
        self.deployment = dep.raw

    def identities(self) -> dict:
        return {"semantic": self.semantic, "numerical_policy": self.numerical_policy,
                "deployment": self.deployment}

    def check(self, region: str, case: str, c: Contract, partitions: int = 1) -> None:
        """Raises IsoError (ISO_ERR_IDENTITY / ISO_ERR_CLAIM / ISO_ERR_ARG)
        unless the call matches the registered composition."""
        _ok(lib.iso_table_check(self._table, len(self._table), region.encode(), case.encode(),
                                ctypes.byref(c), partitions), "iso_table_check")
