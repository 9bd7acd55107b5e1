"""iso_lmhead_logprob_noalloc (the LM-head with the library's static device
scratch, for callers that cannot allocate) gives the bits of
iso_lmhead_logprob, called through the C ABI: two calls in a row, the second
smaller than the first, so the second reads a scratch that still holds the
first call's statistics; bad token ids give NaN either way."""
import ctypes

import numpy as np
import pytest

from gpu_util import dev, dev_i32, host, note, torch
from iso_synth import normal_bf16, uniform_tokens

pytestmark = pytest.mark.gpu

iso = pytest.importorskip("parallelism_invariant_numerics_amd")


def _noalloc(c, dH, dW, dtok, out, M, V, K):
    t = torch()
    stream = t.cuda.current_stream().cuda_stream
    return iso.lib.iso_lmhead_logprob_noalloc(ctypes.byref(c), dH.data_ptr(), dW.data_ptr(),
                                              dtok.data_ptr(), out.data_ptr(), M, V, K, stream)


@pytest.mark.parametrize("first,second", [((700, 9000, 1024, 8), (40, 2000, 512, 4)),
                                          ((16, 151936, 2048, 8), (3, 600, 256, 4))])
def test_noalloc_matches_workspace_call(first, second):
    t = torch()
    for n, (M, V, K, L) in enumerate((first, second)):
        note(f"lmhead noalloc call {n}: M={M} V={V} K={K} L={L}")
        H = normal_bf16(601 + n, (M, K), 1.0)
        W = normal_bf16(611 + n, (V, K), 0.02)
        tok = uniform_tokens(621 + n, M, V)
        tok[::11] = -1
        tok[1] = V
        c = iso.contract(L, K // L, 128)
        dH, dW, dtok = dev(H), dev(W), dev_i32(tok)
        ref = host(iso.lmhead_logprob(dH, dW, dtok, c))
        out = t.full((M,), 7.0, dtype=t.float32, device="cuda")
        assert _noalloc(c, dH, dW, dtok, out, M, V, K) == 0
        got = host(out)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), n
        assert np.isnan(got[::11]).all() and np.isnan(got[1])
        assert np.isfinite(np.delete(got, np.r_[0:M:11, 1])).all()


def test_noalloc_rejects_oversize_before_launch():
    t = torch()
    c = iso.contract(8, 256, 128)
    V = 151936
    M = 3533  # one row past what ISO_LMHEAD_NOALLOC_BYTES holds at this vocabulary
    dH = t.empty((M, 2048), dtype=t.bfloat16, device="cuda")
    dW = t.empty((128, 2048), dtype=t.bfloat16, device="cuda")  # never read
    dtok = t.zeros(M, dtype=t.int32, device="cuda")
    out = t.empty(M, dtype=t.float32, device="cuda")
    assert _noalloc(c, dH, dW, dtok, out, M, V, 2048) == 6  # ISO_ERR_WORKSPACE
