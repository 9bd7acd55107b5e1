"""Benchmark of the invariant matmul / token-logprob path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--quick]

One step is one invariant GEMM of the prefill-shaped linear layer
(A [4096 x 2048] bf16 times W [2048 x 2048] bf16, 8 contiguous leaves of 256
along K, FP32 accumulation and fixed tree, bf16 output) with its inputs
resident in HBM; ``value`` is TFLOP/s (2 M N K per step).  The same run also
times, as sub-measurements reported in the JSON line:
  * the cost of invariance next to a non-invariant comparator on every
    workload: the same tiles with one accumulator over all of K and torch's
    linear layer (prefill and 4096^3 sweep shapes), the fused LM-head with one
    accumulator per logit and torch's linear + log_softmax + gather, the MoE
    block with one-leaf contracts and a plain torch expert loop scattering
    with index_add_;
  * 64 rows of the prefill layer (K split over the workspace);
  * the sweep shape (4096 x 4096 x 4096, 16 leaves) at 1 and 8 partitions and
    at batches of 1, 8 and 64 rows; the LM-head logprob workload (8192 rows x
    2048 x 151936 vocabulary) in rows/s, fused, over 8 vocabulary shards and
    one row per call; the MoE FFN block (4096 tokens, 128 experts, top-8); the
    RMSNorm with residual add in front of the LM-head (8192 x 2048, GB/s); the
    CPR gated delta rule (16 heads of 128, 4096 tokens, chunk 64);
  * bitwise invariance checks (rows alone against the batch, partitions,
    vocabulary shards, token orderings, decode against prefill);
  * workspace bytes of each entry point at these shapes.
With the CPU baseline (default) the oracle is timed on the host cores: the
prefill GEMM on all threads (``cpu_baseline``) and on one thread, the tiny
workload, 64 LM-head rows over the full vocabulary, the 4096^3 sweep layer and
the MoE block; and |gpu - oracle| percentiles with the largest error over
tolerance are reported for 4096 sampled prefill elements and those 64 rows.
Prints ONE JSON line.

Inputs are seeded synthetic data with the workloads' shapes and
distributions (no dataset or trained weights are involved).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# FP32 vector operations (one multiply or one add, no FMA, no packed pairs):
# 256 CUs x 128 FP32 lanes per clock x 2.4 GHz; the 157.3 TFLOP/s vector figure
# counts an FMA as two.  Independent v_add_f32 / v_mul_f32 measure ~71 T/s at
# the loaded clock with four waves per SIMD, ~49 T/s with one.
PEAK_FP32_OPS_T = 78.6


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--quick", action="store_true",
                   help="headline GEMM launches only (for rocprofv3 runs)")
    p.add_argument("--settle", type=float, default=0.3,
                   help="seconds of untimed back-to-back launches before each timing "
                        "(clocks ramp up under sustained load); 0 for counter runs")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="first run one plain copy kernel over 256 MiB (HBM counter calibration)")
    return p.parse_args()


def _dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


SETTLE_S = 0.3


def _settle(fn, seconds=None):
    """Run fn back to back for about `seconds` of wall time, untimed.  The
    GPU raises its clocks only after some tens of milliseconds of sustained
    load; a few warmup steps of a 50 us kernel would time the ramp instead of
    the steady state."""
    import torch
    if seconds is None:
        seconds = SETTLE_S
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            fn()
        torch.cuda.synchronize()


def _time_events(fn, steps, stream):
    """Average duration (ms) of one fn() call: HIP events on `stream` around
    `steps` back-to-back calls (the launches queue up, so host-side call
    overhead does not appear as idle GPU time between them as long as the
    host issues calls faster than the GPU runs them)."""
    import torch
    _settle(fn, 0.66 * SETTLE_S)
    fn()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def _abi_gemm(iso, c, A, W, out, ws, stream):
    """A zero-argument call of iso_gemm through the C ABI with its arguments
    marshalled once, as a C or C++ caller makes it: for calls of ~10 us the
    Python binding's per-call work is about as long as the GPU's, so timing
    through it measures the host."""
    import ctypes
    args = (ctypes.byref(c), A.data_ptr(), W.data_ptr(), out.data_ptr(),
            iso.F32 if out.dtype == __import__("torch").float32 else iso.BF16,
            A.shape[0], W.shape[0], A.shape[1], 1,
            None if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel(),
            stream.cuda_stream)
    f = iso.lib.iso_gemm

    def call():
        if f(*args) != 0:
            raise RuntimeError("iso_gemm failed")
    return call


def _time_graph(fn, inner=20, replays=10, check=None, reset=None):
    """Average duration (ms) of one fn() call replayed from a HIP graph of
    `inner` back-to-back calls: the GPU time of a call without the Python
    launch path (what a serving loop that replays graphs sees).  fn must not
    allocate.  Returns None if capture is not available."""
    import torch
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(inner):
                fn()
        if reset is not None:
            reset()  # eager work between the capture and the replay: the replay must redo it
        g.replay()
        torch.cuda.synchronize()
        if check is not None and not check():
            return float("nan")  # a replay that changes the bits is reported, not timed
        _settle(g.replay, 0.66 * SETTLE_S)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(replays):
            g.replay()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / (replays * inner)
    except RuntimeError:
        return None


def _source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


GEMM_SOURCES = ["parallelism_invariant_numerics_amd/csrc/gemm_core.hpp",
                "parallelism_invariant_numerics_amd/csrc/gemm_wide.hpp",
                "parallelism_invariant_numerics_amd/csrc/gemm.hip",
                "parallelism_invariant_numerics_amd/csrc/device_common.hpp"]


def _traffic(kernel_hash):
    """Measured HBM bytes per launch of the dominant kernel, from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "gemm_leaf_prefill_hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_hash:
        return None
    return rec.get("bytes_per_launch")


def _timed(fn):
    t0 = time.perf_counter()
    r = fn()
    return r, time.perf_counter() - t0


def _cpu_baseline(cfg, target_s=6.0):
    """The oracle (untuned) on the same GEMM: a row sample sized from a 256-row calibration run
    (the whole job at most), repeated until about target_s of CPU time have passed."""
    import oracle
    A, Wt, L = cfg["A"], cfg["Wt"], cfg["leaves"]
    rows = 256
    _, dt = _timed(lambda: oracle.gemm(A[:rows], Wt, L))
    rows = int(min(cfg["M"], max(16, rows * target_s / max(dt, 1e-6))))
    reps, total = 0, 0.0
    while reps == 0 or (total < target_s and reps < 100):
        _, dt = _timed(lambda: oracle.gemm(A[:rows], Wt, L))
        total += dt
        reps += 1
    flops = 2.0 * rows * cfg["N"] * cfg["K"] * reps
    what = (f"the whole prefill GEMM ({rows}x{cfg['N']}x{cfg['K']}, 8 leaves)" if rows == cfg["M"]
            else f"{rows} of {cfg['M']} rows of the prefill GEMM ({rows}x{cfg['N']}x{cfg['K']}, 8 leaves)")
    what += f", {reps} run{'s' if reps > 1 else ''}"
    return {"value": flops / total / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle", "sample": f"{what}, {total:.1f} s"}


def _cpu_more(cfg, lm, mc, single_s=3.0):
    """Oracle timings of the other workloads on all host threads (the tiny one
    whole, 64 rows of the LM-head over the full vocabulary, the 4096^3 sweep
    layer at one partition, the MoE block whole) and of a prefill-GEMM row
    sample on one thread."""
    import oracle
    from iso_synth import make_config, normal_bf16
    out = {}
    ti = make_config("tiny")
    _, dt = _timed(lambda: (oracle.gemm(ti["A"], ti["Wt"], ti["leaves"]),
                            oracle.lmhead_logprob(ti["A"], ti["Wt"], ti["tok"], ti["leaves"])))
    out["tiny_gemm_logprob_s"] = round(dt, 4)
    rows = np.sort(np.random.default_rng(2025).choice(lm["M"], 64, replace=False))
    (lp, _, _), dt = _timed(lambda: oracle.lmhead_logprob(lm["H"][rows], lm["Wvt"], lm["tok"][rows],
                                                          lm["leaves"]))
    out["lmhead_64rows_s"] = round(dt, 3)
    out["lmhead_rows_per_s"] = round(64 / dt, 2)
    Ws = normal_bf16(401, (4096, 4096), 0.02)
    As = normal_bf16(403, (4096, 4096), 1.0)
    _, dt = _timed(lambda: oracle.gemm(As, Ws, 16))
    out["sweep_p1_s"] = round(dt, 3)
    out["sweep_p1_tflops"] = round(2.0 * 4096 ** 3 / dt / 1e12, 4)
    del Ws, As
    _, dt = _timed(lambda: oracle.moe(mc["X"], mc["logits"], mc["Wg"], mc["Wu"], mc["Wd"],
                                      mc["top_k"], mc["leaves_gate_up"], mc["leaves_down"]))
    out["moe_s"] = round(dt, 3)
    out["moe_tokens_per_s"] = round(mc["T"] / dt, 1)
    # one thread: a row sample of the prefill GEMM sized from a 16-row run
    n_all = oracle.threads()
    oracle.set_threads(1)
    try:
        _, dt = _timed(lambda: oracle.gemm(cfg["A"][:16], cfg["Wt"], cfg["leaves"]))
        r1 = int(min(cfg["M"], max(16, 16 * single_s / max(dt, 1e-6))))
        _, dt = _timed(lambda: oracle.gemm(cfg["A"][:r1], cfg["Wt"], cfg["leaves"]))
    finally:
        oracle.set_threads(n_all)
    out["single_thread"] = {"value": 2.0 * r1 * cfg["N"] * cfg["K"] / dt / 1e12, "unit": "TFLOP/s",
                            "cores": 1, "sample": f"{r1} rows of the prefill GEMM, {dt:.1f} s"}
    return out, lp, rows


def _pcts(x):
    x = np.asarray(x, dtype=np.float64)
    return {"p50": float(np.percentile(x, 50)), "p95": float(np.percentile(x, 95)),
            "p99": float(np.percentile(x, 99)), "max": float(np.max(x))}


def _parity(cfg, c2_rows, c2_cols, c2_gpu, lm_rows, c3_gpu, c3_oracle):
    """|gpu - oracle| over the sampled prefill-GEMM elements (FP32 roots) and
    the sampled LM-head rows, with the largest error / tolerance."""
    import oracle
    from iso_synth import bf16_bits_to_f32
    want = oracle.gemm_elems(cfg["A"], cfg["Wt"], cfg["leaves"], c2_rows, c2_cols).astype(np.float64)
    a = np.abs(bf16_bits_to_f32(cfg["A"][c2_rows]).astype(np.float64))
    w = np.abs(bf16_bits_to_f32(cfg["Wt"][c2_cols]).astype(np.float64))
    tol = 1e-5 * np.einsum("ik,ik->i", a, w)
    err = np.abs(c2_gpu.astype(np.float64) - want)
    lerr = np.abs(c3_gpu.astype(np.float64) - c3_oracle)
    assert np.array_equal(lm_rows, np.sort(lm_rows))
    return {"prefill": {"elements": int(err.size), "abs_err": _pcts(err),
                        "max_err_over_tol": float(np.max(err / tol)),
                        "tolerance": "1e-5 * sum_k |a_k b_k| per element"},
            "lmhead": {"rows": int(lerr.size), "abs_err": _pcts(lerr),
                       "max_err_over_tol": float(np.max(lerr) / 1e-5),
                       "tolerance": "1e-5 absolute per logprob"}}


def main():
    args = _args()
    global SETTLE_S
    SETTLE_S = max(0.0, args.settle)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch

    import parallelism_invariant_numerics_amd as iso
    from iso_synth import make_config, normal_bf16

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    if args.calibrate_copy:
        # an elementwise kernel that reads 256 MiB and writes 256 MiB
        src = torch.ones(1 << 26, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.add(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # ---------------- headline: prefill linear layer, invariant GEMM
    cfg = make_config("prefill")
    M, N, K, L = cfg["M"], cfg["N"], cfg["K"], cfg["leaves"]
    A, W = _dev(cfg["A"]), _dev(cfg["Wt"])
    c = iso.contract(L, K // L, 0)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    step = lambda: iso.gemm(A, W, c, out=out, out_dtype=iso.BF16)
    _settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    flop = 2.0 * M * N * K
    value = flop * args.steps / wall / 1e12
    kern_ms = _time_events(step, args.steps, stream)
    achieved = flop / (kern_ms * 1e-3) / 1e12
    src_hash = _source_hash(GEMM_SOURCES)
    line = {
        "metric": "invariant bf16 GEMM TFLOP/s + % MFMA peak; LM-head logprob rows/s; bitwise pass",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefill linear layer: A[4096x2048] bf16 ~N(0,1) x W[2048x2048] "
                               "bf16 ~N(0,0.02), 8 leaves of 256, FP32 accumulation, bf16 out",
                   "M": M, "N": N, "K": K, "leaves": L, "leaf_size": K // L, "partitions": 1},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": _traffic(src_hash), "kernel": "gemm_leaf_kernel<CfgWide, 3>",
                     "kernel_ms": round(kern_ms, 5), "algorithmic_flop": flop,
                     "source_hash": src_hash},
    }
    extra = {}
    if args.quick:
        print(json.dumps(line), flush=True)
        return

    ok = True
    # ---------------- cost of invariance on the same shape
    outb = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    base = lambda: iso.gemm_baseline(A, W, out=outb, out_dtype=iso.BF16)
    for _ in range(3):
        base()
    b_ms = _time_events(base, args.steps, stream)
    # torch's linear layer on the same [N][K] weight storage (hipBLASLt)
    tm = lambda: torch.nn.functional.linear(A, W)
    for _ in range(3):
        tm()
    t_ms = _time_events(tm, args.steps, stream)
    extra["prefill"] = {
        "invariant_tflops": round(achieved, 2),
        "mfma_frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "baseline_tflops": round(flop / (b_ms * 1e-3) / 1e12, 2),
        "torch_linear_tflops": round(flop / (t_ms * 1e-3) / 1e12, 2),
        "invariance_overhead_vs_baseline": round(kern_ms / b_ms - 1.0, 4),
        "invariance_overhead_vs_torch": round(kern_ms / t_ms - 1.0, 4),
    }
    # FP32 roots of sampled elements for the |gpu - oracle| figures (same bits
    # as the bf16 output before its rounding)
    rng = np.random.default_rng(2024)
    c2_rows = rng.integers(0, M, 4096)
    c2_cols = rng.integers(0, N, 4096)
    outf = iso.gemm(A, W, c, out_dtype=iso.F32)
    torch.cuda.synchronize()
    c2_gpu = outf[torch.from_numpy(c2_rows).to("cuda"), torch.from_numpy(c2_cols).to("cuda")].cpu().numpy()
    ok &= bool(torch.equal(outf.to(torch.bfloat16).view(torch.int16), out.view(torch.int16)))
    del outf
    extra["workspace_bytes"] = {
        "prefill_p1": iso.gemm_workspace(c, M, N, 1),
        "prefill_p8": iso.gemm_workspace(c, M, N, 8),
    }
    # bitwise: rows alone / in the batch, and 1 vs 8 partitions
    ref = out.clone()
    alone = torch.empty((8, N), dtype=torch.bfloat16, device="cuda")
    rows = [0, 1, 127, 128, 2048, 4000, 4094, 4095]
    for i, r in enumerate(rows):
        iso.gemm(A[r:r + 1].contiguous(), W, c, out=alone[i:i + 1], out_dtype=iso.BF16)
    torch.cuda.synchronize()
    ok &= bool(torch.equal(alone.view(torch.int16), ref[rows].view(torch.int16)))
    out8 = torch.empty_like(out)
    iso.gemm(A, W, c, out=out8, out_dtype=iso.BF16, partitions=8)
    torch.cuda.synchronize()
    ok &= bool(torch.equal(out8.view(torch.int16), ref.view(torch.int16)))
    del out8, outb
    # 64 rows of the same layer (a small batch through it): K split over the
    # workspace and the roots folded tile by tile; rows 100.. of the batch, so
    # the bits must match it
    A64 = A[100:164].contiguous()
    o64 = torch.empty((64, N), dtype=torch.bfloat16, device="cuda")
    ws64 = torch.empty(max(1, iso.gemm_workspace(c, 64, N, 1)), dtype=torch.uint8, device="cuda")
    a64 = _abi_gemm(iso, c, A64, W, o64, ws64, stream)
    a64()
    ms64 = _time_events(a64, max(10, args.steps), stream)
    ok &= bool(torch.equal(o64.view(torch.int16), ref[100:164].view(torch.int16)))
    extra["prefill"]["rows64_us"] = round(ms64 * 1e3, 2)
    extra["workspace_bytes"]["prefill_rows64"] = iso.gemm_workspace(c, 64, N, 1)
    del A64, o64, ws64

    if not args.quick:
        # ---------------- invariance-sweep shape, 16 leaves
        Ks = 4096
        Ws = _dev(normal_bf16(401, (4096, Ks), 0.02))
        As = _dev(normal_bf16(403, (4096, Ks), 1.0))
        cs = iso.contract(16, 256, 0)
        outs = torch.empty((4096, 4096), dtype=torch.float32, device="cuda")
        ws8 = torch.empty(iso.gemm_workspace(cs, 4096, 4096, 8), dtype=torch.uint8, device="cuda")
        g1 = lambda: iso.gemm(As, Ws, cs, out=outs)
        g8 = lambda: iso.gemm(As, Ws, cs, out=outs, partitions=8, workspace=ws8)
        g1()
        ms1 = _time_events(g1, max(5, args.steps // 5), stream)
        ref_s = outs.clone()
        g8()
        ms8 = _time_events(g8, max(5, args.steps // 5), stream)
        ok &= bool(torch.equal(outs.view(torch.int32), ref_s.view(torch.int32)))
        fs = 2.0 * 4096 * 4096 * Ks
        # the cost of invariance at this shape: one accumulator over all of K
        # on the same tiles, and torch's linear layer (hipBLASLt, bf16 out)
        outsb = torch.empty_like(outs)
        gb = lambda: iso.gemm_baseline(As, Ws, out=outsb)
        gb()
        msb = _time_events(gb, max(5, args.steps // 5), stream)
        gt = lambda: torch.nn.functional.linear(As, Ws)
        gt()
        mst = _time_events(gt, max(5, args.steps // 5), stream)
        del outsb
        extra["sweep"] = {"shape": "4096x4096x4096, 16 leaves of 256, fp32 out",
                          "p1_tflops": round(fs / (ms1 * 1e-3) / 1e12, 2),
                          "p1_mfma_frac": round(fs / (ms1 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "p8_tflops": round(fs / (ms8 * 1e-3) / 1e12, 2),
                          "p1_ms": round(ms1, 4), "p8_ms": round(ms8, 4),
                          "baseline_tflops": round(fs / (msb * 1e-3) / 1e12, 2),
                          "torch_linear_tflops": round(fs / (mst * 1e-3) / 1e12, 2),
                          "invariance_overhead_vs_baseline": round(ms1 / msb - 1.0, 4),
                          "invariance_overhead_vs_torch": round(ms1 / mst - 1.0, 4)}
        extra["workspace_bytes"]["sweep_p8"] = iso.gemm_workspace(cs, 4096, 4096, 8)
        # one row per call (a decode step of the same layer): the weights streamed once
        A1 = As[:1].contiguous()
        o1 = torch.empty((1, 4096), dtype=torch.float32, device="cuda")
        g_1 = lambda: iso.gemm(A1, Ws, cs, out=o1)
        g_1()
        ms_1p = _time_events(g_1, max(10, args.steps), stream)
        ok &= bool(torch.equal(o1.view(torch.int32), ref_s[:1].view(torch.int32)))
        o1.zero_()
        a_1 = _abi_gemm(iso, cs, A1, Ws, o1, None, stream)
        a_1()
        ms_1 = _time_events(a_1, max(10, args.steps), stream)
        ok &= bool(torch.equal(o1.view(torch.int32), ref_s[:1].view(torch.int32)))
        extra["sweep"]["row1_us"] = round(ms_1 * 1e3, 2)
        extra["sweep"]["row1_binding_us"] = round(ms_1p * 1e3, 2)
        extra["sweep"]["row1_weight_gbs"] = round(4096 * Ks * 2 / (ms_1 * 1e-3) / 1e9, 1)
        gr = _time_graph(g_1, reset=o1.zero_,
                         check=lambda: torch.equal(o1.view(torch.int32), ref_s[:1].view(torch.int32)))
        ok &= bool(torch.equal(o1.view(torch.int32), ref_s[:1].view(torch.int32)))
        ok &= gr is None or gr == gr
        extra["sweep"]["row1_graph_us"] = None if gr is None else round(gr * 1e3, 2)
        # batches of 8 and 64 rows of the same layer (the sweep's other batch
        # sizes); rows 100.. of the 4096-row batch, so the bits must match it
        for mb in (8, 64):
            Ab = As[100:100 + mb].contiguous()
            ob = torch.empty((mb, 4096), dtype=torch.float32, device="cuda")
            wsb = torch.empty(max(1, iso.gemm_workspace(cs, mb, 4096, 1)), dtype=torch.uint8,
                              device="cuda")
            g_b = lambda: iso.gemm(Ab, Ws, cs, out=ob, workspace=wsb)
            g_b()
            ms_bp = _time_events(g_b, max(10, args.steps), stream)
            ok &= bool(torch.equal(ob.view(torch.int32), ref_s[100:100 + mb].view(torch.int32)))
            ob.zero_()
            a_b = _abi_gemm(iso, cs, Ab, Ws, ob, wsb, stream)
            a_b()
            ms_b = _time_events(a_b, max(10, args.steps), stream)
            ok &= bool(torch.equal(ob.view(torch.int32), ref_s[100:100 + mb].view(torch.int32)))
            extra["sweep"][f"rows{mb}_us"] = round(ms_b * 1e3, 2)
            extra["sweep"][f"rows{mb}_binding_us"] = round(ms_bp * 1e3, 2)
            extra["sweep"][f"rows{mb}_weight_gbs"] = round(4096 * Ks * 2 / (ms_b * 1e-3) / 1e9, 1)
            gr = _time_graph(g_b, reset=ob.zero_, check=lambda: torch.equal(ob.view(torch.int32),
                                                            ref_s[100:100 + mb].view(torch.int32)))
            ok &= bool(torch.equal(ob.view(torch.int32), ref_s[100:100 + mb].view(torch.int32)))
            ok &= gr is None or gr == gr
            extra["sweep"][f"rows{mb}_graph_us"] = None if gr is None else round(gr * 1e3, 2)
        del Ws, As, outs, ws8, ref_s, A1, o1, Ab, ob, wsb

        # ---------------- LM-head logprob
        lm = make_config("lmhead")
        H, Wv = _dev(lm["H"]), _dev(lm["Wvt"])
        tok = torch.from_numpy(lm["tok"]).to("cuda")
        cl = iso.contract(lm["leaves"], lm["K"] // lm["leaves"], iso.VOCAB_CHUNK)
        lp = torch.empty(lm["M"], dtype=torch.float32, device="cuda")
        wsl = torch.empty(iso.lmhead_workspace(cl, lm["M"], lm["V"], 1), dtype=torch.uint8,
                          device="cuda")
        run_lm = lambda: iso.lmhead_logprob(H, Wv, tok, cl, out=lp, workspace=wsl)
        run_lm()
        lm_ms = _time_events(run_lm, max(3, args.steps // 10), stream)
        lm_flop = 2.0 * lm["M"] * lm["V"] * lm["K"]
        lp_ref = lp.clone()
        lp8 = torch.empty(8, dtype=torch.float32, device="cuda")
        wsl8 = torch.empty(iso.lmhead_workspace(cl, 8, lm["V"], 1), dtype=torch.uint8, device="cuda")
        iso.lmhead_logprob(H[4000:4008].contiguous(), Wv, tok[4000:4008].contiguous(), cl, out=lp8,
                           workspace=wsl8)
        torch.cuda.synchronize()
        ok &= bool(torch.equal(lp8.view(torch.int32), lp_ref[4000:4008].view(torch.int32)))
        extra["lmhead"] = {"shape": "8192 x 2048 x 151936, 8 leaves of 256, 1187 vocab chunks",
                           "rows_per_s": round(lm["M"] / (lm_ms * 1e-3), 1),
                           "ms": round(lm_ms, 4),
                           "tflops": round(lm_flop / (lm_ms * 1e-3) / 1e12, 2),
                           "mfma_frac": round(lm_flop / (lm_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        # the cost of invariance at this shape: the fused kernel with one
        # accumulator per logit (no leaf tree), and torch's unconstrained path
        # (linear layer to bf16 logits, FP32 log_softmax, gather)
        cl1 = iso.contract(1, lm["K"], iso.VOCAB_CHUNK)
        lp1l = torch.empty_like(lp)
        run_l1 = lambda: iso.lmhead_logprob(H, Wv, tok, cl1, out=lp1l, workspace=wsl)
        run_l1()
        l1_ms = _time_events(run_l1, max(3, args.steps // 10), stream)
        tokl = tok.long().unsqueeze(1)

        def run_tl():
            z = torch.nn.functional.linear(H, Wv)
            return torch.log_softmax(z.float(), dim=-1).gather(1, tokl)
        run_tl()
        tl_ms = _time_events(run_tl, 3, stream)
        tlin = lambda: torch.nn.functional.linear(H, Wv)
        tlin()
        tlin_ms = _time_events(tlin, 3, stream)
        lp_t = run_tl().squeeze(1)
        torch.cuda.synchronize()
        extra["lmhead"].update({
            "one_leaf_ms": round(l1_ms, 4),
            "torch_linear_logsoftmax_gather_ms": round(tl_ms, 4),
            "torch_linear_only_ms": round(tlin_ms, 4),
            "invariance_overhead_vs_one_leaf": round(lm_ms / l1_ms - 1.0, 4),
            "invariance_overhead_vs_torch": round(lm_ms / tl_ms - 1.0, 4),
            "torch_bf16_logits_max_abs_diff": round(float((lp_t - lp_ref).abs().max()), 6)})
        del lp1l, lp_t
        extra["workspace_bytes"]["lmhead"] = iso.lmhead_workspace(cl, lm["M"], lm["V"], 1)
        lm_rows = np.sort(np.random.default_rng(2025).choice(lm["M"], 64, replace=False))
        c3_gpu = lp_ref[torch.from_numpy(lm_rows).to("cuda")].cpu().numpy()
        # the same layer split over 8 vocabulary shards (stats exchange + final tree)
        nch = (lm["V"] + 127) // 128
        st8 = torch.empty((lm["M"], nch, 2), dtype=torch.float32, device="cuda")
        tg8 = torch.empty(lm["M"], dtype=torch.float32, device="cuda")
        cuts = [round(i * nch / 8) * 128 for i in range(8)] + [lm["V"]]

        def run_sh():
            for i in range(8):
                iso.lmhead_shard_stats(H, Wv[cuts[i]:cuts[i + 1]], tok, cl, lm["V"], cuts[i],
                                       st8, tg8)
            return iso.lmhead_finish(st8, tg8, tok, lm["V"], out=lp8s)
        lp8s = torch.empty_like(lp_ref)
        run_sh()
        sh_ms = _time_events(run_sh, max(3, args.steps // 10), stream)
        ok &= bool(torch.equal(lp8s.view(torch.int32), lp_ref.view(torch.int32)))
        extra["lmhead"]["vocab_shards8_ms"] = round(sh_ms, 4)
        # decode: one row per call (weights streamed from HBM every step)
        lp1 = torch.empty(1, dtype=torch.float32, device="cuda")
        ws1 = torch.empty(iso.lmhead_workspace(cl, 1, lm["V"], 1), dtype=torch.uint8,
                          device="cuda")
        H1, tok1 = H[:1].contiguous(), tok[:1].contiguous()
        run_d = lambda: iso.lmhead_logprob(H1, Wv, tok1, cl, out=lp1, workspace=ws1)
        run_d()
        d_ms = _time_events(run_d, max(10, args.steps), stream)
        ok &= bool(torch.equal(lp1.view(torch.int32), lp_ref[:1].view(torch.int32)))
        gd = _time_graph(run_d, inner=10, reset=lp1.zero_,
                         check=lambda: torch.equal(lp1.view(torch.int32), lp_ref[:1].view(torch.int32)))
        ok &= bool(torch.equal(lp1.view(torch.int32), lp_ref[:1].view(torch.int32)))
        ok &= gd is None or gd == gd
        extra["decode"] = {"lmhead_1row_us": round(d_ms * 1e3, 2),
                           "lmhead_1row_weight_gbs": round(lm["V"] * lm["K"] * 2 / (d_ms * 1e-3) / 1e9, 1),
                           "lmhead_1row_graph_us": None if gd is None else round(gd * 1e3, 2)}
        del st8, tg8, lp8s, lp1, ws1
        del H, Wv, tok, lp, wsl

        # ---------------- MoE FFN block with the routing-order combine
        mc = make_config("moe")
        T, Hd, E, I, k = mc["T"], mc["H"], mc["E"], mc["I"], mc["top_k"]
        X = _dev(mc["X"])
        lgt = torch.from_numpy(mc["logits"]).to("cuda")
        Wg, Wu, Wd = _dev(mc["Wg"]), _dev(mc["Wu"]), _dev(mc["Wd"])
        cg = iso.contract(mc["leaves_gate_up"], Hd // mc["leaves_gate_up"], 0)
        cd = iso.contract(mc["leaves_down"], I // mc["leaves_down"], 0)
        y = torch.empty((T, Hd), dtype=torch.float32, device="cuda")
        wsm = torch.empty(iso.moe_workspace(T, Hd, E, I, k), dtype=torch.uint8, device="cuda")
        run_moe = lambda: iso.moe_combine(X, lgt, Wg, Wu, Wd, k, cg, cd, out=y, workspace=wsm)
        run_moe()
        moe_ms = _time_events(run_moe, max(3, args.steps // 5), stream)
        y_ref = y.clone()
        rev = torch.arange(T - 1, -1, -1, device="cuda")
        yr = torch.empty_like(y)
        iso.moe_combine(X[rev].contiguous(), lgt[rev].contiguous(), Wg, Wu, Wd, k, cg, cd, out=yr,
                        workspace=wsm)
        torch.cuda.synchronize()
        ok &= bool(torch.equal(yr.view(torch.int32), y_ref[rev].view(torch.int32)))
        moe_flop = 2.0 * T * k * (2 * Hd * I + I * Hd)
        # the cost of invariance: the same kernels with one accumulator per
        # output (one leaf over all of K), and a plain torch expert loop that
        # scatters with index_add_ (atomics: the usual non-invariant MoE)
        cg1 = iso.contract(1, Hd, 0)
        cd1 = iso.contract(1, I, 0)
        y1 = torch.empty_like(y)
        run_m1 = lambda: iso.moe_combine(X, lgt, Wg, Wu, Wd, k, cg1, cd1, out=y1, workspace=wsm)
        run_m1()
        m1_ms = _time_events(run_m1, max(3, args.steps // 5), stream)
        def run_mt():
            p_ = torch.softmax(lgt, dim=-1)
            gv, gi = torch.topk(p_, k, dim=-1)
            gv = (gv / gv.sum(dim=-1, keepdim=True)).reshape(-1)
            flat = gi.reshape(-1)
            order = torch.argsort(flat, stable=True)
            counts = torch.bincount(flat, minlength=E).tolist()
            yt = torch.zeros((T, Hd), dtype=torch.float32, device="cuda")
            off = 0
            for e in range(E):
                seg = order[off:off + counts[e]]
                off += counts[e]
                if seg.numel() == 0:
                    continue
                ts = seg // k
                xe = X[ts]
                g = torch.nn.functional.linear(xe, Wg[e])
                u = torch.nn.functional.linear(xe, Wu[e])
                oe = torch.nn.functional.linear(torch.nn.functional.silu(g) * u, Wd[e]).float()
                yt.index_add_(0, ts, oe * gv[seg].unsqueeze(1))
            return yt
        run_mt()
        mt_ms = _time_events(run_mt, 3, stream)
        extra["moe"] = {"shape": "4096 tokens, hidden 2048, 128 experts, top-8, SwiGLU 512, "
                                 "4 leaves (gate/up 4x512, down 4x128)",
                        "ms": round(moe_ms, 4),
                        "tokens_per_s": round(T / (moe_ms * 1e-3), 1),
                        "tflops": round(moe_flop / (moe_ms * 1e-3) / 1e12, 2),
                        "mfma_frac": round(moe_flop / (moe_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                        "one_leaf_ms": round(m1_ms, 4),
                        "torch_expert_loop_ms": round(mt_ms, 4),
                        "invariance_overhead_vs_one_leaf": round(moe_ms / m1_ms - 1.0, 4),
                        "invariance_overhead_vs_torch_loop": round(moe_ms / mt_ms - 1.0, 4)}
        extra["workspace_bytes"]["moe"] = iso.moe_workspace(T, Hd, E, I, k)
        del X, lgt, Wg, Wu, Wd, y, wsm, yr, y1

        # ---------------- RMSNorm with residual add in front of the LM-head
        Mn, Hn = 8192, 2048
        xn = _dev(normal_bf16(61, (Mn, Hn), 1.0))
        rn = _dev(normal_bf16(62, (Mn, Hn), 1.0))
        wn = _dev(normal_bf16(63, (Hn,), 1.0))
        cn = iso.contract(64, Hn // 64, 0, iso.SCHED_SEQ)
        yn = torch.empty((Mn, Hn), dtype=torch.bfloat16, device="cuda")
        ron = torch.empty_like(rn)
        run_n = lambda: iso.rmsnorm(xn, wn, cn, residual=rn, residual_out=ron, out=yn)
        run_n()
        n_ms = _time_events(run_n, max(10, args.steps), stream)
        y_ref = yn.clone()
        y1 = iso.rmsnorm(xn[4000:4001].contiguous(), wn, cn, residual=rn[4000:4001].contiguous())
        torch.cuda.synchronize()
        ok &= bool(torch.equal(y1.view(torch.int16), y_ref[4000:4001].view(torch.int16)))
        n_bytes = 4 * Mn * Hn * 2 + Hn * 2  # x, residual in; residual, y out; weight
        extra["rmsnorm"] = {"shape": "8192 x 2048, residual add, 64 leaves of 32, bf16 out",
                            "us": round(n_ms * 1e3, 2),
                            "gbs": round(n_bytes / (n_ms * 1e-3) / 1e9, 1),
                            "hbm_frac": round(n_bytes / (n_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        del xn, rn, wn, yn, ron, y_ref

        # ---------------- CPR gated delta rule: prefill and decode of one layer
        from iso_synth import cpr_inputs
        Tc, Hc, Dc, Cc = 4096, 16, 128, 64
        xc = cpr_inputs(Tc, Hc, Dc, seed=601)
        qc, kc, vc = _dev(xc["q"]), _dev(xc["k"]), _dev(xc["v"])
        alc = torch.from_numpy(xc["alpha"]).to("cuda")
        bec = torch.from_numpy(xc["beta"]).to("cuda")
        cc = iso.cpr_contract(Cc)
        wsc = torch.empty(iso.cpr_workspace(cc, Hc, Tc), dtype=torch.uint8, device="cuda")
        oc = torch.empty((Tc, Hc, Dc), dtype=torch.float32, device="cuda")
        snc = torch.empty((Hc, Dc, Dc), dtype=torch.float32, device="cuda")
        rnc = torch.empty_like(snc)
        run_c = lambda: iso.cpr_prefill(qc, kc, vc, alc, bec, cc, out=oc, snap=snc, run=rnc,
                                        workspace=wsc)
        run_c()
        c_ms = _time_events(run_c, max(5, args.steps // 5), stream)
        # decode of the last chunk (64 steps, the last one re-syncs) from a prefill of the rest
        T0 = Tc - Cc
        _, sd, rd = iso.cpr_prefill(qc[:T0], kc[:T0], vc[:T0], alc[:T0], bec[:T0], cc)
        wsd = torch.empty(iso.cpr_workspace(cc, Hc, Cc), dtype=torch.uint8, device="cuda")
        od = torch.empty((Cc, Hc, Dc), dtype=torch.float32, device="cuda")
        for p_ in range(T0, Tc):
            iso.cpr_decode_step(qc, kc, vc, alc, bec, p_, sd, rd, cc, out=od[p_ - T0], workspace=wsd)
        torch.cuda.synchronize()
        ok &= bool(torch.equal(od.view(torch.int32), oc[T0:].view(torch.int32)))
        ok &= bool(torch.equal(sd.view(torch.int32), snc.view(torch.int32)))
        ok &= bool(torch.equal(rd.view(torch.int32), rnc.view(torch.int32)))

        def dec_chunk():
            for p_ in range(T0, Tc):
                iso.cpr_decode_step(qc, kc, vc, alc, bec, p_, sd, rd, cc, out=od[p_ - T0],
                                    workspace=wsd)
        d_ms_p = _time_events(dec_chunk, 3, stream) / Cc
        # the same steps through the C ABI with their arguments marshalled
        # once (a step's kernel is shorter than the binding's per-call work)
        import ctypes
        dec_args = [(ctypes.byref(cc), qc.data_ptr(), kc.data_ptr(), vc.data_ptr(), alc.data_ptr(),
                     bec.data_ptr(), p_, sd.data_ptr(), rd.data_ptr(), od[p_ - T0].data_ptr(), Hc,
                     wsd.data_ptr(), wsd.numel(), stream.cuda_stream) for p_ in range(T0, Tc)]
        f_dec = iso.lib.iso_cpr_decode_step

        def dec_chunk_abi():
            for a_ in dec_args:
                if f_dec(*a_) != 0:
                    raise RuntimeError("iso_cpr_decode_step failed")
        d_ms = _time_events(dec_chunk_abi, 3, stream) / Cc
        # FP32 operations per token and head: step ~7 d^2, chunk form ~7 d^2,
        # boundary pass 2 d^3 / C (d = 128, C = 64)
        c_ops = Tc * Hc * (14.0 * Dc * Dc + 2.0 * Dc ** 3 / Cc)
        extra["cpr"] = {"shape": "16 heads of 128, 4096 tokens, chunk 64 (CPR gated delta rule)",
                        "prefill_ms": round(c_ms, 4),
                        "prefill_tokens_per_s": round(Tc / (c_ms * 1e-3), 1),
                        "decode_us_per_token": round(d_ms * 1e3, 2),
                        "decode_binding_us_per_token": round(d_ms_p * 1e3, 2),
                        "alu_tops": round(c_ops / (c_ms * 1e-3) / 1e12, 2),
                        "alu_frac": round(c_ops / (c_ms * 1e-3) / 1e12 / PEAK_FP32_OPS_T, 4)}
        del qc, kc, vc, alc, bec, wsc, oc, snc, rnc, sd, rd, wsd, od

    extra["bitwise_pass"] = ok
    line["bitwise_pass"] = ok
    line["sub"] = extra
    if not args.no_cpu_baseline:
        cb = _cpu_baseline(cfg)
        more, c3_oracle, rows_or = _cpu_more(cfg, lm, mc)
        assert np.array_equal(rows_or, lm_rows)
        cb["workloads"] = more
        line["cpu_baseline"] = cb
        extra["parity"] = _parity(cfg, c2_rows, c2_cols, c2_gpu, lm_rows, c3_gpu, c3_oracle)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
