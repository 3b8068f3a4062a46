"""Benchmark of the MXFP8 MoE expert grouped-GEMM hot path on one MI355X.

One step = one pass of the whole hot path of an expert linear over one batch:
  1. row-wise group quantize of X and the column-wise requantize of the
     result (saved for wgrad), one fused launch   [T, K]  bf16 -> MXFP8
  2. row + column-wise quantize of W         [G, N, K] bf16 -> MXFP8 (both copies)
  3. forward grouped GEMM (NT)               Y  [T, N] = X W_g^T
  4. row-wise group quantize of dY, its column-wise requantize and dbias,
     one fused launch                        [T, N], dbias [G, N]
  5. dgrad grouped GEMM (NN)                 dX [T, K] = dY W_g
  6. wgrad grouped GEMM (TN)                 dW [G, N, K] = dY_g^T X_g
Workload: 8 experts, hidden 4096 -> expert FFN 14336 (one linear), 16384
tokens routed by a seeded Dirichlet(1) multinomial (multiples of 128); X, dY
~ N(0, 1), W ~ N(0, 0.02) in bf16; fp32 GEMM outputs.  Inputs are resident in
HBM before the timed region.

value = 3 * 2 T N K / step time (TFLOP/s over the whole step, quantize
kernels included).  The timed steps run twice: as eager launches, each
bracketed by events (the per-launch times in kernel_ms, and
ms_per_step_eager), then replayed from a HIP graph of the same launches
(ms_per_step and value; --eager keeps the eager figure).  The grouped-GEMM roofline uses the GEMM launches' own
durations, measured with events on the stream they run on.

HBM traffic of the GEMM launches (roofline "traffic") comes from the FETCH_SIZE
and WRITE_SIZE counter summary under profiles/, scaled by the same counters
read on a plain device copy of known size (--calibrate-copy); it is reported
only while the GEMM source still hashes to the one the counters were taken on.

After the headline step, the other workloads of the same path are timed the
same way (fewer steps) and reported under "other_workloads": the skewed
128-expert linear (hidden 7168 -> 2048, 38 experts without tokens), the fused
expert MLP forward and backward (64 experts, 83968 tokens, 3072 -> 2048 ->
SwiGLU -> 1024 -> 3072, bf16 outputs) and the standalone row + column-wise
group quantize of 131072 x 7168.  Every wgrad launch passes a tile-counter
workspace (mxfp8_grouped_gemm_ws), with which the kernel hands out the wgrad
tiles dynamically unless 1 expert in 8 or more has no token.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-others]
       python bench.py --only NAME           (one of the other workloads alone)
       python bench.py --calibrate-copy      (copy of 1 GiB, for counter scaling)
       python bench.py --summarize trace|traffic|mfma|cache ...   (profiles/ tables from rocprofv3 CSVs)
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "moe8_h4096_f14336"
PEAK_MXFP8_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, 5.0 PFLOP/s
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
GEMM_SOURCE = "moe_expert_grouped_group_amd/csrc/gemm.hip"
QUANTIZE_SOURCE = "moe_expert_grouped_group_amd/csrc/quantize.hip"
COPY_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--eager", action="store_true",
                    help="time the steps as eager launches only (no graph replay)")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the other workloads (skewed 128-expert linear, fused MLP, "
                         "standalone group quantize)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 1 GiB three times (counter scaling)")
    ap.add_argument("--step-only", action="store_true",
                    help="time only the headline step (no launches outside it, no other "
                         "workloads, no CPU baseline): for per-step profiles")
    ap.add_argument("--only", choices=sorted(OTHERS),
                    help="time only this one of the other workloads and print its record "
                         "(for per-workload profiles)")
    return ap.parse_args()


def _source_files(rel):
    """`rel` and every local header it includes (#include "...", followed
    recursively), in a fixed order."""
    seen, order = set(), []

    def visit(path):
        path = os.path.normpath(path)
        if path in seen:
            return
        seen.add(path)
        order.append(path)
        with open(os.path.join(ROOT, path)) as f:
            for inc in re.findall(r'^\s*#include\s+"([^"]+)"', f.read(), re.M):
                visit(os.path.join(os.path.dirname(path), inc))

    visit(rel)
    return order


def _source_hash(rel):
    """sha256 of a kernel source and the local headers it includes, with
    comments and whitespace removed, so that only a change of the code itself
    retires the counters taken on it."""
    h = hashlib.sha256()
    for path in _source_files(rel):
        with open(os.path.join(ROOT, path)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(re.sub(r"\s+", "", text).encode())
    return h.hexdigest()


def gemm_source_hash():
    return _source_hash(GEMM_SOURCE)


def stored_traffic(workload, profiles_dir=None):
    """HBM bytes per GEMM launch from the counter summary, or None when the
    summary is missing or was taken on a different GEMM source."""
    path = os.path.join(profiles_dir or os.path.join(ROOT, "profiles"),
                        f"grouped_gemm_hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        m = re.search(r"```json\n(.*?)\n```", f.read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("source_sha256") != gemm_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def calibrate_copy():
    import torch
    torch.cuda.set_device(0)
    src = torch.full((COPY_BYTES,), 7, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": COPY_BYTES, "copies": 4,
                      "read_bytes_per_copy": COPY_BYTES, "write_bytes_per_copy": COPY_BYTES}),
          flush=True)


def cpu_baseline(w, budget_rows=4096, n_cols=2048):
    """Time the CPU oracle on a bounded sample of the same workload.

    Sample: the first `budget_rows` tokens, re-split as 8 experts of
    budget_rows / 8 = 512 rows each, the first `n_cols` output features of
    every expert's weight, the full hidden size; the same steps as the GPU
    step, each timed on its own.  Returns TFLOP/s of the three GEMMs over the
    oracle's whole wall time, the per-step seconds, the cores the process may
    run on (sched_getaffinity), the BLAS library and its thread count.
    """
    import numpy as np
    import threadpoolctl

    from oracle import gemm as og
    from oracle import mxfp8 as om

    g = w.groups
    rows = budget_rows
    splits = [rows // g] * g
    k = w.hidden
    x = w.tensors["x"][:rows].double().numpy()
    wt = w.tensors["w"][:, :n_cols, :].double().numpy().reshape(g * n_cols, k)
    dy = w.tensors["dy"][:rows, :n_cols].double().numpy()
    ops = {}

    def timed(name, fn):
        t0 = time.perf_counter()
        r = fn()
        ops[name] = round(time.perf_counter() - t0, 3)
        return r

    xq, xs = timed("quantize_x_rowwise", lambda: om.quantize_rowwise(x))
    wq, ws = timed("quantize_w_rowwise", lambda: om.quantize_rowwise(wt))
    wcq, wcs = timed("quantize_w_colwise", lambda: om.quantize_colwise(wt, [g * n_cols]))
    timed("fprop", lambda: og.fprop(xq, xs, wq.reshape(g, n_cols, k),
                                    ws.reshape(g, n_cols, k // 32), splits))
    xcq, xcs = timed("requant_x_colwise", lambda: om.requant_colwise(xq, xs, splits))
    dyq, dys = timed("quantize_dy_rowwise", lambda: om.quantize_rowwise(dy))
    timed("dgrad", lambda: og.dgrad(dyq, dys, wcq, wcs, splits, g))
    dycq, dycs = timed("requant_dy_colwise", lambda: om.requant_colwise(dyq, dys, splits))
    timed("dbias", lambda: om.grouped_dbias(dyq, dys, splits))
    timed("wgrad", lambda: og.wgrad(dycq, dycs, xcq, xcs, splits))
    dt = sum(ops.values())
    flops = 3 * 2.0 * rows * n_cols * k
    blas = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in blas] or [1])
    cores = len(os.sched_getaffinity(0))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(min(threads, cores)),
            "kind": "oracle",
            "sample": f"{WORKLOAD}: first {rows} tokens as {g} experts x {rows // g}, "
                      f"{n_cols} of {w.ffn} output features, K={k}; every step of the path; "
                      f"{dt:.2f} s wall, float64 NumPy",
            "affinity_cores": cores,
            "blas": {"library": blas[0].get("internal_api") if blas else None,
                     "version": blas[0].get("version") if blas else None,
                     "threads": int(threads)},
            "seconds_per_op": ops,
            "note": "GEMMs use the multithreaded BLAS; quantize and requantize are vectorized "
                    "NumPy on one thread; `cores` = the threads the BLAS used, bounded by the "
                    "affinity mask"}


def _time_outside(fn, steps):
    """Mean time (ms) of `fn` over max(steps, 3) launches after two warmups."""
    import numpy as np
    import torch

    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    pairs = []
    for _ in range(max(steps, 3)):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        pairs.append((a, b))
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in pairs]))


def _run_steps(launches, steps, warmup):
    """Time a step made of named launches: warmup steps, then `steps` steps
    between two events; every launch also bracketed by its own events.
    Returns (ms per step, {name: mean ms per launch})."""
    import numpy as np
    import torch

    ev = {}

    def step():
        for name, fn in launches:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            ev.setdefault(name, []).append((a, b))

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev.clear()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    per = {nm: float(np.mean([a.elapsed_time(b) for a, b in pairs])) for nm, pairs in ev.items()}
    return start.elapsed_time(stop) / steps, per


def vendor_reference(m, n, k, steps):
    """The vendor BLAS (hipBLASLt, through torch._scaled_mm) on one dense
    GEMM with the flops of one grouped launch of the headline workload
    (M = all tokens, N, K): MXFP8 with E8M0 block scales, and FP8 with one
    scale per tensor.  Context for the grouped kernel's rate, not part of
    the path; an entry holds the error text where the installed torch lacks a form."""
    import torch
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    a = (torch.randn(m, k, device=dev, generator=gen) * 0.5).to(torch.float8_e4m3fn)
    b = (torch.randn(n, k, device=dev, generator=gen) * 0.5).to(torch.float8_e4m3fn)
    flops = 2.0 * m * n * k
    out = {"shape": [m, n, k], "library": "hipBLASLt via torch._scaled_mm"}

    def run(name, fn):
        try:
            ms = _time_outside(fn, steps)
            out[name] = {"ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}
        except Exception as e:  # noqa: BLE001 - reported, not raised
            out[name] = f"unavailable: {type(e).__name__}: {str(e)[:160]}"

    e8m0 = getattr(torch, "float8_e8m0fnu", None)
    if e8m0 is not None:
        sa = torch.full((m, k // 32), 127, dtype=torch.uint8, device=dev).view(e8m0)
        sb = torch.full((n, k // 32), 127, dtype=torch.uint8, device=dev).view(e8m0)
        run("mxfp8_bf16_out", lambda: torch._scaled_mm(a, b.t(), scale_a=sa, scale_b=sb,
                                                        out_dtype=torch.bfloat16))
        del sa, sb
    one = torch.ones((), device=dev)
    run("fp8_per_tensor_fp32_out", lambda: torch._scaled_mm(a, b.t(), scale_a=one, scale_b=one,
                                                            out_dtype=torch.float32))
    del a, b
    torch.cuda.empty_cache()
    return out


def _gemm_roofline_ms(flops, bytes_):
    """Time bound of one GEMM launch: the larger of its flops at the MFMA peak
    and its algorithmic bytes at the HBM peak."""
    return max(flops / (PEAK_MXFP8_TFLOPS * 1e12), bytes_ / (PEAK_HBM_GBS * 1e9)) * 1e3


def bench_skewed_linear(steps, warmup):
    """128 experts (38 without tokens), hidden 7168 -> 2048, 32768 tokens, X
    with 0.1 % outliers x1000, fp32 outputs.  X arrives row-wise quantized
    (its quantize is not in the step); the weight is quantized in the step."""
    import torch

    import moe_expert_grouped_group_amd as mx
    from moe_expert_grouped_group_amd import workloads as wl

    w = wl.make("skewed_dsv3")
    g, t, k, n = w.groups, w.tokens, w.hidden, w.ffn
    ms = torch.from_numpy(w.m_splits).cuda()
    x, wt, dy = (w.tensors[nm].cuda() for nm in ("x", "w", "dy"))
    xo = mx.group_quantize(x, mx.ROWWISE)
    wo = mx.group_quantize(wt, mx.ROWWISE | mx.COLWISE)
    xc = mx.requant_colwise(xo.row_data, xo.row_scale)
    dyo, db = mx.group_quantize_requant(dy, ms, with_dbias=True)
    dyc = dyo
    f32 = torch.float32
    y = torch.empty(t, n, dtype=f32, device="cuda")
    dx = torch.empty(t, k, dtype=f32, device="cuda")
    dw = torch.empty(g, n, k, dtype=f32, device="cuda")
    ws = torch.empty(mx.dbias_workspace_bytes(t, n), dtype=torch.uint8, device="cuda")
    gws = torch.empty(mx.gemm_workspace_bytes(), dtype=torch.uint8, device="cuda")
    launches = [
        ("quant_w", lambda: mx.group_quantize(wt, mx.ROWWISE | mx.COLWISE, out=wo)),
        ("gemm_fprop", lambda: mx.grouped_gemm("NT", xo.row_data, xo.row_scale, wo.row_data,
                                               wo.row_scale, ms, t, n, k, f32, y)),
        ("requant_x", lambda: mx.requant_colwise(xo.row_data, xo.row_scale, out=xc)),
        ("quant_requant_dy_dbias", lambda: mx.group_quantize_requant(
            dy, ms, with_dbias=True, out=dyo, dbias=db, workspace=ws)),
        ("gemm_dgrad", lambda: mx.grouped_gemm("NN", dyo.row_data, dyo.row_scale, wo.col_data,
                                               wo.col_scale, ms, t, n, k, f32, dx)),
        ("gemm_wgrad", lambda: mx.grouped_gemm("TN", dyc.col_data, dyc.col_scale, xc.col_data,
                                               xc.col_scale, ms, t, n, k, f32, dw,
                                               workspace=gws)),
    ]
    ms_step, per = _run_steps(launches, steps, warmup)
    flop = 2.0 * t * n * k
    busy = int((w.m_splits > 0).sum())
    sc = 1 + 1 / 32
    # algorithmic bytes: A and B (experts with tokens) codes + scales, C once
    gbytes = {"gemm_fprop": t * k * sc + busy * n * k * sc + t * n * 4,
              "gemm_dgrad": t * n * sc + busy * n * k * sc + t * k * 4,
              "gemm_wgrad": t * n * sc + t * k * sc + g * n * k * 4}
    gemm_ms = sum(per[nm] for nm in gbytes)
    bound_ms = sum(_gemm_roofline_ms(flop, b) for b in gbytes.values())
    return {
        "experts": g, "empty_experts": int((w.m_splits == 0).sum()), "tokens": t, "hidden": k,
        "ffn": n, "out_dtype": "f32", "ms_per_step": round(ms_step, 4),
        "tflops_step": round(3 * flop / (ms_step * 1e-3) / 1e12, 2),
        "gemm_tflops": round(3 * flop / (gemm_ms * 1e-3) / 1e12, 2),
        "gemm_roofline_frac": round(bound_ms / gemm_ms, 4),
        "kernel_ms": {nm: round(v, 4) for nm, v in per.items()},
        "note": "X pre-quantized row-wise (not in the step); gemm_roofline_frac = sum over the "
                "three GEMMs of max(flops / MFMA peak, algorithmic bytes / HBM peak) over their "
                "measured time (the fp32 wgrad output makes it HBM-bound)",
    }


def bench_fused_mlp(steps, warmup):
    """Fused expert MLP, forward and backward: 64 experts, 83968 tokens,
    hidden 3072, FC1 3072 -> 2048 (gate | up), SwiGLU to 1024, FC2 1024 ->
    3072, bf16 GEMM outputs; only column-wise copies of X and of the SwiGLU
    output are kept for the backward."""
    import torch

    import moe_expert_grouped_group_amd as mx
    from moe_expert_grouped_group_amd import workloads as wl

    w = wl.make("nemotron_proxy_mlp")
    g, t, k, n2 = w.groups, w.tokens, w.hidden, w.ffn
    f = n2 // 2
    ms = torch.from_numpy(w.m_splits).cuda()
    x, w1, w2, dout = (w.tensors[nm].cuda() for nm in ("x", "w", "w2", "dy"))
    del w
    bf = torch.bfloat16
    R, C = mx.ROWWISE, mx.COLWISE
    xo = mx.group_quantize_requant(x)
    xc = xo
    w1o = mx.group_quantize(w1, R | C)
    w2o = mx.group_quantize(w2, R | C)
    h = torch.empty(t, n2, dtype=bf, device="cuda")
    ao = mx.swiglu_quantize(torch.zeros(t, n2, dtype=bf, device="cuda"), R | C)
    y = torch.empty(t, k, dtype=bf, device="cuda")
    dyo = mx.group_quantize_requant(dout)
    dyc = dyo
    da = torch.empty(t, f, dtype=bf, device="cuda")
    dw2 = torch.empty(g, k, f, dtype=bf, device="cuda")
    dho, db1 = mx.group_quantize_requant(torch.zeros(t, n2, dtype=bf, device="cuda"), ms,
                                         with_dbias=True)
    dhc = dho
    dx = torch.empty(t, k, dtype=bf, device="cuda")
    dw1 = torch.empty(g, n2, k, dtype=bf, device="cuda")
    ws = torch.empty(mx.dbias_workspace_bytes(t, n2), dtype=torch.uint8, device="cuda")
    gws = torch.empty(mx.gemm_workspace_bytes(), dtype=torch.uint8, device="cuda")
    gemm = mx.grouped_gemm
    launches = [
        ("quant_requant_x", lambda: mx.group_quantize_requant(x, out=xo)),
        ("quant_w1", lambda: mx.group_quantize(w1, R | C, out=w1o)),
        ("quant_w2", lambda: mx.group_quantize(w2, R | C, out=w2o)),
        # FC1 with the SwiGLU + quantize in its epilogue: h for the backward
        # and both MXFP8 copies of a = silu(gate) * up for FC2, one launch
        ("fc1_swiglu_quant", lambda: mx.grouped_gemm_swiglu_quantize(
            xo.row_data, xo.row_scale, w1o.row_data, w1o.row_scale, ms, t, f, k, h=h, out=ao)),
        ("fc2_fprop", lambda: gemm("NT", ao.row_data, ao.row_scale, w2o.row_data, w2o.row_scale,
                                   ms, t, k, f, bf, y)),
        ("quant_requant_dy", lambda: mx.group_quantize_requant(dout, out=dyo)),
        ("fc2_dgrad", lambda: gemm("NN", dyo.row_data, dyo.row_scale, w2o.col_data,
                                   w2o.col_scale, ms, t, k, f, bf, da)),
        ("fc2_wgrad", lambda: gemm("TN", dyc.col_data, dyc.col_scale, ao.col_data, ao.col_scale,
                                   ms, t, k, f, bf, dw2, workspace=gws)),
        # the SwiGLU backward fused with the quantize + requantize (+ dbias)
        # of dh for the FC1 backward: dh itself is never written
        ("swiglu_bwd_quant_dbias", lambda: mx.swiglu_bwd_quantize(
            h, da, ms, with_dbias=True, out=dho, dbias=db1, workspace=ws)),
        ("fc1_dgrad", lambda: gemm("NN", dho.row_data, dho.row_scale, w1o.col_data,
                                   w1o.col_scale, ms, t, n2, k, bf, dx)),
        ("fc1_wgrad", lambda: gemm("TN", dhc.col_data, dhc.col_scale, xc.col_data, xc.col_scale,
                                   ms, t, n2, k, bf, dw1, workspace=gws)),
    ]
    ms_step, per = _run_steps(launches, steps, warmup)
    flops = 3 * 2.0 * t * k * n2 + 3 * 2.0 * t * f * k
    gemm_ms = sum(v for nm, v in per.items() if nm.startswith("fc"))
    return {
        "experts": g, "empty_experts": int((ms == 0).sum().item()), "tokens": t, "hidden": k,
        "fc1_out": n2, "fc2_in": f, "out_dtype": "bf16", "tflop_per_step": round(flops / 1e12, 4),
        "ms_per_step": round(ms_step, 4),
        "tflops_step": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "gemm_tflops": round(flops / (gemm_ms * 1e-3) / 1e12, 2),
        "gemm_frac_of_peak": round(flops / (gemm_ms * 1e-3) / 1e12 / PEAK_MXFP8_TFLOPS, 4),
        "kernel_ms": {nm: round(v, 4) for nm, v in per.items()},
        "note": "fc1_swiglu_quant is FC1 with the SwiGLU + row/column MXFP8 quantize in its "
                "epilogue (mxfp8_grouped_gemm_swiglu_quantize); the GEMM time includes it",
    }


def bench_fc1_swiglu(steps, warmup):
    """FC1 of the fused MLP (83968 tokens, 3072 -> 2 x 1024, 64 experts) as
    one launch with the SwiGLU + quantize epilogue, against the two launches
    it replaces (the bf16 FC1 GEMM, then swiglu_quantize of its output)."""
    import torch

    import moe_expert_grouped_group_amd as mx
    from moe_expert_grouped_group_amd import workloads as wl

    del warmup
    w = wl.make("nemotron_proxy_mlp")
    t, k, n2 = w.tokens, w.hidden, w.ffn
    f = n2 // 2
    ms = torch.from_numpy(w.m_splits).cuda()
    R, C = mx.ROWWISE, mx.COLWISE
    xo = mx.group_quantize(w.tensors["x"].cuda(), R)
    w1o = mx.group_quantize(w.tensors["w"].cuda(), R | C)
    del w
    h = torch.empty(t, n2, dtype=torch.bfloat16, device="cuda")
    ao = mx.swiglu_quantize(torch.zeros_like(h), R | C)
    fc1 = lambda: mx.grouped_gemm("NT", xo.row_data, xo.row_scale, w1o.row_data,  # noqa: E731
                                  w1o.row_scale, ms, t, n2, k, torch.bfloat16, h)
    sq = lambda: mx.swiglu_quantize(h, R | C, out=ao)  # noqa: E731
    fused = lambda: mx.grouped_gemm_swiglu_quantize(  # noqa: E731
        xo.row_data, xo.row_scale, w1o.row_data, w1o.row_scale, ms, t, f, k, h=h, out=ao)
    fc1_ms = _time_outside(fc1, steps)
    sq_ms = _time_outside(sq, steps)
    fused_ms = _time_outside(fused, steps)
    return {"tokens": t, "hidden": k, "fc1_out": n2, "fc1_ms": round(fc1_ms, 4),
            "swiglu_quant_ms": round(sq_ms, 4), "unfused_ms": round(fc1_ms + sq_ms, 4),
            "fused_ms": round(fused_ms, 4),
            "note": "same h and MXFP8 bytes either way (tests); the fused MLP step uses the "
                    "fused launch"}


def bench_swiglu_bwd_quant(steps, warmup):
    """The fused MLP's SwiGLU backward (83968 tokens, F = 1024, 64 experts)
    fused with the row-wise quantize, column-wise requantize and dbias of its
    output dh, against the two launches it replaces (swiglu_bwd, then
    group_quantize_requant of dh with dbias)."""
    import torch

    import moe_expert_grouped_group_amd as mx
    from moe_expert_grouped_group_amd import workloads as wl

    del warmup
    name = "nemotron_proxy_mlp"
    splits = wl.splits_for(name)
    t, f = int(splits.sum()), wl.make(name, parts=set()).ffn // 2
    ms = torch.from_numpy(splits).cuda()
    gen = torch.Generator(device="cuda").manual_seed(7)
    bf = torch.bfloat16
    h = (torch.randn(t, 2 * f, device="cuda", generator=gen) * 3).to(bf)
    da = torch.randn(t, f, device="cuda", generator=gen).to(bf)
    dh = torch.empty_like(h)
    out, db = mx.group_quantize_requant(dh.zero_(), ms, with_dbias=True)
    ws = torch.empty(mx.dbias_workspace_bytes(t, 2 * f), dtype=torch.uint8, device="cuda")
    bwd = lambda: mx.swiglu_bwd(h, da, out=dh)  # noqa: E731
    qr = lambda: mx.group_quantize_requant(dh, ms, with_dbias=True, out=out,  # noqa: E731
                                           dbias=db, workspace=ws)
    fused = lambda: mx.swiglu_bwd_quantize(h, da, ms, with_dbias=True, out=out,  # noqa: E731
                                           dbias=db, workspace=ws)
    bwd_ms = _time_outside(bwd, steps)
    qr_ms = _time_outside(qr, steps)
    fused_ms = _time_outside(fused, steps)
    nbytes = t * 2 * f * 2 + t * f * 2 + 2 * t * 2 * f * (1 + 1 / 32)
    return {"tokens": t, "ffn": f, "swiglu_bwd_ms": round(bwd_ms, 4),
            "quant_requant_dbias_ms": round(qr_ms, 4), "unfused_ms": round(bwd_ms + qr_ms, 4),
            "fused_ms": round(fused_ms, 4),
            "fused_gbs": round(nbytes / (fused_ms * 1e-3) / 1e9, 1),
            "note": "same MXFP8 bytes and dbias bits either way (tests); the fused MLP step uses "
                    "the fused launch; fused_gbs counts h and da read, both MXFP8 copies written"}


def bench_group_quantize(steps, warmup):
    """Standalone row + column-wise group quantize of a 131072 x 7168 bf16
    tensor (256 experts, Student-t(3) values, 1 % zero tiles)."""
    import torch

    import moe_expert_grouped_group_amd as mx
    from moe_expert_grouped_group_amd import workloads as wl

    w = wl.make("group_quantize_131072x7168")
    t, k = w.tokens, w.hidden
    x = w.tensors["x"].cuda()
    del w
    out = mx.group_quantize(x, mx.ROWWISE | mx.COLWISE)
    ms_step, per = _run_steps(
        [("quant_rowcol", lambda: mx.group_quantize(x, mx.ROWWISE | mx.COLWISE, out=out))],
        steps, warmup)
    nbytes = t * k * (2 + 2 * (1 + 1 / 32))
    gbs = nbytes / (per["quant_rowcol"] * 1e-3) / 1e9
    return {"tokens": t, "hidden": k, "experts": 256, "ms": round(per["quant_rowcol"], 4),
            "algorithmic_bytes": int(nbytes), "gbs": round(gbs, 1),
            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}


OTHERS = {}   # filled below: name -> bench function of the other workloads


# ---------------------------------------------------------------------------
# rocprofv3 summaries: the tables under profiles/ are written by these from the
# CSV output of the commands they quote (python bench.py --summarize ...).

def _csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _short_kernel(name):
    """'void mx::quant_rowcol_kernel<true>(...)' -> 'quant_rowcol_kernel<true>'."""
    n = name.replace("void ", "")
    n = n.split("(")[0]
    return n.replace("mx::", "")


def _labels(names, cycles=None):
    """Launch labels in dispatch order: the grouped GEMM's instantiations by
    layout (<false, *, false> alternates forward and dgrad, as every step
    launches them in that order), every other kernel by its short name.
    `cycles` maps a short kernel name to the names its successive launches
    take in turn (a step that launches one kernel for several purposes)."""
    out, mgrouped, seen = [], {}, {}
    for n in names:
        k = _short_kernel(n)
        if cycles and k in cycles:
            i = seen.get(k, 0)
            seen[k] = i + 1
            out.append(cycles[k][i % len(cycles[k])])
        elif k.startswith("grouped_gemm_kernel<"):
            targs = [a.strip() == "true" for a in k[k.index("<") + 1:k.rindex(">")].split(",")]
            kg, bf, acc = targs[:3]
            dt = "_bf16" if bf else ""
            if len(targs) > 3 and targs[3]:
                out.append("forward_NT_swiglu_quantize")
            elif acc:
                out.append("wgrad_accumulate_TN")
            elif kg:
                out.append("wgrad_TN" + dt)
            else:
                i = mgrouped.get(dt, 0)
                mgrouped[dt] = i + 1
                out.append(("forward_NT" if i % 2 == 0 else "dgrad_NN") + dt)
        else:
            out.append(k)
    return out


def algorithmic_bytes(workload):
    """Algorithmic HBM bytes per launch of each kernel of a workload's step:
    codes and scales (1/32 of the codes) read or written once, fp32 outputs
    and partials once."""
    from moe_expert_grouped_group_amd import workloads as wl
    sc = 1 + 1 / 32
    if workload == "group_quantize_131072x7168":
        t, k = 131072, 7168
        return {"quant_rowcol_kernel": t * k * (2 + 2 * sc)}
    g, t = len(wl.splits_for(workload)), int(wl.splits_for(workload).sum())
    if workload == "nemotron_proxy_mlp":
        k, n2, f = 3072, 2048, 1024
        return {
            "fc1_fprop": t * k * sc + g * n2 * k * sc + t * n2 * 2,
            # FC1 with the SwiGLU + quantize epilogue: h and both copies of a
            "fc1_swiglu_quant": t * k * sc + g * n2 * k * sc + t * n2 * 2 + 2 * t * f * sc,
            "fc2_fprop": t * f * sc + g * k * f * sc + t * k * 2,
            "fc2_dgrad": t * k * sc + g * k * f * sc + t * f * 2,
            "fc1_dgrad": t * n2 * sc + g * n2 * k * sc + t * k * 2,
            "fc2_wgrad": t * k * sc + t * f * sc + g * k * f * 2,
            "fc1_wgrad": t * n2 * sc + t * k * sc + g * n2 * k * 2,
        }
    k, n = {"moe8_h4096_f14336": (4096, 14336)}[workload]
    return {
        "forward_NT": t * k * sc + g * n * k * sc + t * n * 4,
        "dgrad_NN": t * n * sc + g * n * k * sc + t * k * 4,
        "wgrad_TN": t * n * sc + t * k * sc + g * n * k * 4,
        "wgrad_accumulate_TN": t * n * sc + t * k * sc + 2 * g * n * k * 4,
        "quant_row_requant_kernel<false>": t * k * (2 + 2 * sc),
        "quant_row_requant_kernel<true>": t * n * (2 + 2 * sc) + (t // 128) * n * 4,
        "quant_rowcol_kernel": g * n * k * (2 + 2 * sc),
        "dbias_finalize_kernel": (t // 128) * n * 4 + g * n * 4,
    }


def _counter_means(path, cycles=None):
    """Mean counter value and duration (us) per launch label of a --pmc CSV."""
    import collections
    rows = _csv(path)
    labels = _labels([r["Kernel_Name"] for r in rows], cycles)
    vals, durs = collections.defaultdict(list), collections.defaultdict(list)
    for r, lab in zip(rows, labels):
        vals[lab].append(float(r["Counter_Value"]))
        durs[lab].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return ({k: sum(v) / len(v) for k, v in vals.items()},
            {k: len(v) for k, v in vals.items()},
            {k: sum(v) / len(v) for k, v in durs.items()})


def summarize_traffic(workload, cal_fetch, cal_write, fetch, write, title, commands, cycles=None):
    """Markdown + JSON of HBM bytes per launch from FETCH_SIZE and WRITE_SIZE
    runs, scaled by the same counters on the 1 GiB copy of --calibrate-copy."""
    cf, _, _ = _counter_means(os.path.join(cal_fetch, "p_counter_collection.csv"))
    cw, _, _ = _counter_means(os.path.join(cal_write, "p_counter_collection.csv"))
    copy = [k for k in cf if "copyBuffer" in k][0]
    ff = round(COPY_BYTES / 1024 / cf[copy], 4)
    fw = round(COPY_BYTES / 1024 / cw[copy], 4)
    f, nf, df = _counter_means(os.path.join(fetch, "p_counter_collection.csv"), cycles)
    w, _, _ = _counter_means(os.path.join(write, "p_counter_collection.csv"), cycles)
    alg = algorithmic_bytes(workload)
    per, tab = {}, []
    for lab in sorted(f, key=lambda x: (x not in alg, x)):
        if lab not in w:
            continue
        rd, wr = f[lab] * 1024 * ff, w[lab] * 1024 * fw
        a = alg.get(lab)
        per[lab] = {"fetch_kib": round(f[lab], 1), "write_kib": round(w[lab], 1),
                    "read_bytes": int(rd), "write_bytes": int(wr), "hbm_bytes": int(rd + wr),
                    "algorithmic_bytes": None if a is None else int(a), "launches": nf[lab],
                    "us_under_counters": round(df[lab], 1)}
        tab.append(f"| {lab} | {nf[lab]} | {f[lab]:.0f} | {w[lab]:.0f} | {rd / 1e9:.3f} | "
                   f"{wr / 1e9:.3f} | " + (f"{a / 1e9:.3f} | {(rd + wr) / a:.2f}" if a else "- | -")
                   + f" | {df[lab]:.1f} |")
    step3 = [per[x]["hbm_bytes"] for x in ("forward_NT", "dgrad_NN", "wgrad_TN") if x in per]
    rec = {"workload": workload, "source_sha256": gemm_source_hash(),
           "quantize_source_sha256": quantize_source_hash(),
           "copy_fetch_factor": ff, "copy_write_factor": fw, "per_launch": per}
    if len(step3) == 3:
        rec["hbm_bytes_per_launch"] = int(sum(step3) / 3)
    cmd = "\n".join(commands)
    md = f"""# {title}

Counters, each in a run of its own (from the repository root, one MI355X):

```
{cmd}
```

Calibration: the 1 GiB device copy of `bench.py --calibrate-copy` reads {cf[copy]:.0f} KiB by FETCH_SIZE and writes {cw[copy]:.0f} KiB by WRITE_SIZE per copy, so the counters are scaled by {ff} (fetch) and {fw} (write).

| launch | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | read GB (scaled) | written GB (scaled) | algorithmic GB | ratio | us per launch under counters |
|---|---|---|---|---|---|---|---|---|
""" + "\n".join(tab) + f"""

Algorithmic bytes: codes and E8M0 scales read or written once, fp32 outputs and partial sums once (the accumulating wgrad also reads its output).  FETCH_SIZE counts reads from L2 to the memory fabric (Infinity Cache hits included), so a ratio above 1 is re-fetch of data that fell out of L2, or partial lines written back piecemeal.  Durations under counter collection are longer than bench.py's event times.  Written by `python bench.py --summarize traffic ...` from the runs above.

```json
{json.dumps(rec, indent=1)}
```
"""
    return md


def summarize_trace(trace_dir, title, commands, note="", cycles=None):
    """Markdown table of a --kernel-trace run: per launch label (the GEMM by
    layout, in dispatch order), calls, mean / min / max duration and total."""
    import collections
    path = [os.path.join(trace_dir, x) for x in os.listdir(trace_dir)
            if x.endswith("kernel_trace.csv")][0]
    rows = _csv(path)
    labels = _labels([r["Kernel_Name"] for r in rows], cycles)
    d = collections.defaultdict(list)
    for r, lab in zip(rows, labels):
        d[lab].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in d.values())
    tab = ["| launch | calls | avg us | median us | min us | max us | total ms | % |",
           "|---|---|---|---|---|---|---|---|"]
    for lab, v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
        sv = sorted(v)
        tab.append(f"| `{lab}` | {len(v)} | {sum(v) / len(v):.1f} | {sv[len(sv) // 2]:.1f} | "
                   f"{sv[0]:.1f} | {sv[-1]:.1f} | {sum(v) / 1e3:.3f} | "
                   f"{100 * sum(v) / total:.1f} |")
    cmd = "\n".join(commands)
    return f"""# {title}

Command (from the repository root, one MI355X):

```
{cmd}
```

From `{os.path.basename(path)}`, one row per launch label: the grouped GEMM's forward (`forward_NT`) and dgrad (`dgrad_NN`) are the two launches of `grouped_gemm_kernel<false, *, false>` in dispatch order, `wgrad_TN` is `<true, *, false>`, `wgrad_accumulate_TN` is `<true, false, true>`; a `_bf16` suffix marks bf16 outputs.""" + ("" if not cycles else "  Kernels launched for several purposes per step are named in launch order: " + "; ".join(f"`{k}` = {', '.join(v)}" for k, v in cycles.items()) + ".") + """  Written by `python bench.py --summarize trace ...`.

""" + "\n".join(tab) + ("\n\n" + note if note else "") + "\n"


def summarize_mfma(pmc_dir, title, commands, cycles=None):
    """Markdown of a --pmc run with GRBM_GUI_ACTIVE, SQ_VALU_MFMA_BUSY_CYCLES
    and SQ_INSTS_VALU_MFMA_MOPS_F8: per launch label the duration, the mean
    shader clock (active cycles of one XCD over the duration), the matrix
    cores' busy fraction of the active SIMD cycles, and the F8 MFMA work."""
    import collections
    import statistics as st
    rows = _csv(os.path.join(pmc_dir, "p_counter_collection.csv"))
    by = collections.OrderedDict()
    for r in rows:
        d = by.setdefault(int(r["Dispatch_Id"]), {
            "name": r["Kernel_Name"],
            "dur": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    labels = _labels([d["name"] for d in by.values()], cycles)
    agg = collections.defaultdict(list)
    for d, lab in zip(by.values(), labels):
        gui = d["GRBM_GUI_ACTIVE"] / 8          # summed over the 8 XCDs
        agg[lab].append((d["dur"] / 1e3, gui / d["dur"],
                         d["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * 1024),
                         d["SQ_INSTS_VALU_MFMA_MOPS_F8"] * 512 / 1e12))
    tab = ["| launch | launches | duration us (mean) | clock GHz (active cycles / duration) | "
           "MFMA busy (of active SIMD cycles) | F8 MFMA work, TFLOP |", "|---|---|---|---|---|---|"]
    for lab, v in agg.items():
        m = lambda i: st.mean(x[i] for x in v)  # noqa: E731
        tab.append(f"| {lab} | {len(v)} | {m(0):.0f} | {m(1):.2f} (range "
                   f"{min(x[1] for x in v):.2f}-{max(x[1] for x in v):.2f}) | {100 * m(2):.1f} % | "
                   f"{m(3):.3f} |")
    cmd = "\n".join(commands)
    return f"""# {title}

Command (from the repository root, one MI355X; one run, every counter in it within the hardware's per-block limits):

```
{cmd}
```

""" + "\n".join(tab) + """

Per launch: GRBM_GUI_ACTIVE is summed over the 8 XCDs, so divided by 8 and by the launch's duration (its timestamps in the same CSV) it is the mean shader clock; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (active cycles x 1024 SIMDs); F8 MFMA work = SQ_INSTS_VALU_MFMA_MOPS_F8 x 512 (the counter's unit is 512 multiply-adds; the scaled FP8 MFMA counts as F8).  Durations are longer than bench.py's event times (counter collection serialises the launches).  Written by `python bench.py --summarize mfma ...`.
"""


def summarize_cache(pmc_dirs, title, commands, cycles=None):
    """Markdown of --pmc runs (one directory each; launches matched by label
    in dispatch order) with TCC_HIT_sum / TCC_MISS_sum, TCC_EA0_RDREQ_sum /
    TCC_EA0_RDREQ_LEVEL_sum, SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES and TA_BUSY_avr
    / GRBM_GUI_ACTIVE: per launch label the L2 hit rate, the mean latency of
    the reads that miss L2 (Little's law: outstanding requests summed per
    cycle over requests), the share of wave cycles spent waiting, and the
    texture-address unit's busy share."""
    import collections
    import statistics as st
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for d in pmc_dirs:
        rows = _csv(os.path.join(d, "p_counter_collection.csv"))
        by = collections.OrderedDict()
        for r in rows:
            e = by.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]})
            e[r["Counter_Name"]] = float(r["Counter_Value"])
        labels = _labels([e["name"] for e in by.values()], cycles)
        for e, lab in zip(by.values(), labels):
            if "TCC_HIT_sum" in e:
                per[lab]["hit"].append(e["TCC_HIT_sum"] / (e["TCC_HIT_sum"] + e["TCC_MISS_sum"]))
            if "TCC_EA0_RDREQ_sum" in e and e["TCC_EA0_RDREQ_sum"] > 0:
                per[lab]["lat"].append(e["TCC_EA0_RDREQ_LEVEL_sum"] / e["TCC_EA0_RDREQ_sum"])
            if "SQ_WAVE_CYCLES" in e:
                per[lab]["wait"].append(e["SQ_WAIT_INST_ANY"] / e["SQ_WAVE_CYCLES"])
            if "TA_BUSY_avr" in e:
                per[lab]["ta"].append(e["TA_BUSY_avr"] / (e["GRBM_GUI_ACTIVE"] / 8))
    f = lambda v, fmt: "-" if not v else fmt.format(st.mean(v))  # noqa: E731
    tab = ["| launch | L2 hit rate | mean latency of L2-miss reads, cycles | wave cycles "
           "waiting | address unit busy |", "|---|---|---|---|---|"]
    for lab, v in per.items():
        tab.append(f"| {lab} | {f([100 * x for x in v['hit']], '{:.0f} %')} | "
                   f"{f(v['lat'], '{:.0f}')} | {f([100 * x for x in v['wait']], '{:.0f} %')} | "
                   f"{f([100 * x for x in v['ta']], '{:.0f} %')} |")
    cmd = "\n".join(commands)
    return f"""# {title}

Counters, each group in a run of its own (from the repository root, one MI355X):

```
{cmd}
```

""" + "\n".join(tab) + """

Per launch label (mean over its launches): L2 hit rate = TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum); mean latency of the reads that miss L2 = TCC_EA0_RDREQ_LEVEL_sum / TCC_EA0_RDREQ_sum (the outstanding read requests of the L2 to the memory fabric, summed per cycle, over the requests: Little's law, in L2 cycles); wave cycles waiting = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (waits on memory counters and barriers); address unit busy = TA_BUSY_avr over the active cycles of one XCD (GRBM_GUI_ACTIVE / 8).  Written by `python bench.py --summarize cache ...`.
"""


def quantize_source_hash():
    return _source_hash(QUANTIZE_SOURCE)


def summarize_main(argv):
    ap = argparse.ArgumentParser(prog="bench.py --summarize")
    ap.add_argument("kind", choices=["trace", "traffic", "mfma", "cache"])
    ap.add_argument("--out", required=True, help="markdown file to write")
    ap.add_argument("--title", required=True)
    ap.add_argument("--command", action="append", default=[],
                    help="the rocprofv3 command line(s) the CSVs came from (quoted in the file)")
    ap.add_argument("--dir", action="append", default=[],
                    help="trace, mfma: the rocprofv3 output directory (cache: one per run)")
    ap.add_argument("--note", default="")
    ap.add_argument("--cycle", action="append", default=[],
                    help="trace: KERNEL=name1,name2,... names for successive launches of KERNEL")
    ap.add_argument("--workload", help="traffic: workload of the algorithmic bytes")
    ap.add_argument("--cal-fetch")
    ap.add_argument("--cal-write")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    a = ap.parse_args(argv)
    cycles = {c.split("=")[0]: c.split("=")[1].split(",") for c in a.cycle}
    if a.kind == "trace":
        md = summarize_trace(a.dir[0], a.title, a.command, a.note, cycles or None)
    elif a.kind == "mfma":
        md = summarize_mfma(a.dir[0], a.title, a.command, cycles or None)
    elif a.kind == "cache":
        md = summarize_cache(a.dir, a.title, a.command, cycles or None)
    else:
        md = summarize_traffic(a.workload, a.cal_fetch, a.cal_write, a.fetch, a.write, a.title,
                               a.command, cycles or None)
    with open(a.out, "w") as f:
        f.write(md)
    print(md)


OTHERS.update({"skewed_dsv3": bench_skewed_linear, "nemotron_proxy_mlp": bench_fused_mlp,
               "fc1_swiglu_quantize": bench_fc1_swiglu,
               "swiglu_bwd_quantize": bench_swiglu_bwd_quant,
               "group_quantize_131072x7168": bench_group_quantize})


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize":
        summarize_main(sys.argv[2:])
        return
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.only:
        import torch
        torch.cuda.set_device(0)
        print(json.dumps({args.only: OTHERS[args.only](args.steps, args.warmup)}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the MXFP8 grouped-GEMM "
              "path here has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_expert_grouped_group_amd as mx
    from moe_expert_grouped_group_amd import workloads as wl

    torch.cuda.set_device(0)
    w = wl.make(args.workload)
    g, t, k, n = w.groups, w.tokens, w.hidden, w.ffn
    dev = "cuda"
    x = w.tensors["x"].to(dev)
    wt = w.tensors["w"].to(dev)
    dy = w.tensors["dy"].to(dev)
    ms = torch.from_numpy(w.m_splits).to(dev)
    out_dtype = torch.bfloat16 if w.out_dtype == "bf16" else torch.float32

    u8 = dict(dtype=torch.uint8, device=dev)
    # row-wise copies (forward, dgrad) and the column-wise requantized copies
    # (wgrad) of X and dY, written by one fused launch each
    xo = mx.MXFP8Tensor(torch.empty(t, k, **u8), torch.empty(t, k // 32, **u8),
                        torch.empty(k, t, **u8), torch.empty(k, t // 32, **u8))
    wo = mx.MXFP8Tensor(torch.empty(g * n, k, **u8), torch.empty(g * n, k // 32, **u8),
                        torch.empty(k, g * n, **u8), torch.empty(k, g * n // 32, **u8))
    xc = xo
    dyo = mx.MXFP8Tensor(torch.empty(t, n, **u8), torch.empty(t, n // 32, **u8),
                         torch.empty(n, t, **u8), torch.empty(n, t // 32, **u8))
    dyc = dyo
    y = torch.empty(t, n, dtype=out_dtype, device=dev)
    dx = torch.empty(t, k, dtype=out_dtype, device=dev)
    dw = torch.empty(g, n, k, dtype=out_dtype, device=dev)
    db = torch.empty(g, n, dtype=torch.float32, device=dev)
    ws = torch.empty(mx.dbias_workspace_bytes(t, n), **u8)
    gws = torch.empty(mx.gemm_workspace_bytes(), **u8)   # wgrad tile counter

    ev = {}

    def timed(name, fn):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        r = fn()
        b.record()
        ev.setdefault(name, []).append((a, b))
        return r

    def step_plain():
        mx.group_quantize_requant(x, out=xo)
        mx.group_quantize(wt, mx.ROWWISE | mx.COLWISE, out=wo)
        mx.grouped_gemm("NT", xo.row_data, xo.row_scale, wo.row_data, wo.row_scale, ms, t, n, k,
                        out_dtype, y)
        mx.group_quantize_requant(dy, ms, with_dbias=True, out=dyo, dbias=db, workspace=ws)
        mx.grouped_gemm("NN", dyo.row_data, dyo.row_scale, wo.col_data, wo.col_scale, ms, t, n, k,
                        out_dtype, dx)
        mx.grouped_gemm("TN", dyc.col_data, dyc.col_scale, xc.col_data, xc.col_scale, ms, t, n, k,
                        out_dtype, dw, workspace=gws)

    def step():
        timed("quant_requant_x", lambda: mx.group_quantize_requant(x, out=xo))
        timed("quant_w", lambda: mx.group_quantize(wt, mx.ROWWISE | mx.COLWISE, out=wo))
        timed("gemm_fprop", lambda: mx.grouped_gemm(
            "NT", xo.row_data, xo.row_scale, wo.row_data, wo.row_scale, ms, t, n, k, out_dtype, y))
        timed("quant_requant_dy_dbias", lambda: mx.group_quantize_requant(
            dy, ms, with_dbias=True, out=dyo, dbias=db, workspace=ws))
        timed("gemm_dgrad", lambda: mx.grouped_gemm(
            "NN", dyo.row_data, dyo.row_scale, wo.col_data, wo.col_scale, ms, t, n, k, out_dtype,
            dx))
        timed("gemm_wgrad", lambda: mx.grouped_gemm(
            "TN", dyc.col_data, dyc.col_scale, xc.col_data, xc.col_scale, ms, t, n, k, out_dtype,
            dw, workspace=gws))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev.clear()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = start.elapsed_time(stop) / args.steps
    ms_step_eager = ms_step

    per = {name: float(np.mean([a.elapsed_time(b) for a, b in pairs])) for name, pairs in ev.items()}

    if not args.eager:
        # The timed steps again, replayed from a HIP graph of the same six
        # launches (captured once; every output buffer is caller-owned, so a
        # replay rewrites the same memory): no host launch gaps between the
        # kernels.  The per-launch times above come from the eager steps.
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            step_plain()
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=cap):
                step_plain()
        torch.cuda.current_stream().wait_stream(cap)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        start.record()
        for _ in range(args.steps):
            graph.replay()
        stop.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        ms_step = start.elapsed_time(stop) / args.steps

    if args.step_only:
        args.no_others = args.no_cpu = True
    # Outside the step: wgrad accumulated into an fp32 main_grad (the
    # production form of the wgrad launch), timed on the same operands.
    acc_ms = sb_ms = sw_ms = sw_chain_ms = None
    sb_bytes = sw_bytes = 0
    sw_t, sw_f = 83968, 1024
    if out_dtype == torch.float32 and not args.step_only:
        main_grad = torch.zeros(g, n, k, dtype=torch.float32, device=dev)
        acc = lambda: mx.grouped_gemm_wgrad_accumulate(  # noqa: E731
            dyc.col_data, dyc.col_scale, xc.col_data, xc.col_scale, ms, t, n, k, main_grad,
            workspace=gws)
        acc_ms = _time_outside(acc, args.steps)
        del main_grad

    # Outside the step: gradients of a routing-scaled bias (dbias weighted by
    # each token's scale, and each token's scale gradient) from row-wise dY.
    if not args.step_only:
        gen = torch.Generator(device=dev)
        gen.manual_seed(7)
        r_scales = torch.rand(t, device=dev, generator=gen)
        r_bias = torch.randn(g, n, device=dev, generator=gen)
        sb_ws = torch.empty(mx.load_library().mxfp8_scaled_bias_workspace_bytes(t, n), **u8)
        sb_ms = _time_outside(lambda: mx.grouped_scaled_bias_grad(
            dyo.row_data, dyo.row_scale, ms, r_scales, r_bias, workspace=sb_ws), args.steps)
        # dY codes and scales read once, scales and bias read, both partial
        # sums written and read back, both outputs written
        sb_bytes = (t * n * (1 + 1 / 32) + t * 4 + g * n * 4 + 2 * (t // 128) * n * 4
                    + 2 * t * (n // 512) * 4 + g * n * 4 + t * 4)
        del r_scales, r_bias, sb_ws
        # Outside the step: the fused expert MLP's activation (SwiGLU of the
        # FC1 output, quantized row- and column-wise for FC2) at the
        # Nemotron-proxy MLP shape (T = 83968 tokens, FC1 out 2F = 2048),
        # fused in one kernel and as the two-kernel chain it replaces.
        hgen = torch.Generator(device=dev)
        hgen.manual_seed(11)
        h_sw = (torch.randn(sw_t, 2 * sw_f, device=dev, generator=hgen) * 3).to(torch.bfloat16)
        sw_out = mx.swiglu_quantize(h_sw)
        a_sw = mx.swiglu_fwd(h_sw)
        sw_ms = _time_outside(lambda: mx.swiglu_quantize(h_sw, out=sw_out), args.steps)
        sw_chain_ms = _time_outside(lambda: mx.group_quantize(
            mx.swiglu_fwd(h_sw, out=a_sw), mx.ROWWISE | mx.COLWISE, out=sw_out), args.steps)
        # fused: h read (4 B per output element), row + column copies written
        sw_bytes = sw_t * sw_f * (4 + 2 * (1 + 1 / 32))
        del h_sw, sw_out, a_sw

    flop_one = 2.0 * t * n * k
    gemm_ms = per["gemm_fprop"] + per["gemm_dgrad"] + per["gemm_wgrad"]
    gemm_tflops = 3 * flop_one / (gemm_ms * 1e-3) / 1e12
    value = 3 * flop_one / (ms_step * 1e-3) / 1e12
    # algorithmic HBM bytes of the streaming kernels
    q_bytes = {
        "quant_requant_x": t * k * (2 + 2 * (1 + 1 / 32)),
        "quant_w": g * n * k * (2 + 2 * (1 + 1 / 32)),
        "quant_requant_dy_dbias": t * n * (2 + 2 * (1 + 1 / 32)) + t * n * 4 / 128 * 2 + g * n * 4,
    }
    quant_ms = sum(per[nm] for nm in q_bytes)
    quant_gbs = sum(q_bytes.values()) / (quant_ms * 1e-3) / 1e9

    res = {
        "metric": "MXFP8 grouped GEMM TFLOP/s (fprop+dgrad+wgrad); group-quantize HBM GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_eager": round(ms_step_eager, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8-e4m3 (fp32 accumulate, fp32 out)" if out_dtype == torch.float32
                 else "mxfp8-e4m3 (fp32 accumulate, bf16 out)",
        "data": "synthetic",
        "config": {"workload": args.workload, "experts": g, "tokens": t, "hidden": k,
                   "ffn": n, "m_splits": [int(v) for v in w.m_splits],
                   "out_dtype": w.out_dtype},
        "gemm_tflops": round(gemm_tflops, 2),
        "group_quantize_gbs": round(quant_gbs, 1),
        "kernel_ms": {nm: round(v, 4) for nm, v in per.items()},
        "wgrad_accumulate": None if acc_ms is None else {
            "ms": round(acc_ms, 4), "tflops": round(flop_one / (acc_ms * 1e-3) / 1e12, 2),
            "note": "main_grad += dY^T X in fp32, outside the step"},
        "scaled_bias_grad": None if sb_ms is None else {
            "ms": round(sb_ms, 4), "gbs": round(sb_bytes / (sb_ms * 1e-3) / 1e9, 1),
            "note": "dbias and dscales of a routing-scaled bias from row-wise dY, outside the "
                    "step"},
        "swiglu_quantize": None if sw_ms is None else {
            "ms": round(sw_ms, 4), "gbs": round(sw_bytes / (sw_ms * 1e-3) / 1e9, 1),
            "unfused_ms": round(sw_chain_ms, 4),
            "note": f"SwiGLU + row/col MXFP8 of h [{sw_t}, {2 * sw_f}] in one kernel vs "
                    "swiglu_fwd + group_quantize, outside the step"},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2),
                     "peak": PEAK_MXFP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / PEAK_MXFP8_TFLOPS, 4),
                     "traffic": stored_traffic(args.workload),
                     "kernel": "grouped_gemm_kernel (3 launches per step)"},
        "quantize_roofline": {"bound": "hbm", "achieved": round(quant_gbs, 1),
                              "peak": PEAK_HBM_GBS, "unit": "GB/s",
                              "frac": round(quant_gbs / PEAK_HBM_GBS, 4)},
        "wall_s": round(wall, 3),
    }
    if not args.no_others:
        # the other workloads, each timed the same way (fewer steps), outside
        # the headline step
        del x, wt, dy, xo, wo, xc, dyo, dyc, y, dx, dw, db, ws
        torch.cuda.empty_cache()
        o_steps, o_warm = max(3, min(args.steps, 10)), max(1, min(args.warmup, 2))
        others = {}
        for name, fn in OTHERS.items():
            others[name] = fn(o_steps, o_warm)
            torch.cuda.empty_cache()
        res["other_workloads"] = others
        res["vendor_reference"] = vendor_reference(t, n, k, o_steps)
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
