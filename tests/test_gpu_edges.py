"""Degenerate and limit cases of the hot path, through the C ABI: no token
routed anywhere (T = 0) and the largest expert count the scheduler's
expert table holds (1024 experts, most of them without tokens).

T = 0: forward and dgrad write nothing (every output row belongs to an
expert, and there are none), the wgrad is all zeros for every expert, the
accumulating wgrad leaves main_grad untouched, dbias (standalone or fused
with the requantize) is zero, and the quantize and SwiGLU calls accept the
empty tensors (their device pointers are NULL).  1024
experts: the three GEMMs against the oracle's per-expert loop (integer-valued
operands, so the fp32 sums are exact and the outputs must match exactly) and
dbias against its fp64 sum, with the split chosen so that the experts with
tokens sit at both ends of the table and in the middle.
"""

import numpy as np
import pytest
import torch

import moe_expert_grouped_group_amd as mx
from oracle import gemm as og
from oracle import mxfp8 as om

from gpu_util import dev, f64, log

pytestmark = pytest.mark.gpu

_INTS = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50], dtype=np.uint8)  # 0..8


def _int_mx(rng, rows, cols):
    q = _INTS[rng.integers(0, _INTS.size, size=(rows, cols))]
    q |= (rng.integers(0, 2, size=(rows, cols)) << 7).astype(np.uint8)
    return q, np.full((rows, cols // 32), 127, dtype=np.uint8)


def test_no_tokens_anywhere():
    g, n, k = 3, 512, 1024
    ms = dev(np.zeros(g, dtype=np.int64))
    u8 = dict(dtype=torch.uint8, device="cuda")
    e = lambda *s: torch.zeros(*s, **u8)  # noqa: E731 (empty operands: T = 0)
    w = torch.zeros(g * n, k, **u8)
    ws = torch.full((g * n, k // 32), 127, **u8)
    wc = torch.zeros(k, g * n, **u8)
    wcs = torch.full((k, g * n // 32), 127, **u8)
    log("edges: T = 0 forward, dgrad, wgrad, accumulate, dbias")
    y = torch.full((0, n), 5.0, device="cuda")
    mx.grouped_gemm("NT", e(0, k), e(0, k // 32), w, ws, ms, 0, n, k, torch.float32, y)
    mx.grouped_gemm("NN", e(0, n), e(0, n // 32), wc, wcs, ms, 0, n, k, torch.float32,
                    torch.empty(0, k, device="cuda"))
    dw = torch.full((g, n, k), 3.0, device="cuda")
    mx.grouped_gemm("TN", e(n, 0), e(n, 0), e(k, 0), e(k, 0), ms, 0, n, k, torch.float32, dw)
    main = torch.full((g, n, k), 2.5, device="cuda")
    mx.grouped_gemm_wgrad_accumulate(e(n, 0), e(n, 0), e(k, 0), e(k, 0), ms, 0, n, k, main)
    db = mx.grouped_dbias(e(0, n), e(0, n // 32), ms, dbias=torch.full((g, n), 9.0, device="cuda"))
    log("edges: T = 0 quantize, requant with dbias, SwiGLU, SwiGLU backward + quantize")
    bf = torch.bfloat16
    xo = mx.group_quantize(torch.zeros(0, k, dtype=bf, device="cuda"), mx.ROWWISE | mx.COLWISE)
    _, db2 = mx.requant_colwise(xo.row_data, xo.row_scale, ms, with_dbias=True,
                                dbias=torch.full((g, k), 4.0, device="cuda"))
    h = torch.zeros(0, 2 * n, dtype=bf, device="cuda")
    ao = mx.swiglu_quantize(h)
    a = mx.swiglu_fwd(h)
    dh = mx.swiglu_bwd(h, a)
    bq, db3 = mx.swiglu_bwd_quantize(h, a, ms, with_dbias=True,
                                     dbias=torch.full((g, 2 * n), 6.0, device="cuda"))
    torch.cuda.synchronize()
    assert torch.count_nonzero(dw).item() == 0
    assert torch.all(main == 2.5)
    assert torch.count_nonzero(db).item() == 0
    assert torch.count_nonzero(db2).item() == 0
    assert xo.col_data.shape == (k, 0) and ao.row_data.shape == (0, n) and dh.shape == (0, 2 * n)
    assert torch.count_nonzero(db3).item() == 0 and bq.col_data.shape == (2 * n, 0)


@pytest.mark.parametrize("seed", [0, 1])
def test_1024_experts(seed):
    g, n, k = 1024, 512, 512
    rng = np.random.default_rng(300 + seed)
    splits = np.zeros(g, dtype=np.int64)
    busy = np.concatenate([[0, g - 1, g // 2], rng.choice(np.arange(1, g - 1), 37, replace=False)])
    splits[busy] = 128 * rng.integers(1, 4, size=busy.size)
    t = int(splits.sum())
    sp = [int(v) for v in splits]
    xq, xs = _int_mx(rng, t, k)
    wq, ws = _int_mx(rng, g * n, k)
    dyq, dys = _int_mx(rng, t, n)
    wcq, wcs = _int_mx(rng, k, g * n)
    dycq, dycs = om.requant_colwise(dyq, dys, sp)
    xcq, xcs = om.requant_colwise(xq, xs, sp)
    ms = dev(splits)
    log(f"edges: 1024 experts seed {seed}, T = {t}")
    y = mx.grouped_gemm("NT", dev(xq), dev(xs), dev(wq), dev(ws), ms, t, n, k)
    dx = mx.grouped_gemm("NN", dev(dyq), dev(dys), dev(wcq), dev(wcs), ms, t, n, k)
    dw = mx.grouped_gemm("TN", dev(dycq), dev(dycs), dev(xcq), dev(xcs), ms, t, n, k)
    db = mx.grouped_dbias(dev(dyq), dev(dys), ms)
    torch.cuda.synchronize()
    assert np.array_equal(f64(y), og.fprop(xq, xs, wq.reshape(g, n, k), ws.reshape(g, n, k // 32),
                                           sp))
    assert np.array_equal(f64(dx), og.dgrad(dyq, dys, wcq, wcs, sp, g))
    assert np.array_equal(f64(dw), og.wgrad(dycq, dycs, xcq, xcs, sp))
    # integer values with unit scales: the per-expert column sums are exact
    assert np.array_equal(f64(db), om.grouped_dbias(dyq, dys, sp))
