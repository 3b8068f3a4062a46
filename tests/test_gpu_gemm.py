"""GPU parity of the grouped MXFP8 GEMMs (forward NT, dgrad NN, wgrad TN)
against the CPU oracle.

fp32 outputs of forward and dgrad on well-scaled data (the Gaussian
workloads, contractions of 512 and more): |gpu - oracle| <= 1e-5 * sum_k
|a_k b_k| + 1e-6 per element.  Everywhere else (wgrad, whose contraction is
one expert's few 128-token windows; outliers; random codes over the whole
E4M3 range with random block scales) the bound adds the MFMA window term of
oracle.gemm.tolerance_mfma, derived from the measured accumulation of the
scaled MFMA (pinned by test_gpu_mfma_accumulation.py).  bf16 outputs: within
1 bf16 ulp of the oracle rounded to bf16, widened by the same accumulation
allowance for outputs that cancel.  Integer-valued operands with unit scales:
exactly equal.
"""

import numpy as np
import pytest
import torch

import moe_expert_grouped_group_amd as mx
from moe_expert_grouped_group_amd import workloads as wl
from oracle import gemm as og
from oracle import mxfp8 as om

from gpu_util import dev, f64, log, random_mx, u8

pytestmark = pytest.mark.gpu


def _check(got, ref, mag, out_dtype, win=None):
    """win None: the 1e-5 rule; else the MFMA window bound (tolerance_mfma)."""
    tol = og.tolerance_f32(mag) if win is None else og.tolerance_mfma(mag, win)
    if out_dtype == torch.float32:
        err = np.abs(got - ref)
        bad = err > tol
        assert not bad.any(), (int(bad.sum()), float((err / tol).max()))
    else:
        ok = og.within_bf16_ulp(got, ref, tol)
        assert ok.all(), int((~ok).sum())


def _mx_rows(rng, rows, cols, kind):
    if kind == "random":
        return random_mx(rng, rows, cols)
    # integer-valued codes (|v| <= 16) with unit scales: fp32 sums are exact
    ints = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50, 0x51, 0x52, 0x53,
                     0x54, 0x55, 0x56, 0x57, 0x58], dtype=np.uint8)   # 0, 1, 2, ..., 16
    q = ints[rng.integers(0, ints.size, size=(rows, cols))]
    q |= (rng.integers(0, 2, size=(rows, cols)) << 7).astype(np.uint8)
    s = np.full((rows, cols // 32), 127, dtype=np.uint8)
    return q, s


CASES = [
    # (splits, N, K)
    ([128, 256, 0, 384], 512, 512),
    ([512], 1024, 512),
    ([0, 128, 0, 0, 640, 128, 256, 0], 512, 1024),
    # T = 128: fewer tokens than one 256-row tile (the upper waves copy rows
    # of the lower ones; nothing past the last token is read or written)
    ([128], 512, 512),
    ([0, 128, 0], 512, 1536),
]


@pytest.mark.parametrize("kind", ["random", "integer"])
@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_three_layouts_synthetic(kind, case, out_dtype):
    splits, n, k = CASES[case]
    g = len(splits)
    t = sum(splits)
    rng = np.random.default_rng(1000 + case)
    xq, xs = _mx_rows(rng, t, k, kind)
    wq, ws = _mx_rows(rng, g * n, k, kind)
    dyq, dys = _mx_rows(rng, t, n, kind)
    wcq, wcs = _mx_rows(rng, k, g * n, kind)         # any valid column-wise copy
    dycq, dycs = _mx_rows(rng, n, t, kind)
    xcq, xcs = _mx_rows(rng, k, t, kind)
    ms = dev(np.asarray(splits, dtype=np.int64))

    log(f"gemm NT {kind} case {case} {out_dtype}")
    y = mx.grouped_gemm("NT", dev(xq), dev(xs), dev(wq), dev(ws), ms, t, n, k, out_dtype)
    log(f"gemm NN {kind} case {case} {out_dtype}")
    dx = mx.grouped_gemm("NN", dev(dyq), dev(dys), dev(wcq), dev(wcs), ms, t, n, k, out_dtype)
    log(f"gemm TN {kind} case {case} {out_dtype}")
    dw = mx.grouped_gemm("TN", dev(dycq), dev(dycs), dev(xcq), dev(xcs), ms, t, n, k, out_dtype)
    torch.cuda.synchronize()

    ref, mag, win = og.fprop(xq, xs, wq.reshape(g, n, k), ws.reshape(g, n, k // 32), splits,
                             True, True)
    ref2, mag2, win2 = og.dgrad(dyq, dys, wcq, wcs, splits, g, True, True)
    ref3, mag3, win3 = og.wgrad(dycq, dycs, xcq, xcs, splits, True, True)
    if kind == "integer" and out_dtype == torch.float32:
        assert np.array_equal(f64(y), ref)
        assert np.array_equal(f64(dx), ref2)
        assert np.array_equal(f64(dw), ref3)
    else:
        # random codes span the whole E4M3 range with random block scales
        _check(f64(y), ref, mag, out_dtype, win)
        _check(f64(dx), ref2, mag2, out_dtype, win2)
        _check(f64(dw), ref3, mag3, out_dtype, win3)
    for gi, m in enumerate(splits):
        if m == 0:
            assert np.all(f64(dw)[gi] == 0)


@pytest.mark.parametrize("kind", ["random", "integer"])
@pytest.mark.parametrize("layout", ["NT", "NN"])
def test_split_contraction_halves(kind, layout):
    """Forward and dgrad launches whose last round holds few, long tiles split
    each of those tiles into two contraction halves added into a zeroed C
    (fp32 output).  Here every tile is split: 384 tokens as [256, 128, 0, 0]
    (a full tile, and a 128-row tile of the second expert whose copied rows
    are shifted back to stay inside the operand), 5120-long contractions, 512
    outputs, a grid of 10 workgroups for 4 tiles.  The output buffer starts as
    garbage: the split
    tiles must be cleared before their halves are added."""
    splits = [256, 128, 0, 0]
    g, t = len(splits), sum(splits)
    kc, other = 5120, 512
    rng = np.random.default_rng(77 if kind == "random" else 78)
    ms = dev(np.asarray(splits, dtype=np.int64))
    if layout == "NT":
        n, k = other, kc
        aq, as_ = _mx_rows(rng, t, k, kind)
        bq, bs = _mx_rows(rng, g * n, k, kind)
        ref, mag, win = og.fprop(aq, as_, bq.reshape(g, n, k), bs.reshape(g, n, k // 32), splits,
                                 True, True)
        shape = (t, n)
    else:
        n, k = kc, other
        aq, as_ = _mx_rows(rng, t, n, kind)
        bq, bs = _mx_rows(rng, k, g * n, kind)
        ref, mag, win = og.dgrad(aq, as_, bq, bs, splits, g, True, True)
        shape = (t, k)
    for rep in range(2):
        out = torch.full(shape, 7.0 + rep, dtype=torch.float32, device="cuda")
        log(f"gemm {layout} split halves {kind} call {rep}")
        mx.grouped_gemm(layout, dev(aq), dev(as_), dev(bq), dev(bs), ms, t, n, k, torch.float32,
                        out)
        torch.cuda.synchronize()
        if kind == "integer":
            assert np.array_equal(f64(out), ref)
        else:
            _check(f64(out), ref, mag, torch.float32, win)


# wgrad tile-counter cases beyond CASES: most tokens on one expert of 24 (a
# few long tiles beside many short ones), one empty expert, so the tiles go
# through the counter; at N = K = 512 that is 96 tiles (fewer than the CUs),
# at N = K = 2048 1536 tiles, several per workgroup, with 4 x 2 tile blocks
# per expert (the blocked order of the accumulating and bf16 wgrads); then 8 experts, none
# empty, 1024 tiles.
COUNTER_CASES = [
    ([0, 3072, 128, 256, 128] + [128] * 19, 1024, 512),
    ([0, 3072, 128, 256, 128] + [128] * 19, 2048, 2048),
    ([256, 896, 384, 128, 512, 640, 128, 256], 4096, 2048),
]


@pytest.mark.parametrize("case", range(len(CASES) + len(COUNTER_CASES)))
def test_wgrad_tile_counter_same_bytes(case):
    """The wgrad with a tile counter (mxfp8_grouped_gemm_ws: tiles handed out
    as workgroups finish) gives the same bytes as the fixed assignment, in
    fp32 and bf16 and accumulated into main_grad, twice with one workspace.
    The COUNTER_CASES have fewer than 1 in 8 experts empty, so their tiles go
    through the counter (the last two with several tiles per workgroup: the
    counter's hand-out past the first round, and the blocked order of the
    bf16 and accumulating wgrads); the CASES (1 in 4 or more empty, or a single expert)
    cover the kernel's choice of the fixed order despite a workspace."""
    if case < len(CASES):
        splits, n, k = CASES[case]
    else:
        splits, n, k = COUNTER_CASES[case - len(CASES)]
    g, t = len(splits), sum(splits)
    rng = np.random.default_rng(500 + case)
    aq, as_ = random_mx(rng, n, t)
    bq, bs = random_mx(rng, k, t)
    ms = dev(np.asarray(splits, dtype=np.int64))
    ws = torch.empty(mx.gemm_workspace_bytes(), dtype=torch.uint8, device="cuda")
    A, As, B, Bs = dev(aq), dev(as_), dev(bq), dev(bs)
    log(f"gemm TN tile counter case {case}: {g} experts, {t} tokens, N={n}, K={k}")
    for dt in (torch.float32, torch.bfloat16):
        ref = mx.grouped_gemm("TN", A, As, B, Bs, ms, t, n, k, dt)
        for _ in range(2):
            got = mx.grouped_gemm("TN", A, As, B, Bs, ms, t, n, k, dt, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8))
    base = torch.from_numpy(rng.standard_normal((g, n, k)).astype(np.float32)).cuda()
    m1, m2 = base.clone(), base.clone()
    mx.grouped_gemm_wgrad_accumulate(A, As, B, Bs, ms, t, n, k, m1)
    mx.grouped_gemm_wgrad_accumulate(A, As, B, Bs, ms, t, n, k, m2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(m1.view(torch.uint8), m2.view(torch.uint8))


@pytest.mark.parametrize("use_ws", [False, True])
def test_wgrad_accumulate_many_tiles_exact(use_ws):
    """The accumulating wgrad where every workgroup takes several tiles (8
    experts, none empty, 4096 x 2048 outputs: 1024 tiles of 256 x 256), in
    the fixed order and through the tile counter (the blocked per-XCD order):
    on integer-valued operands with unit scales and an integer main_grad every
    fp32 sum is exact, so the result must equal the oracle exactly."""
    splits, n, k = [256, 896, 384, 128, 512, 640, 128, 256], 4096, 2048
    g, t = len(splits), sum(splits)
    rng = np.random.default_rng(4242)
    dycq, dycs = _mx_rows(rng, n, t, "integer")
    xcq, xcs = _mx_rows(rng, k, t, "integer")
    base = rng.integers(-64, 65, size=(g, n, k)).astype(np.float32)
    ms = dev(np.asarray(splits, dtype=np.int64))
    mg = dev(base)
    ws = torch.empty(mx.gemm_workspace_bytes(), dtype=torch.uint8, device="cuda") if use_ws else None
    log(f"wgrad accumulate, 1024 tiles, workspace={use_ws}")
    mx.grouped_gemm_wgrad_accumulate(dev(dycq), dev(dycs), dev(xcq), dev(xcs), ms, t, n, k, mg,
                                     workspace=ws)
    torch.cuda.synchronize()
    ref = og.wgrad_accumulate(base, dycq, dycs, xcq, xcs, splits)
    assert np.array_equal(mg.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("kind", ["random", "integer"])
@pytest.mark.parametrize("case", [0, 2, 4])
def test_wgrad_accumulate(kind, case):
    """main_grad[g] += dY_g^T X_g in place.  Bound: the wgrad bound of the
    product plus one fp32 rounding of the final sum (2^-24 of its size);
    integer-valued data is exact.  Experts without tokens keep their slice
    bit for bit (their base holds negative zeros, which an added +0 would
    turn positive)."""
    splits, n, k = CASES[case]
    g = len(splits)
    t = sum(splits)
    rng = np.random.default_rng(2000 + case)
    dycq, dycs = _mx_rows(rng, n, t, kind)
    xcq, xcs = _mx_rows(rng, k, t, kind)
    if kind == "integer":
        base = rng.integers(-64, 65, size=(g, n, k)).astype(np.float32)
    else:
        base = (rng.standard_normal((g, n, k)) * 100).astype(np.float32)
    for gi, m in enumerate(splits):
        if m == 0:
            base[gi, ::3] = -0.0
    ms = dev(np.asarray(splits, dtype=np.int64))
    mg = dev(base)
    log(f"wgrad accumulate {kind} case {case}")
    mx.grouped_gemm_wgrad_accumulate(dev(dycq), dev(dycs), dev(xcq), dev(xcs), ms, t, n, k, mg)
    torch.cuda.synchronize()
    got = mg.cpu().numpy()
    ref, mag, win = og.wgrad_accumulate(base, dycq, dycs, xcq, xcs, splits, True, True)
    for gi, m in enumerate(splits):
        if m == 0:
            assert np.array_equal(got[gi].view(np.uint32), base[gi].view(np.uint32)), gi
    if kind == "integer":
        assert np.array_equal(got.astype(np.float64), ref)
    else:
        tol = og.tolerance_mfma(mag, win) + 2.0 ** -24 * np.abs(ref)
        err = np.abs(got.astype(np.float64) - ref)
        assert not (err > tol).any(), (int((err > tol).sum()), float((err / tol).max()))


def test_single_group_is_dense():
    rng = np.random.default_rng(5)
    t, n, k = 384, 512, 1024
    xq, xs = random_mx(rng, t, k)
    wq, ws = random_mx(rng, n, k)
    log("gemm single group")
    y = mx.grouped_gemm("NT", dev(xq), dev(xs), dev(wq), dev(ws),
                        dev(np.array([t], dtype=np.int64)), t, n, k)
    torch.cuda.synchronize()
    ref, mag, win = og.fprop(xq, xs, wq[None], ws[None], [t], True, True)
    xh, wh = om.dequantize_rowwise(xq, xs), om.dequantize_rowwise(wq, ws)
    assert np.array_equal(ref, xh @ wh.T)
    _check(f64(y), ref, mag, torch.float32, win)


def test_rows_outside_experts_untouched():
    # forward writes only the rows of its experts; a canary value elsewhere in
    # a larger buffer (rows past T) survives
    rng = np.random.default_rng(6)
    splits, n, k = [128, 0, 256], 512, 512
    t = sum(splits)
    xq, xs = random_mx(rng, t, k)
    wq, ws = random_mx(rng, 3 * n, k)
    big = torch.full((t + 128, n), 12345.0, device="cuda")
    log("gemm canary")
    mx.grouped_gemm("NT", dev(xq), dev(xs), dev(wq), dev(ws),
                    dev(np.asarray(splits, dtype=np.int64)), t, n, k, out=big[:t])
    torch.cuda.synchronize()
    assert torch.all(big[t:] == 12345.0)
    ref, mag, win = og.fprop(xq, xs, wq.reshape(3, n, k), ws.reshape(3, n, k // 32), splits,
                             True, True)
    _check(f64(big[:t]), ref, mag, torch.float32, win)


@pytest.mark.parametrize("name", ["tiny_fwd", "small_moe8", "small_skewed", "small_nemotron_mlp"])
def test_workload_fwd_bwd(name):
    """The hot path on a workload recipe: quantize, forward, requant, dgrad,
    wgrad, dbias.  Every oracle input is the oracle's own quantization of the
    bf16 tensors; the GPU's bytes are checked equal to it stage by stage."""
    w = wl.make(name)
    g, t, k, n = w.groups, w.tokens, w.hidden, w.ffn
    out_dtype = torch.bfloat16 if w.out_dtype == "bf16" else torch.float32
    outliers = "skewed" in name      # X carries 0.1 % outliers x1000
    ms = dev(w.m_splits)
    splits = [int(v) for v in w.m_splits]
    x64 = w.tensors["x"].double().numpy()
    w64 = w.tensors["w"].double().numpy().reshape(g * n, k)
    xq, xs = om.quantize_rowwise(x64)
    wq, ws = om.quantize_rowwise(w64)
    log(f"workload {name}: quantize")
    xo = mx.group_quantize(w.tensors["x"].to("cuda"), mx.ROWWISE)
    wo = mx.group_quantize(w.tensors["w"].to("cuda"), mx.ROWWISE | mx.COLWISE)
    log(f"workload {name}: forward")
    y = mx.grouped_gemm("NT", xo.row_data, xo.row_scale, wo.row_data, wo.row_scale, ms, t, n, k,
                        out_dtype)
    torch.cuda.synchronize()
    assert np.array_equal(u8(xo.row_data), xq) and np.array_equal(u8(xo.row_scale), xs)
    assert np.array_equal(u8(wo.row_data), wq) and np.array_equal(u8(wo.row_scale), ws)
    ref, mag, win = og.fprop(xq, xs, wq.reshape(g, n, k), ws.reshape(g, n, k // 32), splits,
                             True, True)
    _check(f64(y), ref, mag, out_dtype, win if outliers else None)
    if name == "tiny_fwd":
        return
    dy_t = w.tensors["dy"]
    if dy_t.shape[1] != n:     # fused-MLP workloads carry the FC2 gradient; use an FC1-shaped one
        dy_t = wl.bf16_normal([w.wid, wl.STREAM_DY, 99], (t, n))
    dyq, dys = om.quantize_rowwise(dy_t.double().numpy())
    wcq, wcs = om.quantize_colwise(w64, [g * n])
    log(f"workload {name}: backward")
    dyo = mx.group_quantize(dy_t.to("cuda"), mx.ROWWISE)
    xo2, _db_x = mx.requant_colwise(xo.row_data, xo.row_scale, ms, with_dbias=True)
    dyo2, db = mx.requant_colwise(dyo.row_data, dyo.row_scale, ms, with_dbias=True)
    dx = mx.grouped_gemm("NN", dyo.row_data, dyo.row_scale, wo.col_data, wo.col_scale, ms, t, n,
                         k, out_dtype)
    dw = mx.grouped_gemm("TN", dyo2.col_data, dyo2.col_scale, xo2.col_data, xo2.col_scale, ms,
                         t, n, k, out_dtype)
    torch.cuda.synchronize()
    assert np.array_equal(u8(dyo.row_data), dyq) and np.array_equal(u8(dyo.row_scale), dys)
    assert np.array_equal(u8(wo.col_data), wcq) and np.array_equal(u8(wo.col_scale), wcs)
    # column-wise copies: bit-exact against the oracle's requant
    dycq, dycs = om.requant_colwise(dyq, dys, splits)
    assert np.array_equal(u8(dyo2.col_data), dycq) and np.array_equal(u8(dyo2.col_scale), dycs)
    xcq, xcs = om.requant_colwise(xq, xs, splits)
    assert np.array_equal(u8(xo2.col_data), xcq) and np.array_equal(u8(xo2.col_scale), xcs)
    ref2, mag2 = og.dgrad(dyq, dys, wcq, wcs, splits, g, True)
    _check(f64(dx), ref2, mag2, out_dtype)
    ref3, mag3, win3 = og.wgrad(dycq, dycs, xcq, xcs, splits, True, True)
    # wgrad contracts over one expert's tokens (a few 128-element windows):
    # the window truncation does not average out, so it is gated on the
    # window bound even for Gaussian data
    _check(f64(dw), ref3, mag3, out_dtype, win3)
    refb = om.grouped_dbias(dyq, dys, splits)
    xh = np.abs(om.dequantize_rowwise(dyq, dys))
    row = 0
    for gi, m in enumerate(splits):
        magb = xh[row:row + m].sum(axis=0)
        assert np.all(np.abs(f64(db)[gi] - refb[gi]) <= og.tolerance_f32(magb))
        row += m
        if m == 0:
            assert np.all(f64(dw)[gi] == 0)
