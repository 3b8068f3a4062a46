"""GPU parity of the streaming kernels against the CPU oracle.

Quantized bytes and scales must be bit-exact; dbias (fp32 sums) must be
within 1e-5 * sum|x| + 1e-6; SwiGLU (bf16 out) within 1 bf16 ulp of the
oracle rounded to bf16.
"""

import numpy as np
import pytest
import torch

import moe_expert_grouped_group_amd as mx
from moe_expert_grouped_group_amd import workloads as wl
from oracle import gemm as og
from oracle import mxfp8 as om
from oracle import swiglu as osw

from gpu_util import (all_bf16_bits, bf16_from_bits, dev, f64, log, random_mx, sweep_bf16_bits,
                      u8)

pytestmark = pytest.mark.gpu


def _check_row(x_cpu_bf16, out):
    q, s = om.quantize_rowwise(f64(x_cpu_bf16))
    assert np.array_equal(u8(out.row_scale), s)
    assert np.array_equal(u8(out.row_data), q)


def _check_col(x_cpu_bf16, out, splits=None):
    x = f64(x_cpu_bf16)
    splits = [x.shape[0]] if splits is None else splits
    q, s = om.quantize_colwise(x, splits)
    assert np.array_equal(u8(out.col_scale), s)
    assert np.array_equal(u8(out.col_data), q)


@pytest.mark.parametrize("rows,cols,seed", [(256, 512, 1), (1024, 1536, 2), (128, 4096, 3)])
def test_rowwise_sweep(rows, cols, seed):
    log(f"rowwise sweep {rows}x{cols} seed {seed}")
    x = bf16_from_bits(sweep_bf16_bits(rows, cols, seed))
    out = mx.group_quantize(x.to("cuda"), mx.ROWWISE)
    torch.cuda.synchronize()
    _check_row(x, out)


def test_rowwise_every_bf16_value():
    log("rowwise every bf16 value")
    x = bf16_from_bits(all_bf16_bits(512))
    out = mx.group_quantize(x.to("cuda"), mx.ROWWISE)
    torch.cuda.synchronize()
    _check_row(x, out)


@pytest.mark.parametrize("usage", [mx.COLWISE, mx.ROWWISE | mx.COLWISE])
@pytest.mark.parametrize("rows,cols,seed", [(256, 512, 4), (640, 1024, 5)])
def test_rowcol_sweep(usage, rows, cols, seed):
    log(f"rowcol sweep usage {usage} {rows}x{cols}")
    x = bf16_from_bits(sweep_bf16_bits(rows, cols, seed))
    out = mx.group_quantize(x.to("cuda"), usage)
    torch.cuda.synchronize()
    _check_col(x, out)
    if usage & mx.ROWWISE:
        _check_row(x, out)


def test_rowcol_every_bf16_value():
    log("rowcol every bf16 value")
    x = bf16_from_bits(all_bf16_bits(512))
    out = mx.group_quantize(x.to("cuda"), mx.ROWWISE | mx.COLWISE)
    torch.cuda.synchronize()
    _check_row(x, out)
    _check_col(x, out)


@pytest.mark.parametrize("name", ["tiny_fwd", "small_moe8", "small_skewed",
                                  "small_group_quantize", "small_nemotron_mlp"])
def test_workload_quantize(name):
    log(f"workload quantize {name}")
    w = wl.make(name)
    x = w.tensors["x"]
    out = mx.group_quantize(x.to("cuda"), mx.ROWWISE | mx.COLWISE)
    torch.cuda.synchronize()
    _check_row(x, out)
    _check_col(x, out, list(w.m_splits))
    if "w" in w.tensors:
        wt = w.tensors["w"]
        g, n, k = wt.shape
        wo = mx.group_quantize(wt.to("cuda"), mx.ROWWISE | mx.COLWISE)
        torch.cuda.synchronize()
        _check_row(wt.reshape(g * n, k), wo)
        _check_col(wt.reshape(g * n, k), wo)


def test_preallocated_outputs_reused():
    log("preallocated outputs reused")
    x1 = bf16_from_bits(sweep_bf16_bits(256, 512, 7))
    x2 = bf16_from_bits(sweep_bf16_bits(256, 512, 8))
    out = mx.group_quantize(x1.to("cuda"), mx.ROWWISE | mx.COLWISE)
    ptrs = (out.row_data.data_ptr(), out.col_data.data_ptr())
    out = mx.group_quantize(x2.to("cuda"), mx.ROWWISE | mx.COLWISE, out=out)
    torch.cuda.synchronize()
    assert (out.row_data.data_ptr(), out.col_data.data_ptr()) == ptrs
    _check_row(x2, out)
    _check_col(x2, out)


def _requant_case(q, s, splits, seed):
    log(f"requant {q.shape} splits {splits[:6]} seed {seed}")
    ms = dev(np.asarray(splits, dtype=np.int64))
    out, db = mx.requant_colwise(dev(q), dev(s), ms, with_dbias=True)
    torch.cuda.synchronize()
    qc, sc = om.requant_colwise(q, s, splits)
    assert np.array_equal(u8(out.col_scale), sc)
    assert np.array_equal(u8(out.col_data), qc)
    ref = om.grouped_dbias(q, s, splits)
    mag = np.zeros_like(ref)
    xh = np.abs(om.dequantize_rowwise(q, s))
    row = 0
    for g, m in enumerate(splits):
        mag[g] = xh[row:row + m].sum(axis=0)
        row += m
    got = f64(db)
    assert np.all(np.abs(got - ref) <= og.tolerance_f32(mag))
    for g, m in enumerate(splits):
        if m == 0:
            assert np.all(got[g] == 0)


@pytest.mark.parametrize("seed", [0, 1])
def test_requant_random_codes(seed):
    rng = np.random.default_rng(100 + seed)
    splits = [256, 0, 128, 384, 0, 256]
    q, s = random_mx(rng, sum(splits), 1024)
    _requant_case(q, s, splits, seed)


def test_requant_wide_scales():
    # scale bytes spread over the whole E8M0 range used by bf16 data
    rng = np.random.default_rng(7)
    splits = [512, 128]
    q, s = random_mx(rng, 640, 512, smin=0, smax=240)
    q[:, :64] = 0        # zero column blocks
    _requant_case(q, s, splits, 7)


def test_requant_scale_bytes_above_fast_range():
    """Row scale bytes 247..254 (beyond what bf16 data produces) decode past
    the fp32 range, so the kernel requantizes such tiles with its integer
    path; tiles 0 and 2 of the 128-row tiles hold such bytes, tile 1 does not."""
    rng = np.random.default_rng(13)
    q, s = random_mx(rng, 384, 512, smin=100, smax=246)
    s[:128, :4] = rng.integers(247, 255, size=(128, 4))       # tile (0, 0): every row
    s[300, 9] = 254                                           # tile (2, 2): one byte
    log("requant with scale bytes 247..254")
    out = mx.requant_colwise(dev(q), dev(s))
    torch.cuda.synchronize()
    qc, sc = om.requant_colwise(q, s, [384])
    assert np.array_equal(u8(out.col_scale), sc)
    assert np.array_equal(u8(out.col_data), qc)
    # with dbias: values small enough that the fp32 sums stay finite (codes
    # <= 3 * 2^-9 under the bytes above 246, other bytes at most 200)
    q2, s2 = q.copy(), np.where(s > 246, s, np.minimum(s, 200)).astype(np.uint8)
    q2[:128, :128] &= 0x83
    q2[300, 288:320] &= 0x83
    _requant_case(q2, s2, [128, 256], 13)


def test_requant_of_quantized_sweep():
    x = bf16_from_bits(sweep_bf16_bits(512, 512, 9))
    q, s = om.quantize_rowwise(f64(x))
    # keep the values small enough for fp32 dbias sums (exponent fields < 200)
    s = np.minimum(s, 200).astype(np.uint8)
    _requant_case(q, s, [128, 256, 128], 9)


def test_requant_without_dbias_matches():
    rng = np.random.default_rng(11)
    q, s = random_mx(rng, 384, 512)
    log("requant without dbias")
    out = mx.requant_colwise(dev(q), dev(s))
    torch.cuda.synchronize()
    qc, sc = om.requant_colwise(q, s, [384])
    assert np.array_equal(u8(out.col_data), qc) and np.array_equal(u8(out.col_scale), sc)


@pytest.mark.parametrize("splits", [[128, 0, 256, 128], [512], [0, 0, 384]])
def test_grouped_dbias(splits):
    log(f"grouped dbias {splits}")
    rng = np.random.default_rng(sum(splits))
    q, s = random_mx(rng, sum(splits), 1024)
    db = mx.grouped_dbias(dev(q), dev(s), dev(np.asarray(splits, dtype=np.int64)))
    torch.cuda.synchronize()
    ref = om.grouped_dbias(q, s, splits)
    xh = np.abs(om.dequantize_rowwise(q, s))
    row = 0
    got = f64(db)
    for g, m in enumerate(splits):
        mag = xh[row:row + m].sum(axis=0)
        assert np.all(np.abs(got[g] - ref[g]) <= og.tolerance_f32(mag))
        row += m


@pytest.mark.parametrize("splits,n", [([128, 0, 256, 128], 1024), ([0, 0, 384], 512),
                                      ([256, 128, 128, 0, 0, 640], 1536)])
def test_scaled_bias_grad(splits, n):
    """dbias = sum of scales[r] dY[r] per expert and dscales = dY[r] . bias[g]
    from row-wise dY; fp32 sums held to 1e-5 * (sum of |terms|) + 1e-6."""
    log(f"scaled bias grad {splits} n {n}")
    rng = np.random.default_rng(sum(splits) + n)
    t = sum(splits)
    q, s = random_mx(rng, t, n)
    scales = rng.random(t).astype(np.float32)
    bias = rng.standard_normal((len(splits), n)).astype(np.float32)
    ms = dev(np.asarray(splits, dtype=np.int64))
    db, ds = mx.grouped_scaled_bias_grad(dev(q), dev(s), ms, dev(scales), dev(bias))
    torch.cuda.synchronize()
    ref_db, ref_ds = om.grouped_scaled_bias_grad(q, s, splits, scales, bias)
    xh = np.abs(om.dequantize_rowwise(q, s))
    mag_db = np.zeros_like(ref_db)
    mag_ds = np.zeros_like(ref_ds)
    row = 0
    for g, m in enumerate(splits):
        mag_db[g] = (scales[row:row + m, None].astype(np.float64) * xh[row:row + m]).sum(axis=0)
        mag_ds[row:row + m] = xh[row:row + m] @ np.abs(bias[g].astype(np.float64))
        row += m
    assert np.all(np.abs(f64(db) - ref_db) <= og.tolerance_f32(mag_db))
    assert np.all(np.abs(f64(ds) - ref_ds) <= og.tolerance_f32(mag_ds))
    for g, m in enumerate(splits):
        if m == 0:
            assert np.all(f64(db)[g] == 0)
    # either output alone
    db2, none = mx.grouped_scaled_bias_grad(dev(q), dev(s), ms, dev(scales), None,
                                            want_dscales=False)
    none2, ds2 = mx.grouped_scaled_bias_grad(dev(q), dev(s), ms, None, dev(bias),
                                             want_dbias=False)
    torch.cuda.synchronize()
    assert none is None and none2 is None
    assert torch.equal(db2, db) and torch.equal(ds2, ds)


def test_validate_splits():
    log("validate splits")
    cases = [([128, 256, 0], 384, 0), ([128, 100], 228, 2), ([-128, 256], 128, 1),
             ([128, 128], 512, 4), ([130, -2], 128, 3)]
    for splits, t, want in cases:
        flag = mx.validate_splits(dev(np.asarray(splits, dtype=np.int64)), t)
        assert int(flag.item()) == want, (splits, t)


@pytest.mark.parametrize("t,f", [(256, 1024), (384, 512)])
def test_swiglu(t, f):
    log(f"swiglu {t}x{f}")
    rng = np.random.default_rng(t + f)
    h = torch.from_numpy((rng.standard_normal((t, 2 * f)) * 3).astype(np.float32)).to(torch.bfloat16)
    da = torch.from_numpy(rng.standard_normal((t, f)).astype(np.float32)).to(torch.bfloat16)
    a = mx.swiglu_fwd(h.to("cuda"))
    dh = mx.swiglu_bwd(h.to("cuda"), da.to("cuda"))
    torch.cuda.synchronize()
    assert og.within_bf16_ulp(f64(a), osw.swiglu_fwd(f64(h))).all()
    assert og.within_bf16_ulp(f64(dh), osw.swiglu_bwd(f64(h), f64(da))).all()


def _swiglu_input(t, f, seed):
    """FC1-output-like h [T, 2F] bf16: N(0, 3^2), with the gate of the first
    32 rows zeroed (all-zero blocks, signed zeros from negative up values)."""
    rng = np.random.default_rng(seed)
    h = (rng.standard_normal((t, 2 * f)) * 3).astype(np.float32)
    h[:32, :f] = 0.0
    return torch.from_numpy(h).to(torch.bfloat16)


def _mx_bytes(out):
    return [u8(b) for b in (out.row_data, out.row_scale, out.col_data, out.col_scale)
            if b is not None]


@pytest.mark.parametrize("usage", [mx.ROWWISE | mx.COLWISE, mx.ROWWISE, mx.COLWISE])
@pytest.mark.parametrize("t,f,seed", [(256, 1024, 11), (384, 512, 12), (1024, 1536, 13)])
def test_swiglu_quantize_matches_unfused(usage, t, f, seed):
    """The fused kernel gives the bytes of swiglu_fwd followed by the group
    quantize (each pinned to the oracle by the tests above)."""
    log(f"swiglu_quantize vs unfused usage {usage} {t}x{f}")
    h = _swiglu_input(t, f, seed).to("cuda")
    fused = mx.swiglu_quantize(h, usage)
    unfused = mx.group_quantize(mx.swiglu_fwd(h), usage)
    torch.cuda.synchronize()
    for a, b in zip(_mx_bytes(fused), _mx_bytes(unfused)):
        assert np.array_equal(a, b)


def _near_codes(gpu, ref):
    """Same sign and at most one E4M3 step apart (codes are monotone in the
    magnitude within a sign)."""
    g = gpu.astype(np.int32)
    r = ref.astype(np.int32)
    same_sign = ((g ^ r) & 0x80) == 0
    return same_sign & (np.abs((g & 0x7F) - (r & 0x7F)) <= 1)


@pytest.mark.parametrize("t,f,seed", [(256, 1024, 21), (640, 512, 22)])
def test_swiglu_quantize_vs_oracle(t, f, seed):
    """Against the oracle: quantize(round_to_bf16(swiglu(h))).  The device
    forms silu in fp32, so its bf16 activation may sit one bf16 step from the
    oracle's (the allowance of the plain SwiGLU test); such an element can move
    its code by one step, or its block's scale by one at a power of two.
    Everything else must match exactly, and the moves must be rare."""
    log(f"swiglu_quantize vs oracle {t}x{f}")
    h = _swiglu_input(t, f, seed)
    out = mx.swiglu_quantize(h.to("cuda"), mx.ROWWISE | mx.COLWISE)
    torch.cuda.synchronize()
    a_ref = om.round_to_bf16(osw.swiglu_fwd(f64(h)))
    qr, sr = om.quantize_rowwise(a_ref)
    qc, sc = om.quantize_colwise(a_ref, [t])
    for q_gpu, s_gpu, q_ref, s_ref in ((u8(out.row_data), u8(out.row_scale), qr, sr),
                                       (u8(out.col_data), u8(out.col_scale), qc, sc)):
        ds = s_gpu.astype(np.int32) - s_ref.astype(np.int32)
        assert np.abs(ds).max() <= 1
        assert np.count_nonzero(ds) <= max(2, s_ref.size // 1000)
        same_scale = np.repeat(ds == 0, 32, axis=1)
        diff = (q_gpu != q_ref) & same_scale
        assert _near_codes(q_gpu[diff], q_ref[diff]).all()
        assert np.count_nonzero(diff) <= max(4, q_ref.size // 1000)
    # the zeroed gate rows quantize to signed zeros with scale byte 0
    assert np.array_equal(u8(out.row_scale)[:32], np.zeros((32, f // 32), np.uint8))
    assert np.array_equal(u8(out.row_data)[:32], qr[:32])


def test_swiglu_quantize_reuses_outputs():
    log("swiglu_quantize reuses outputs")
    h1 = _swiglu_input(256, 512, 31).to("cuda")
    h2 = _swiglu_input(256, 512, 32).to("cuda")
    out = mx.swiglu_quantize(h1)
    ptrs = (out.row_data.data_ptr(), out.col_data.data_ptr())
    out = mx.swiglu_quantize(h2, out=out)
    ref = mx.group_quantize(mx.swiglu_fwd(h2), mx.ROWWISE | mx.COLWISE)
    torch.cuda.synchronize()
    assert (out.row_data.data_ptr(), out.col_data.data_ptr()) == ptrs
    for a, b in zip(_mx_bytes(out), _mx_bytes(ref)):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("usage", [mx.ROWWISE, mx.COLWISE, mx.ROWWISE | mx.COLWISE])
def test_noop_flag(usage):
    """A set no-op flag leaves every output as the last call wrote it; a
    cleared one quantizes as usual (both kernels: row-wise only, and the
    row + column kernel)."""
    log(f"noop flag usage {usage}")
    x1 = bf16_from_bits(sweep_bf16_bits(256, 1024, 41))
    x2 = bf16_from_bits(sweep_bf16_bits(256, 1024, 42))
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = mx.group_quantize(x1.to("cuda"), usage, noop_flag=flag)
    flag.fill_(1)
    out = mx.group_quantize(x2.to("cuda"), usage, out=out, noop_flag=flag)
    torch.cuda.synchronize()
    if usage & mx.ROWWISE:
        _check_row(x1, out)
    if usage & mx.COLWISE:
        _check_col(x1, out)
    flag.fill_(0)
    out = mx.group_quantize(x2.to("cuda"), usage, out=out, noop_flag=flag)
    torch.cuda.synchronize()
    if usage & mx.ROWWISE:
        _check_row(x2, out)
    if usage & mx.COLWISE:
        _check_col(x2, out)


def _quantize_requant_case(x_cpu, splits, with_dbias):
    """The fused call against the two calls it replaces (every byte, and dbias
    bit for bit) and against the oracle's row-wise quantize + requantize."""
    x = x_cpu.to("cuda")
    ms = dev(np.asarray(splits, dtype=np.int64))
    ref = mx.group_quantize(x, mx.ROWWISE)
    if with_dbias:
        refc, refdb = mx.requant_colwise(ref.row_data, ref.row_scale, ms, with_dbias=True)
        got, db = mx.group_quantize_requant(x, ms, with_dbias=True)
    else:
        refc = mx.requant_colwise(ref.row_data, ref.row_scale)
        got = mx.group_quantize_requant(x)
    torch.cuda.synchronize()
    for a, b in ((got.row_data, ref.row_data), (got.row_scale, ref.row_scale),
                 (got.col_data, refc.col_data), (got.col_scale, refc.col_scale)):
        assert torch.equal(a, b)
    if with_dbias:
        assert torch.equal(db.view(torch.uint8), refdb.view(torch.uint8))
    q, s = om.quantize_rowwise(f64(x_cpu))
    cq, cs = om.requant_colwise(q, s, splits)
    assert np.array_equal(u8(got.row_data), q) and np.array_equal(u8(got.row_scale), s)
    assert np.array_equal(u8(got.col_data), cq) and np.array_equal(u8(got.col_scale), cs)


@pytest.mark.parametrize("rows,cols,seed", [(256, 512, 31), (640, 1536, 32), (1024, 4096, 33)])
@pytest.mark.parametrize("with_dbias", [False, True])
def test_quantize_requant_sweep(rows, cols, seed, with_dbias):
    """Row-wise quantize fused with the column-wise requantize of its result,
    on inputs spanning the encoder's relative exponents and whole-range
    values, with zero blocks; dbias over uneven experts (one empty)."""
    log(f"quantize+requant sweep {rows}x{cols} dbias {with_dbias}")
    x = bf16_from_bits(sweep_bf16_bits(rows, cols, seed))
    splits = [128, 0, rows - 128]
    _quantize_requant_case(x, splits, with_dbias)


def test_quantize_requant_every_bf16_value():
    log("quantize+requant every bf16 value")
    x = bf16_from_bits(all_bf16_bits(512))
    _quantize_requant_case(x, [x.shape[0]], True)


@pytest.mark.parametrize("name", ["small_moe8", "small_skewed"])
def test_quantize_requant_workloads(name):
    log(f"quantize+requant workload {name}")
    w = wl.make(name)
    _quantize_requant_case(w.tensors["dy"], [int(v) for v in w.m_splits], True)
    _quantize_requant_case(w.tensors["x"], [int(v) for v in w.m_splits], False)


def _swiglu_bwd_case(t, f, seed, splits, with_dbias):
    """mxfp8_swiglu_bwd_quantize against the two calls it replaces (every byte,
    and dbias bit for bit), and its quantize part against the oracle applied
    to the device's dh (which test_swiglu pins to within a bf16 ulp of the
    oracle's SwiGLU backward)."""
    h_cpu = _swiglu_input(t, f, seed)
    rng = np.random.default_rng(seed + 1000)
    da_cpu = torch.from_numpy(rng.standard_normal((t, f)).astype(np.float32)).to(torch.bfloat16)
    h, da = h_cpu.to("cuda"), da_cpu.to("cuda")
    ms = dev(np.asarray(splits, dtype=np.int64))
    dh = mx.swiglu_bwd(h, da)
    if with_dbias:
        ref, refdb = mx.group_quantize_requant(dh, ms, with_dbias=True)
        got, db = mx.swiglu_bwd_quantize(h, da, ms, with_dbias=True)
    else:
        ref = mx.group_quantize_requant(dh)
        got = mx.swiglu_bwd_quantize(h, da)
    torch.cuda.synchronize()
    for a, b in zip(_mx_bytes(got), _mx_bytes(ref)):
        assert np.array_equal(a, b)
    if with_dbias:
        assert torch.equal(db.view(torch.uint8), refdb.view(torch.uint8))
    dh64 = f64(dh)
    assert og.within_bf16_ulp(dh64, osw.swiglu_bwd(f64(h_cpu), f64(da_cpu))).all()
    q, s = om.quantize_rowwise(dh64)
    cq, cs = om.requant_colwise(q, s, splits)
    assert np.array_equal(u8(got.row_data), q) and np.array_equal(u8(got.row_scale), s)
    assert np.array_equal(u8(got.col_data), cq) and np.array_equal(u8(got.col_scale), cs)
    if with_dbias:
        ref_db = om.grouped_dbias(q, s, splits)
        absx = np.abs(om.dequantize_rowwise(q, s))
        bound = np.zeros_like(ref_db)
        start = 0
        for g, m in enumerate(splits):
            bound[g] = absx[start:start + m].sum(axis=0)
            start += m
        assert np.all(np.abs(db.cpu().numpy().astype(np.float64) - ref_db) <= 1e-5 * bound + 1e-6)


@pytest.mark.parametrize("t,f,seed,splits", [
    (256, 256, 41, [256]),
    (384, 512, 42, [128, 0, 256]),
    (1024, 1536, 43, [384, 128, 0, 512]),
])
@pytest.mark.parametrize("with_dbias", [False, True])
def test_swiglu_bwd_quantize(t, f, seed, splits, with_dbias):
    log(f"swiglu_bwd_quantize {t}x{f} splits {splits} dbias {with_dbias}")
    _swiglu_bwd_case(t, f, seed, splits, with_dbias)


def test_swiglu_bwd_quantize_reuses_outputs():
    log("swiglu_bwd_quantize reuses outputs")
    t, f = 256, 512
    h1, h2 = _swiglu_input(t, f, 51).to("cuda"), _swiglu_input(t, f, 52).to("cuda")
    da = torch.ones(t, f, dtype=torch.bfloat16, device="cuda")
    out = mx.swiglu_bwd_quantize(h1, da)
    ptrs = (out.row_data.data_ptr(), out.col_data.data_ptr())
    out = mx.swiglu_bwd_quantize(h2, da, out=out)
    ref = mx.group_quantize_requant(mx.swiglu_bwd(h2, da))
    torch.cuda.synchronize()
    assert (out.row_data.data_ptr(), out.col_data.data_ptr()) == ptrs
    for a, b in zip(_mx_bytes(out), _mx_bytes(ref)):
        assert np.array_equal(a, b)
