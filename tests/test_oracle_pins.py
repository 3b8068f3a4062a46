"""Pins of the CPU oracle to facts outside itself (no GPU).

Each test checks the oracle against something it does not compute itself:
the OCP format tables (golden files), hand-derived block conversions, a
brute-force nearest-value search, torch's own float8_e4m3fn conversion, exact
rational arithmetic, and invariants the definitions imply.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import gemm as ogemm
from oracle import mxfp8 as om
from oracle import swiglu as osw

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def _parse_value(tok):
    if tok == "nan":
        return float("nan")
    if tok == "-0":
        return -0.0
    sign = -1.0 if tok.startswith("-") else 1.0
    tok = tok.lstrip("-")
    if "*" in tok:
        a, b = tok.split("*")
        return sign * float(a) * _parse_value(b)
    if "^" in tok:
        base, exp = tok.split("^")
        return sign * float(base) ** int(exp)
    if "/" in tok:
        a, b = tok.split("/")
        return sign * float(Fraction(int(a), int(b)))
    return sign * float(tok)


def _all_e4m3_values():
    """All 127 non-negative finite E4M3 magnitudes, built from the format's
    definition (not from the oracle): subnormals m*2^-9, normals
    (1+m/8)*2^(e-7), largest 448."""
    vals = [m * 2.0 ** -9 for m in range(8)]
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            vals.append((1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


def _all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    return f[np.isfinite(f)].astype(np.float64)


# ----------------------------------------------------------------------------
# codecs
# ----------------------------------------------------------------------------

def test_e4m3_decode_golden():
    for line in _golden_lines("e4m3_codes.txt"):
        code, val = line.split()
        got = om.decode_e4m3(np.uint8(int(code, 16)))
        want = _parse_value(val)
        if math.isnan(want):
            assert np.isnan(got)
        else:
            assert got == want and np.signbit(got) == np.signbit(want), (code, got, want)


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = om.decode_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    assert nan.sum() == 2  # only 0x7F and 0xFF


def test_e8m0_decode():
    u = np.arange(255, dtype=np.uint8)
    got = om.decode_e8m0(u)
    assert np.array_equal(got, [2.0 ** (int(v) - 127) for v in u])
    assert np.isnan(om.decode_e8m0(np.uint8(255)))


def _bruteforce_encode(y):
    """Nearest E4M3 magnitude by exhaustive search; ties to the even code."""
    table = _all_e4m3_values()                       # index == 7-bit code
    a = np.minimum(np.abs(y), 448.0)
    d = np.abs(a[:, None] - table[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among tied candidates prefer the even code
    even = cand & (np.arange(table.size)[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return (pick | (np.signbit(y).astype(np.int64) << 7)).astype(np.uint8)


def test_encode_vs_bruteforce_all_bf16():
    y = _all_finite_bf16()
    assert np.array_equal(om.encode_e4m3(y), _bruteforce_encode(y))


def test_encode_vs_bruteforce_midpoints():
    # exact midpoints between neighbouring E4M3 values (and just off them)
    t = _all_e4m3_values()
    mids = (t[:-1] + t[1:]) / 2
    y = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 1), -mids,
                        [448.0, 464.0, np.nextafter(464.0, 0), 480.0, 1e30, 2.0 ** -10]])
    assert np.array_equal(om.encode_e4m3(y), _bruteforce_encode(y))


def test_encode_vs_torch_cast_all_bf16():
    y = _all_finite_bf16()
    ref = torch.from_numpy(y).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(om.encode_e4m3(y), ref)


def test_shared_exponent_closed_forms():
    cases = {1.0: -8, 1.5: -8, 2.0: -7, 448.0: 0, 0.0: -127, 2.0 ** -126: -127,
             2.0 ** -130: -127, 2.0 ** -118: -126, 2.0 ** 127: 119,
             3.00405527047391e38: 119, 255.0: -1, 256.0: 0, 2.0 ** -119: -127}
    for amax, x in cases.items():
        assert om.shared_exponent(np.float64(amax)) == x, amax


# ----------------------------------------------------------------------------
# block quantization
# ----------------------------------------------------------------------------

def _golden_blocks():
    for line in _golden_lines("mx_block_cases.txt"):
        name, vals, sbyte, codes = [p.strip() for p in line.split(";")]
        x = np.zeros(32)
        for tok in vals.split():
            i, v = tok.split(":")
            x[int(i)] = float(v)
        want = np.zeros(32, dtype=np.uint8)
        for tok in codes.split():
            i, c = tok.split(":")
            want[int(i)] = int(c, 16)
        yield name, x, int(sbyte), want


def test_block_golden_cases():
    n = 0
    for name, x, sbyte, want in _golden_blocks():
        q, s = om.quantize_rowwise(x[None, :])
        assert s[0, 0] == sbyte, name
        assert np.array_equal(q[0], want), (name, q[0], want)
        n += 1
    assert n >= 15


def test_scale_shape_golden():
    for line in _golden_lines("scale_shape.txt"):
        t, k, r, c = map(int, line.split())
        assert om.scale_shape(t, k) == (r, c)


def _bf16_values(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).double().numpy()


def test_power_of_two_equivariance():
    # Q(2^j x) has the same codes and scale + j (no clamping in range)
    rng = np.random.default_rng(7)
    x = _bf16_values(rng, (64, 256))
    q0, s0 = om.quantize_rowwise(x)
    for j in (-20, -3, 1, 9, 40):
        q1, s1 = om.quantize_rowwise(np.ldexp(x, j))
        assert np.array_equal(q0, q1)
        assert np.array_equal(s1.astype(int), s0.astype(int) + j)


def test_round_trip_idempotent():
    # dequantized MXFP8 blocks are exactly representable: re-quantizing them
    # reproduces the values (lossless round trip) and the same bytes
    rng = np.random.default_rng(8)
    x = _bf16_values(rng, (96, 512), 3.0)
    x[5, :32] = 0.0
    q, s = om.quantize_rowwise(x)
    xh = om.dequantize_rowwise(q, s)
    q2, s2 = om.quantize_rowwise(xh)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    assert np.array_equal(om.dequantize_rowwise(q2, s2), xh)


def test_quantization_error_bound():
    # |x - deq(Q(x))| <= half the E4M3 spacing at x / 2^X (times 2^X), or the
    # clipped amount for saturated elements
    rng = np.random.default_rng(9)
    x = _bf16_values(rng, (128, 256), 10.0)
    q, s = om.quantize_rowwise(x)
    xh = om.dequantize_rowwise(q, s)
    X = (s.astype(np.int64) - 127).repeat(32, axis=1)
    y = np.abs(x) / np.exp2(X)
    ey = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
    half_spacing = np.exp2(ey - 3) / 2 * np.exp2(X)
    sat = y > 448
    err = np.abs(x - xh)
    assert np.all(err[~sat] <= half_spacing[~sat])
    assert np.all(np.abs(xh[sat]) == 448 * np.exp2(X[sat]))
    # the block max is never flushed: its code has the top exponent field 15
    blk_max_code = (q.reshape(128, 8, 32) & 0x7F).max(axis=2)
    assert np.all(blk_max_code >> 3 == 15)


def test_colwise_equals_rowwise_of_transpose():
    rng = np.random.default_rng(10)
    x = _bf16_values(rng, (512, 64))
    qc, sc = om.quantize_colwise(x, [128, 0, 256, 128])
    qr, sr = om.quantize_rowwise(x.T.copy())
    assert np.array_equal(qc, qr) and np.array_equal(sc, sr)


def test_colwise_blocks_by_hand():
    # one column, one block: codes must equal the row-wise encoding of that
    # column's 32 values, computed element by element here
    rng = np.random.default_rng(11)
    x = _bf16_values(rng, (256, 32))
    qc, sc = om.quantize_colwise(x, [128, 128])
    for col in (0, 17, 31):
        for blk in range(8):
            v = x[32 * blk:32 * blk + 32, col]
            amax = np.abs(v).max()
            e = math.frexp(amax)[1] - 1 - 8
            assert sc[col, blk] == e + 127
            for i in range(32):
                y = math.ldexp(v[i], -e)
                assert qc[col, 32 * blk + i] == _bruteforce_encode(np.array([y]))[0]


def test_requant_colwise_and_dbias():
    rng = np.random.default_rng(12)
    splits = [128, 0, 256]
    x = _bf16_values(rng, (384, 64), 2.0)
    q, s = om.quantize_rowwise(x)
    qc, sc = om.requant_colwise(q, s, splits)
    xh = om.dequantize_rowwise(q, s)
    qc2, sc2 = om.quantize_rowwise(xh.T.copy())
    assert np.array_equal(qc, qc2) and np.array_equal(sc, sc2)
    db = om.grouped_dbias(q, s, splits)
    # by hand: Python loop over rows in each group
    want = np.zeros((3, 64))
    row = 0
    for g, m in enumerate(splits):
        for r in range(row, row + m):
            want[g] += xh[r]
        row += m
    assert np.allclose(db, want, rtol=0, atol=1e-12)
    assert np.all(db[1] == 0)


def test_requant_can_clip():
    # a column whose max has significand 1.875 (E4M3 code 0x3F) re-quantizes
    # with scale 2^(0-8) and saturates to 448 (480 is not an E4M3 value)
    q = np.zeros((128, 32), dtype=np.uint8)
    s = np.full((128, 1), 127, dtype=np.uint8)
    q[0, 0] = 0x3F
    qc, sc = om.requant_colwise(q, s, [128])
    assert sc[0, 0] == 127 - 8
    assert qc[0, 0] == 0x7E


def test_scaled_bias_grad_special_cases_and_bruteforce():
    """Unit scales give the ordinary grouped dbias; a zero bias gives zero
    dscales; both outputs are linear in the scales / the bias; and a tiny
    case is checked element by element with Python loops."""
    rng = np.random.default_rng(31)
    splits = [128, 0, 256]
    t, n = sum(splits), 64
    q = rng.integers(0, 256, size=(t, n)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x7E
    s = rng.integers(120, 134, size=(t, n // 32)).astype(np.uint8)
    ones = np.ones(t)
    bias = rng.standard_normal((3, n))
    db1, _ = om.grouped_scaled_bias_grad(q, s, splits, ones, bias)
    assert np.allclose(db1, om.grouped_dbias(q, s, splits), rtol=1e-12, atol=0)
    _, ds0 = om.grouped_scaled_bias_grad(q, s, splits, ones, np.zeros((3, n)))
    assert np.all(ds0 == 0)
    sc = rng.random(t)
    db_a, ds_a = om.grouped_scaled_bias_grad(q, s, splits, sc, bias)
    db_b, ds_b = om.grouped_scaled_bias_grad(q, s, splits, 2 * sc, 3 * bias)
    assert np.allclose(db_b, 2 * db_a, rtol=1e-12) and np.allclose(ds_b, 3 * ds_a, rtol=1e-12)
    assert np.all(db_a[1] == 0)
    xh = om.dequantize_rowwise(q, s)
    group_of = [0] * 128 + [2] * 256
    for r in range(0, t, 29):
        want = 0.0
        for c in range(n):
            want += float(xh[r, c]) * float(bias[group_of[r], c])
        assert abs(ds_a[r] - want) <= 1e-9 * (abs(want) + 1)
    for g, (r0, r1) in [(0, (0, 128)), (2, (128, 384))]:
        for c in range(0, n, 7):
            want = 0.0
            for r in range(r0, r1):
                want += float(sc[r]) * float(xh[r, c])
            assert abs(db_a[g, c] - want) <= 1e-9 * (abs(want) + 1)


# ----------------------------------------------------------------------------
# grouped GEMM
# ----------------------------------------------------------------------------

def _rand_mx(rng, rows, cols, smin=120, smax=134):
    q = rng.integers(0, 256, size=(rows, cols)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x00                     # no NaN codes
    s = rng.integers(smin, smax, size=(rows, cols // 32)).astype(np.uint8)
    return q, s


def _exact(code, sbyte):
    """Exact rational value of one MXFP8 element, from the bit fields."""
    c = int(code)
    sign = -1 if c & 0x80 else 1
    e, m = (c >> 3) & 15, c & 7
    mag = Fraction(m, 2 ** 9) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
    return sign * mag * Fraction(2) ** (int(sbyte) - 127)


def test_fprop_exact_rational():
    rng = np.random.default_rng(20)
    G, N, K, splits = 3, 4, 64, [128, 0, 128]
    T = sum(splits)
    xq, xs = _rand_mx(rng, T, K)
    wq, ws = _rand_mx(rng, G * N, K)
    out = ogemm.fprop(xq, xs, wq.reshape(G, N, K), ws.reshape(G, N, K // 32), splits)
    for t in range(0, T, 37):
        g = 0 if t < 128 else 2
        for n in range(N):
            acc = sum(_exact(xq[t, k], xs[t, k // 32]) * _exact(wq[g * N + n, k], ws[g * N + n, k // 32])
                      for k in range(K))
            assert out[t, n] == float(acc), (t, n)


def test_dgrad_exact_rational():
    rng = np.random.default_rng(21)
    G, N, K, splits = 2, 64, 32, [128, 128]
    T = sum(splits)
    dyq, dys = _rand_mx(rng, T, N)
    wcq, wcs = _rand_mx(rng, K, G * N)               # column-wise W copy: [K, G*N]
    out = ogemm.dgrad(dyq, dys, wcq, wcs, splits, G)
    for t in range(0, T, 41):
        g = t // 128
        for k in range(0, K, 5):
            acc = sum(_exact(dyq[t, n], dys[t, n // 32]) *
                      _exact(wcq[k, g * N + n], wcs[k, (g * N + n) // 32]) for n in range(N))
            assert out[t, k] == float(acc), (t, k)


def test_wgrad_exact_rational():
    rng = np.random.default_rng(22)
    N, K, splits = 3, 4, [128, 0, 128]
    T = sum(splits)
    dycq, dycs = _rand_mx(rng, N, T)
    xcq, xcs = _rand_mx(rng, K, T)
    out = ogemm.wgrad(dycq, dycs, xcq, xcs, splits)
    assert out.shape == (3, N, K)
    assert np.all(out[1] == 0)
    for g, (r0, r1) in enumerate([(0, 128), (128, 128), (128, 256)]):
        for n in range(N):
            for k in range(K):
                acc = sum(_exact(dycq[n, t], dycs[n, t // 32]) * _exact(xcq[k, t], xcs[k, t // 32])
                          for t in range(r0, r1))
                assert out[g, n, k] == float(acc), (g, n, k)


def test_wgrad_accumulate_exact_rational():
    """main_grad + dY_g^T X_g against exact rational sums (the fp32 base
    value plus the exact product, rounded once); an expert without rows
    keeps its slice bit for bit, negative zeros included."""
    rng = np.random.default_rng(24)
    N, K, splits = 3, 4, [128, 0, 128]
    T = sum(splits)
    dycq, dycs = _rand_mx(rng, N, T)
    xcq, xcs = _rand_mx(rng, K, T)
    base = rng.standard_normal((3, N, K)).astype(np.float32)
    base[1, 0, :] = -0.0
    out = ogemm.wgrad_accumulate(base, dycq, dycs, xcq, xcs, splits)
    assert np.array_equal(out[1].astype(np.float32).view(np.uint32), base[1].view(np.uint32))
    for g, (r0, r1) in [(0, (0, 128)), (2, (128, 256))]:
        for n in range(N):
            for k in range(K):
                acc = Fraction(float(base[g, n, k])) + sum(
                    _exact(dycq[n, t], dycs[n, t // 32]) * _exact(xcq[k, t], xcs[k, t // 32])
                    for t in range(r0, r1))
                assert out[g, n, k] == float(acc), (g, n, k)
    # a zero base gives the plain wgrad
    zero = np.zeros((3, N, K), dtype=np.float32)
    assert np.array_equal(ogemm.wgrad_accumulate(zero, dycq, dycs, xcq, xcs, splits),
                          ogemm.wgrad(dycq, dycs, xcq, xcs, splits))


def test_grouped_equals_per_group_and_dense():
    rng = np.random.default_rng(23)
    G, N, K, splits = 4, 64, 128, [256, 0, 128, 128]
    T = sum(splits)
    xq, xs = _rand_mx(rng, T, K)
    wq, ws = _rand_mx(rng, G * N, K)
    out = ogemm.fprop(xq, xs, wq.reshape(G, N, K), ws.reshape(G, N, K // 32), splits)
    off = 0
    for g, m in enumerate(splits):
        single = ogemm.fprop(xq[off:off + m], xs[off:off + m], wq[g * N:(g + 1) * N][None],
                             ws[g * N:(g + 1) * N][None], [m])
        assert np.array_equal(out[off:off + m], single)
        off += m
    # G = 1 is the dense GEMM
    dense = om.dequantize_rowwise(xq, xs) @ om.dequantize_rowwise(wq[:N], ws[:N]).T
    one = ogemm.fprop(xq, xs, wq[:N][None], ws[:N][None], [T])
    assert np.array_equal(one, dense)


def test_expert_permutation():
    rng = np.random.default_rng(24)
    G, N, K, splits = 3, 32, 64, [128, 256, 128]
    T = sum(splits)
    xq, xs = _rand_mx(rng, T, K)
    wq, ws = _rand_mx(rng, G * N, K)
    wq3, ws3 = wq.reshape(G, N, K), ws.reshape(G, N, K // 32)
    out = ogemm.fprop(xq, xs, wq3, ws3, splits)
    perm = [2, 0, 1]
    offs = np.concatenate([[0], np.cumsum(splits)])
    rows = np.concatenate([np.arange(offs[p], offs[p + 1]) for p in perm])
    out_p = ogemm.fprop(xq[rows], xs[rows], wq3[perm], ws3[perm], [splits[p] for p in perm])
    assert np.array_equal(out_p, out[rows])


def test_tolerance_closed_form():
    assert ogemm.tolerance_f32(0.0) == 1e-6
    assert ogemm.tolerance_f32(1e5) == pytest.approx(1.0 + 1e-6)


def test_round_to_bf16_matches_torch_from_f32():
    rng = np.random.default_rng(26)
    x = rng.standard_normal(20000).astype(np.float32).astype(np.float64) * 100
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(om.round_to_bf16(x), want)
    assert np.all(om.bf16_ulp(np.array([1.0, 1.5, 2.0])) == [2.0 ** -7, 2.0 ** -7, 2.0 ** -6])


# ----------------------------------------------------------------------------
# SwiGLU (parity unpinned by the pages; pinned here to calculus only)
# ----------------------------------------------------------------------------

def test_swiglu_closed_forms():
    h = np.array([[0.0, 3.0], [50.0, 2.0], [-50.0, 2.0], [1.0, 1.0]])
    a = osw.swiglu_fwd(h)[:, 0]
    assert a[0] == 0.0
    assert a[1] == pytest.approx(100.0)
    assert abs(a[2]) < 1e-18
    assert a[3] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)))


def test_swiglu_bwd_finite_difference():
    rng = np.random.default_rng(27)
    h = rng.standard_normal((16, 8)) * 2
    da = rng.standard_normal((16, 4))
    dh = osw.swiglu_bwd(h, da)
    eps = 1e-6
    num = np.zeros_like(h)
    for i in range(h.shape[0]):
        for j in range(h.shape[1]):
            hp, hm = h.copy(), h.copy()
            hp[i, j] += eps
            hm[i, j] -= eps
            num[i, j] = ((osw.swiglu_fwd(hp) - osw.swiglu_fwd(hm)) * da).sum() / (2 * eps)
    assert np.allclose(dh, num, rtol=1e-6, atol=1e-8)


def test_window_run_max_bruteforce():
    from oracle.gemm import _window_run_max
    rng = np.random.default_rng(28)
    a = np.abs(rng.standard_normal((3, 256)))
    b = np.abs(rng.standard_normal((2, 256)))
    got = _window_run_max(a, b)
    for i in range(3):
        for j in range(2):
            total = 0.0
            for w0 in (0, 128):
                runs = [sum(a[i, k] * b[j, k] for k in range(r0, r0 + 8)) for r0 in range(w0, w0 + 128, 8)]
                total += max(runs)
            assert got[i, j] == pytest.approx(total, rel=1e-12)


def test_tolerance_mfma_closed_form():
    assert ogemm.tolerance_mfma(0.0, 0.0) == 1e-6
    assert ogemm.tolerance_mfma(1e5, 2.0 ** 9) == pytest.approx(1.0 + 1.0 + 1e-6)
