"""The device conversion helpers against the oracle's codec over every
(value, scale byte) pair (OCP Microscaling Formats v1.0: E4M3 element
encoding, section 5.3; E8M0 scale, section 5.4; block conversion, section
6.3).  Every quantize kernel encodes and decodes through these helpers, so
this sweep is what makes their bytes exact for any input, not only for the
sampled tensors of the other parity tests.

Domains (what the kernels can present to the helpers):
* encode of a bf16 value v with scale byte s (X = s - 127): every finite bf16
  with |v| / 2^X < 512, i.e. X >= floor(log2 |v|) - 8 (the block maximum sets
  X, so no element exceeds that bound); all scale bytes 0..254;
* requantize of code c decoded with row scale byte s and encoded with column
  block byte x: s in 0..246 (the kernels take their integer path above that),
  every non-NaN code, x with X >= floor(log2 |c 2^S|) - 8;
* decode with scale bytes 0..246: the exact value code * 2^S as fp32.
"""

import numpy as np
import pytest

import moe_expert_grouped_group_amd as mx
from oracle import mxfp8 as om

from gpu_util import log

pytestmark = pytest.mark.gpu

MAX_FAST_SCALE_BYTE = 246


def _floor_log2(v):
    """floor(log2 |v|) of non-zero float64 values (frexp, exact); -10^6 for 0."""
    _, p = np.frexp(np.abs(v))
    return np.where(v != 0, p - 1, -10 ** 6)


def test_encode_every_bf16_and_scale():
    log("convert sweep: encode bf16")
    got = mx.convert_sweep(0).cpu().numpy().view(np.uint16).reshape(256, 1 << 16)
    h = np.arange(1 << 16, dtype=np.uint32)
    finite = (h & 0x7F80) != 0x7F80
    with np.errstate(invalid="ignore"):      # the NaN patterns, excluded below
        v = np.where(finite, (h << 16).view(np.float32).astype(np.float64), 0.0)
    fl = _floor_log2(np.where(finite, v, 0.0))
    checked = 0
    for s in range(255):
        x = s - 127
        dom = finite & (fl - 8 <= x)
        y = np.where(dom, v, 0.0) / 2.0 ** x
        want = om.encode_e4m3(y).astype(np.uint16) | (om.encode_e4m3(-y).astype(np.uint16) << 8)
        bad = dom & (got[s] != want)
        assert not bad.any(), (s, [hex(int(b)) for b in h[bad][:4]])
        checked += int(dom.sum())
    assert checked > 8_000_000


def test_requantize_every_code_and_scale_pair():
    log("convert sweep: requantize")
    got = mx.convert_sweep(1).cpu().numpy().reshape(256, 256, 256)   # [x, s, c]
    c = np.arange(256)
    val = om.decode_e4m3(c.astype(np.uint8))
    ok = ~np.isnan(val)
    checked = 0
    for s in range(MAX_FAST_SCALE_BYTE + 1):
        d = np.where(ok, val, 0.0) * 2.0 ** (s - 127)
        fl = _floor_log2(d)
        for xb in range(255):
            x = xb - 127
            dom = ok & (fl - 8 <= x)
            want = om.encode_e4m3(np.where(dom, d, 0.0) / 2.0 ** x)
            bad = dom & (got[xb, s] != want)
            assert not bad.any(), (s, xb, np.nonzero(bad)[0][:4])
            checked += int(dom.sum())
    assert checked > 8_000_000


def test_decode_every_code_and_scale():
    log("convert sweep: decode")
    got = mx.convert_sweep(2).cpu().numpy().view(np.uint32).reshape(256, 256, 2)
    c = np.arange(256)
    val = om.decode_e4m3(c.astype(np.uint8))
    for s in range(MAX_FAST_SCALE_BYTE + 1):
        want = val * 2.0 ** (s - 127)
        for k, sign in ((0, 1.0), (1, -1.0)):
            g = got[s, :, k].view(np.float32).astype(np.float64)
            ok = np.isnan(want) | (g == sign * want)
            # the sign of a decoded zero is kept
            ok &= (want != 0) | (np.signbit(g) == (np.signbit(val) if sign > 0 else ~np.signbit(val)))
            assert ok.all(), (s, k, np.nonzero(~ok)[0][:4])
