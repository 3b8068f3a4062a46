"""Helpers shared by the GPU parity tests (conversion only, no arithmetic of
the method)."""

import sys

import numpy as np
import torch

DEV = "cuda"


def log(msg):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print(msg, file=sys.stderr, flush=True)


def f64(t):
    """bf16/fp32 tensor -> float64 numpy (exact)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def u8(t):
    return t.detach().cpu().numpy()


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)) if isinstance(a, np.ndarray) else a
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def bf16_from_bits(bits):
    """uint16 numpy bit patterns -> bf16 torch CPU tensor (no rounding)."""
    return torch.from_numpy(np.ascontiguousarray(bits.astype(np.uint16)).view(np.int16)).view(
        torch.bfloat16)


def sweep_bf16_bits(rows, cols, seed):
    """bf16 bit patterns that cover the encoder's input space.

    Half of the 32-blocks have an anchor element with a random exponent field
    (1..254) and 31 elements whose exponent fields lie 0..40 below it (field
    0 = subnormal or zero), all with random mantissas and signs; the rest are
    uniformly random finite bit patterns.  A few blocks are all +0 or -0.
    """
    rng = np.random.default_rng(seed)
    nb = rows * cols // 32
    sign = rng.integers(0, 2, size=(nb, 32)) << 15
    mant = rng.integers(0, 128, size=(nb, 32))
    ea = rng.integers(1, 255, size=(nb, 1))
    rel = rng.integers(0, 41, size=(nb, 32))
    rel[:, 0] = 0
    e = np.clip(ea - rel, 0, 254)
    anchored = sign | (e << 7) | mant
    rand = rng.integers(0, 1 << 16, size=(nb, 32))
    rand_e = (rand >> 7) & 0xFF
    rand = np.where(rand_e == 255, rand & ~(1 << 14), rand)   # no inf / NaN
    pick = rng.random((nb, 1)) < 0.5
    bits = np.where(pick, anchored, rand)
    zero_blocks = rng.random(nb) < 0.01
    bits[zero_blocks] = 0
    negz = rng.random(nb) < 0.005
    bits[negz] = 0x8000
    return bits.reshape(rows, cols).astype(np.uint16)


def all_bf16_bits(cols=512):
    """Every finite bf16 pattern once (padded with zeros to whole rows), as
    [R, cols] with R a multiple of 128, in a fixed shuffled order."""
    b = np.arange(1 << 16, dtype=np.uint32)
    b = b[((b >> 7) & 0xFF) != 0xFF]
    rng = np.random.default_rng(1234)
    b = rng.permutation(b)
    per = 128 * cols
    pad = (-b.size) % per
    b = np.concatenate([b, np.zeros(pad, dtype=np.uint32)])
    return b.reshape(-1, cols).astype(np.uint16)


def random_mx(rng, rows, cols, smin=112, smax=142):
    """Random non-NaN E4M3 codes with random E8M0 scales (row-wise layout)."""
    q = rng.integers(0, 256, size=(rows, cols)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x7E
    s = rng.integers(smin, smax + 1, size=(rows, cols // 32)).astype(np.uint8)
    return q, s


def tol_report(tag, got, ref, mag, out_dtype_is_f32, win=None):
    """Record how far a GEMM output sits from the stated bound.

    fp32: the worst |gpu - oracle| / (1e-5 * sum|ab| + 1e-6), and the same
    against the MFMA window bound when `win` is given.  bf16: the worst
    |gpu - bf16(oracle)| in units of one bf16 ulp of bf16(oracle), and the
    count of outputs beyond one ulp.  Printed, and appended as a JSON line to
    the file named by MX_TOL_REPORT when that variable is set.
    """
    import json
    import os

    from oracle import gemm as og
    from oracle import mxfp8 as om

    got = np.asarray(got, dtype=np.float64)
    rec = {"case": tag, "n": int(got.size)}
    if out_dtype_is_f32:
        err = np.abs(got - ref)
        rec["max_err_over_f32_bound"] = float((err / og.tolerance_f32(mag)).max())
        rec["n_over_f32_bound"] = int((err > og.tolerance_f32(mag)).sum())
        if win is not None:
            rec["max_err_over_mfma_bound"] = float((err / og.tolerance_mfma(mag, win)).max())
    else:
        r16 = om.round_to_bf16(ref)
        ulps = np.abs(got - r16) / om.bf16_ulp(r16)
        rec["max_err_in_bf16_ulp"] = float(ulps.max())
        rec["n_over_1_ulp"] = int((ulps > 1).sum())
        rec["max_err_over_ulp_plus_f32_bound"] = float(
            (np.abs(got - r16) / (om.bf16_ulp(r16) + og.tolerance_f32(mag))).max())
    log("TOL " + json.dumps(rec))
    path = os.environ.get("MX_TOL_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")
    return rec
