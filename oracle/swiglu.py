"""SwiGLU between the two expert linears of the fused expert MLP (CPU oracle).

TEST INFRASTRUCTURE ONLY: used by tests and the smoke check; never by the
product path.

PARITY UNPINNED BY THE PAGES.  The fused grouped MLP of "[PyTorch] Fix
distributed BF16 weights and trim NVFP4 saved state in the fused grouped
MLP" (PR #3545, Description) runs FC1 -> activation -> FC2 but the pages do
not define the activation.  The reading adopted here is the usual gated
SiLU: the FC1 output h [T, 2F] is split into a gate half (columns [0, F))
and an up half (columns [F, 2F)), and

    a = silu(gate) * up,   silu(z) = z * sigmoid(z) = z / (1 + exp(-z)).

Backward, for an incoming gradient da:

    d gate = da * up * sigmoid(gate) * (1 + gate * (1 - sigmoid(gate)))
    d up   = da * silu(gate)

All in float64; outputs are compared after rounding to bf16.
"""

import numpy as np


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z * sigmoid(z)


def swiglu_fwd(h):
    """h: float64 [T, 2F] -> a: float64 [T, F]."""
    h = np.asarray(h, dtype=np.float64)
    f = h.shape[1] // 2
    gate, up = h[:, :f], h[:, f:]
    return silu(gate) * up


def swiglu_bwd(h, da):
    """h: [T, 2F], da: [T, F] -> dh: float64 [T, 2F] (gate half, then up half)."""
    h = np.asarray(h, dtype=np.float64)
    da = np.asarray(da, dtype=np.float64)
    f = h.shape[1] // 2
    gate, up = h[:, :f], h[:, f:]
    sg = sigmoid(gate)
    dgate = da * up * sg * (1.0 + gate * (1.0 - sg))
    dup = da * gate * sg
    return np.concatenate([dgate, dup], axis=1)
