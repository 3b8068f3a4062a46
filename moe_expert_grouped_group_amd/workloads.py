"""Seeded synthetic inputs for the MXFP8 grouped-GEMM hot path.

This module only draws random numbers and rounds them to bf16 (with
torch's CPU conversion); it holds none of the method's arithmetic, so both
the HIP path and the CPU oracle take their inputs from it.

Every tensor is drawn in float32 from ``numpy.random.default_rng`` with the
key ``[workload id, stream, chunk]`` (chunks of 8192 rows), then rounded to
bf16.  Streams: 0 routing, 1 X, 2 W (FC1 weight), 3 dY, 4 W2 (FC2 weight),
5 masks (outliers, zero tiles).  Routing splits are multiples of 128 rows
(the per-expert alignment of the FP8 dispatch) and sum to the token count.

Workloads (sizes as the expert layers they stand for; no trained weights or
routing traces are involved):

* ``tiny_fwd``: 4 experts x 128 tokens, K = N = 512; forward only.
* ``moe8_h4096_f14336``: 8 experts, hidden 4096 -> expert FFN 14336 (one
  linear), 16384 tokens routed by Dirichlet(1) multinomial; forward, dgrad,
  wgrad and dbias.
* ``nemotron_proxy_mlp``: 64 experts, 83968 tokens (656 x 128), hidden 3072,
  FC1 3072 -> 2048 (SwiGLU to 1024), FC2 1024 -> 3072; Zipf(1.1) routing.
* ``skewed_dsv3``: 128 experts, hidden 7168 -> 2048, 32768 tokens; 38
  experts empty, the other 90 get 1 + Multinomial(166, Zipf(1.5)) units of
  128; X ~ N(0,1) with 0.1 % of elements scaled by 1000.
* ``group_quantize_131072x7168``: 131072 x 7168 bf16, 256 groups from a
  Dirichlet(1) multinomial; Student-t(3) values with 1 % of the aligned
  32 x 32 tiles set to zero.

``small_*`` variants keep each recipe at sizes a float64 CPU oracle
finishes in seconds while still spanning several 256-wide tiles.
"""

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import os

import numpy as np
import torch

ALIGN = 128
CHUNK_ROWS = 8192

STREAM_ROUTING, STREAM_X, STREAM_W, STREAM_DY, STREAM_W2, STREAM_MASK = range(6)


def _rng(key):
    return np.random.default_rng([int(v) for v in key])


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ----------------------------------------------------------------------------
# routing (m_splits)
# ----------------------------------------------------------------------------

def routing_dirichlet(wid, groups, tokens, alpha=1.0):
    units = tokens // ALIGN
    r = _rng([wid, STREAM_ROUTING])
    p = r.dirichlet(np.full(groups, alpha))
    return (r.multinomial(units, p) * ALIGN).astype(np.int64)


def routing_zipf(wid, groups, tokens, s):
    """Truncated Zipf(s) over the experts (rank r has weight r^-s), ranks permuted."""
    units = tokens // ALIGN
    r = _rng([wid, STREAM_ROUTING])
    w = np.arange(1, groups + 1, dtype=np.float64) ** -s
    p = (w / w.sum())[r.permutation(groups)]
    return (r.multinomial(units, p) * ALIGN).astype(np.int64)


def routing_skewed(wid, groups, tokens, n_empty, s):
    """n_empty experts get nothing; each other expert 1 unit plus a Zipf(s) share."""
    units = tokens // ALIGN
    r = _rng([wid, STREAM_ROUTING])
    empty = r.choice(groups, size=n_empty, replace=False)
    live = np.setdiff1d(np.arange(groups), empty)
    w = np.arange(1, live.size + 1, dtype=np.float64) ** -s
    p = (w / w.sum())[r.permutation(live.size)]
    counts = np.zeros(groups, dtype=np.int64)
    counts[live] = 1 + r.multinomial(units - live.size, p)
    return counts * ALIGN


# ----------------------------------------------------------------------------
# bf16 tensors
# ----------------------------------------------------------------------------

def _fill_chunks(shape, key, draw):
    """Draw a float32 [rows, cols] array chunk by chunk (8192 rows per chunk)."""
    rows, cols = shape
    out = np.empty((rows, cols), dtype=np.float32)
    starts = list(range(0, rows, CHUNK_ROWS))

    def work(ci):
        r0 = starts[ci]
        r1 = min(rows, r0 + CHUNK_ROWS)
        out[r0:r1] = draw(_rng(list(key) + [ci]), (r1 - r0, cols))

    if len(starts) == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(len(starts))))
    return out


def to_bf16(a):
    """float32 numpy -> bf16 torch CPU tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def bf16_normal(key, shape, std=1.0):
    def draw(r, sh):
        v = r.standard_normal(sh, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        return v
    return to_bf16(_fill_chunks(shape, key, draw))


def bf16_normal_outliers(key, shape, frac, factor):
    """N(0,1) with a fraction `frac` of elements multiplied by `factor`."""
    def draw(r, sh):
        v = r.standard_normal(sh, dtype=np.float32)
        mask = r.random(sh, dtype=np.float32) < frac
        v[mask] *= np.float32(factor)
        return v
    return to_bf16(_fill_chunks(shape, key, draw))


def bf16_student_t_zero_tiles(key, shape, df, zero_frac):
    """Student-t(df) values; a fraction of the aligned 32 x 32 tiles set to 0."""
    def draw(r, sh):
        z = r.standard_normal(sh, dtype=np.float32)
        chi = np.zeros(sh, dtype=np.float32)
        for _ in range(df):
            g = r.standard_normal(sh, dtype=np.float32)
            chi += g * g
        v = z / np.sqrt(chi / np.float32(df))
        tr, tc = sh[0] // 32, sh[1] // 32
        zt = r.random((tr, tc)) < zero_frac
        v.reshape(tr, 32, tc, 32)[zt[:, None, :, None].repeat(32, 1).repeat(32, 3)] = 0.0
        return v
    return to_bf16(_fill_chunks(shape, key, draw))


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    wid: int
    groups: int
    tokens: int
    hidden: int                 # K of the first linear (input features)
    ffn: int                    # N of the first linear (output features)
    m_splits: np.ndarray
    out_dtype: str = "f32"      # GEMM output dtype
    ffn2: int = 0               # FC2 input features (fused MLP only)
    tensors: dict = field(default_factory=dict)

    @property
    def flops_linear(self):
        return 2.0 * self.tokens * self.hidden * self.ffn


_SPECS = {
    # name: (wid, G, T, K, N, routing, out dtype)
    "tiny_fwd": (1, 4, 512, 512, 512, ("fixed", [128] * 4), "f32"),
    "moe8_h4096_f14336": (2, 8, 16384, 4096, 14336, ("dirichlet", 1.0), "f32"),
    "nemotron_proxy_mlp": (3, 64, 83968, 3072, 2048, ("zipf", 1.1), "bf16"),
    "skewed_dsv3": (4, 128, 32768, 7168, 2048, ("skewed", 38, 1.5), "f32"),
    "group_quantize_131072x7168": (5, 256, 131072, 7168, 0, ("dirichlet", 1.0), "f32"),
    # small versions of the same recipes (own workload ids, same streams)
    "small_moe8": (12, 8, 2048, 512, 1024, ("dirichlet", 1.0), "f32"),
    "small_nemotron_mlp": (13, 16, 4096, 512, 1024, ("zipf", 1.1), "bf16"),
    "small_skewed": (14, 32, 4096, 512, 512, ("skewed", 10, 1.5), "f32"),
    "small_group_quantize": (15, 24, 3072, 1536, 0, ("dirichlet", 1.0), "f32"),
}

WORKLOAD_NAMES = tuple(_SPECS)


def splits_for(name):
    wid, g, t, _k, _n, routing, _ = _SPECS[name]
    kind = routing[0]
    if kind == "fixed":
        return np.asarray(routing[1], dtype=np.int64)
    if kind == "dirichlet":
        return routing_dirichlet(wid, g, t, routing[1])
    if kind == "zipf":
        return routing_zipf(wid, g, t, routing[1])
    if kind == "skewed":
        return routing_skewed(wid, g, t, routing[1], routing[2])
    raise KeyError(kind)


def make(name, parts=None):
    """Build a workload's routing and the bf16 tensors named in `parts`.

    parts (default: all the workload uses): subset of
    {"x", "w", "dy", "w2"}.  Shapes: x [T, K], w [G, N, K], dy [T, N];
    the fused MLP also has w2 [G, K, N/2] (FC2: N/2 -> K) and dy is then the
    gradient of the FC2 output, [T, K].
    """
    wid, g, t, k, n, _routing, out_dtype = _SPECS[name]
    wl = Workload(name=name, wid=wid, groups=g, tokens=t, hidden=k, ffn=n,
                  m_splits=splits_for(name), out_dtype=out_dtype)
    mlp = "nemotron" in name
    if mlp:
        wl.ffn2 = n // 2
    quant_only = n == 0
    if parts is None:
        parts = {"x"} if quant_only else ({"x", "w", "dy", "w2"} if mlp else {"x", "w", "dy"})
    if "x" in parts:
        if quant_only:
            wl.tensors["x"] = bf16_student_t_zero_tiles([wid, STREAM_X], (t, k), 3, 0.01)
        elif "skewed" in name:
            wl.tensors["x"] = bf16_normal_outliers([wid, STREAM_X], (t, k), 1e-3, 1000.0)
        else:
            wl.tensors["x"] = bf16_normal([wid, STREAM_X], (t, k))
    if "w" in parts:
        wl.tensors["w"] = bf16_normal([wid, STREAM_W], (g * n, k), 0.02).view(g, n, k)
    if "dy" in parts:
        wl.tensors["dy"] = bf16_normal([wid, STREAM_DY], (t, k if mlp else n))
    if "w2" in parts and mlp:
        wl.tensors["w2"] = bf16_normal([wid, STREAM_W2], (g * k, n // 2), 0.02).view(g, k, n // 2)
    return wl
