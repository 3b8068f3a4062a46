"""The allocation-free fused quantize + requantize
(mxfp8_group_quantize_requant_noalloc: dbias partials in the library's
static per-GPU scratch instead of a caller workspace) against the entry point
with a workspace, byte for byte (dbias bit for bit), on two calls in a row,
the second smaller than the first; and its size limit.  Through the C ABI."""

import numpy as np
import pytest
import torch

import moe_expert_grouped_group_amd as mx
from moe_expert_grouped_group_amd import _native

from gpu_util import log

pytestmark = pytest.mark.gpu


def _splits(t, g, seed):
    rng = np.random.default_rng(seed)
    units = rng.multinomial(t // 128, rng.dirichlet(np.ones(g)))
    return torch.from_numpy((units * 128).astype(np.int64)).cuda()


def _bf16_normal(seed, shape):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    return torch.randn(shape, device="cuda", generator=gen).to(torch.bfloat16)


def _same(a, b, what):
    assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), what


@pytest.mark.parametrize("with_dbias", [True, False])
def test_noalloc_matches_workspace_form_twice(with_dbias):
    """First call 16384 x 14336 over 8 experts (the bench dY: 14336 tiles,
    several per workgroup, 7.3 MB of partials), then 2048 x 1024 over 5
    experts, one of them empty; each against mxfp8_group_quantize_requant
    with its own workspace, on the same inputs."""
    for i, (t, k, g) in enumerate(((16384, 14336, 8), (2048, 1024, 5))):
        x = _bf16_normal(90 + i, (t, k))
        ms = _splits(t, g, 100 + i)
        if i == 1:
            ms[2] += ms[3]
            ms[3] = 0
        log(f"noalloc call {i}: T={t} K={k} G={g} dbias={with_dbias}")
        if with_dbias:
            ref, db_ref = mx.group_quantize_requant(x, ms, with_dbias=True)
            got, db = mx.group_quantize_requant_noalloc(x, ms, with_dbias=True)
        else:
            ref = mx.group_quantize_requant(x)
            got = mx.group_quantize_requant_noalloc(x)
        torch.cuda.synchronize()
        for part in ("row_data", "row_scale", "col_data", "col_scale"):
            _same(getattr(got, part), getattr(ref, part), f"call {i} {part}")
        if with_dbias:
            _same(db, db_ref, f"call {i} dbias")
            if i == 1:
                assert torch.count_nonzero(db[3]).item() == 0
        del x, ref, got


def test_noalloc_size_limit():
    """dbias partials beyond the static scratch are refused on the host
    (EINVAL, ValueError in the binding) before anything is launched; the
    largest T that fits is accepted."""
    lib = _native.load()
    k = 14336
    t_max = (mx.NOALLOC_SCRATCH_BYTES // (k * 4)) * 128
    assert mx.dbias_workspace_bytes(t_max, k) <= mx.NOALLOC_SCRATCH_BYTES
    assert mx.dbias_workspace_bytes(t_max + 128, k) > mx.NOALLOC_SCRATCH_BYTES
    fake = 0x1000   # never dereferenced: the call fails its size check first
    st = lib.mxfp8_group_quantize_requant_noalloc(fake, t_max + 128, k, fake, fake, fake, fake,
                                                  fake, 1, fake, None)
    assert st == _native.MXFP8_EINVAL
    assert b"static scratch" in lib.mxfp8_last_error()
    log(f"noalloc largest T with dbias: {t_max}")
    x = _bf16_normal(91, (t_max, k))
    ms = torch.tensor([t_max // 2, t_max - t_max // 2], dtype=torch.int64).cuda()
    ms = (ms // 128) * 128
    ms[1] = t_max - ms[0]
    ref, db_ref = mx.group_quantize_requant(x, ms, with_dbias=True)
    got, db = mx.group_quantize_requant_noalloc(x, ms, with_dbias=True)
    torch.cuda.synchronize()
    _same(db, db_ref, "dbias at the limit")
    _same(got.col_data, ref.col_data, "col data at the limit")
