"""The fused MLP's FC1 with the SwiGLU + quantize epilogue
(mxfp8_grouped_gemm_swiglu_quantize) against the unfused chain it replaces:
the forward grouped GEMM with bf16 output h, then mxfp8_swiglu_quantize on
that h.  h and every code and scale byte must be identical, for each usage,
on routings with experts whose token count is an odd multiple of 128 (tiles
that hold 128 rows), experts without tokens, fewer tokens than one tile, and
at the full size of the Nemotron-proxy MLP.  One case is also checked
stage-wise against the oracle (its SwiGLU + quantize of the GPU's h), with the
SiLU allowance of the SwiGLU tests.  Through the C ABI."""

import numpy as np
import pytest
import torch

import moe_expert_grouped_group_amd as mx
from moe_expert_grouped_group_amd import workloads as wl
from oracle import mxfp8 as om
from oracle import swiglu as osw

from gpu_util import f64, log, u8

pytestmark = pytest.mark.gpu

R, C = mx.ROWWISE, mx.COLWISE


def _operands(splits, f, k, seed):
    t, g = sum(splits), len(splits)
    x = wl.bf16_normal([70, 1, seed], (t, k)).cuda()
    w1 = (wl.bf16_normal([70, 2, seed], (g * 2 * f, k)).float() * 0.05).to(torch.bfloat16).cuda()
    ms = torch.tensor(splits, dtype=torch.int64).cuda()
    xo = mx.group_quantize(x, R)
    wo = mx.group_quantize(w1, R)
    return xo, wo, ms


def _same(a, b, what):
    assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), what


def _compare(xo, wo, ms, t, f, k, usage, tag):
    log(f"swiglu GEMM {tag}: usage {usage}")
    h, out = mx.grouped_gemm_swiglu_quantize(xo.row_data, xo.row_scale, wo.row_data,
                                             wo.row_scale, ms, t, f, k, usage)
    h_ref = mx.grouped_gemm("NT", xo.row_data, xo.row_scale, wo.row_data, wo.row_scale, ms, t,
                            2 * f, k, torch.bfloat16)
    ref = mx.swiglu_quantize(h_ref, usage)
    torch.cuda.synchronize()
    _same(h, h_ref, f"{tag}: h")
    for part in ("row_data", "row_scale", "col_data", "col_scale"):
        if getattr(ref, part) is not None:
            _same(getattr(out, part), getattr(ref, part), f"{tag}: {part}")
    return h, out


CASES = [
    # (splits, F, K): 128-token experts (tiles of 128 rows, shifted back at
    # the end of the tokens), experts without tokens, several tiles
    ([128, 256, 0, 384], 512, 512),
    ([0, 640, 128, 0, 256, 128], 1024, 1024),
    # fewer tokens than one 256-row tile
    ([128], 512, 512),
    ([0, 128, 0], 1024, 1536),
]


@pytest.mark.parametrize("usage", [R | C, R, C])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_swiglu_gemm_matches_unfused(case, usage):
    splits, f, k = CASES[case]
    xo, wo, ms = _operands(splits, f, k, case)
    _compare(xo, wo, ms, sum(splits), f, k, usage, f"case {case}")


def test_swiglu_gemm_workload_and_oracle():
    """The small Nemotron-proxy MLP recipe (16 experts, Zipf routing, 4 of
    them without tokens): the same bytes as the unfused chain, and against
    the oracle's SwiGLU + quantize of the GPU's h (stage-wise)."""
    w = wl.make("small_nemotron_mlp")
    g, t, k, n2 = w.groups, w.tokens, w.hidden, w.ffn
    f = n2 // 2
    ms = torch.from_numpy(w.m_splits).cuda()
    xo = mx.group_quantize(w.tensors["x"].cuda(), R)
    wo = mx.group_quantize(w.tensors["w"].cuda(), R)
    h, out = _compare(xo, wo, ms, t, f, k, R | C, "small_nemotron_mlp")
    a_ref = om.round_to_bf16(osw.swiglu_fwd(f64(h)))
    qr, sr = om.quantize_rowwise(a_ref)
    qc, sc = om.quantize_colwise(a_ref, [int(v) for v in w.m_splits])
    for q_gpu, s_gpu, q_ref, s_ref in ((u8(out.row_data), u8(out.row_scale), qr, sr),
                                       (u8(out.col_data), u8(out.col_scale), qc, sc)):
        ds = s_gpu.astype(np.int32) - s_ref.astype(np.int32)
        assert np.abs(ds).max() <= 1
        assert np.count_nonzero(ds) <= max(2, s_ref.size // 1000)
        diff = (q_gpu != q_ref) & np.repeat(ds == 0, 32, axis=1)
        gi, ri = q_gpu[diff].astype(np.int32), q_ref[diff].astype(np.int32)
        assert ((((gi ^ ri) & 0x80) == 0) & (np.abs((gi & 0x7F) - (ri & 0x7F)) <= 1)).all()
        assert np.count_nonzero(diff) <= max(4, q_ref.size // 1000)


def test_swiglu_gemm_no_tokens():
    """T = 0: nothing to read or write, no error."""
    ms = torch.zeros(4, dtype=torch.int64, device="cuda")
    e = torch.empty(0, dtype=torch.uint8, device="cuda")
    h, out = mx.grouped_gemm_swiglu_quantize(e, e, torch.zeros(4 * 1024, 512, dtype=torch.uint8,
                                                               device="cuda"),
                                             torch.zeros(4 * 1024, 16, dtype=torch.uint8,
                                                         device="cuda"),
                                             ms, 0, 512, 512)
    torch.cuda.synchronize()
    assert h.shape == (0, 1024) and out.row_data.shape == (0, 512)


def test_swiglu_gemm_fullsize():
    """The Nemotron-proxy MLP's FC1 at full size (64 experts, 83968 tokens,
    3072 -> 2 x 1024): whole tensors equal to the unfused chain."""
    w = wl.make("nemotron_proxy_mlp")
    t, k, n2 = w.tokens, w.hidden, w.ffn
    ms = torch.from_numpy(w.m_splits).cuda()
    xo = mx.group_quantize(w.tensors["x"].cuda(), R)
    wo = mx.group_quantize(w.tensors["w"].cuda(), R)
    del w
    _compare(xo, wo, ms, t, n2 // 2, k, R | C, "nemotron_proxy_mlp full size")
