"""The C-ABI library loads, exports what the header declares, and rejects bad
arguments on the host before touching the GPU (no compute calls here)."""

import ctypes
import os
import re

import numpy as np
import pytest

import moe_expert_grouped_group_amd as mx
from moe_expert_grouped_group_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp8moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_native.lib_path()):
        from moe_expert_grouped_group_amd import build
        build.build()
    return _native.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxfp8_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    # and the binding declares a signature for each of them
    assert sorted(_native.SIGNATURES) == names


def test_only_one_hip_runtime(lib):
    assert len(_native._hip_runtimes_mapped()) <= 1


def test_abi_version_and_workspace(lib):
    assert lib.mxfp8_abi_version() == _native.ABI_VERSION
    assert lib.mxfp8_dbias_workspace_bytes(16384, 14336) == 128 * 14336 * 4
    assert lib.mxfp8_dbias_workspace_bytes(0, 512) == 0


def _status_msg(lib, st):
    return st, lib.mxfp8_last_error().decode()


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def test_quantize_rejects(lib):
    q = lib.mxfp8_group_quantize
    assert _status_msg(lib, q(None, 128, 512, 1, FAKE, FAKE, None, None, None, None))[0] == 1
    st, msg = _status_msg(lib, q(FAKE, 100, 512, 1, FAKE, FAKE, None, None, None, None))
    assert st == 1 and "128" in msg
    st, msg = _status_msg(lib, q(FAKE, 128, 96, 1, FAKE, FAKE, None, None, None, None))
    assert st == 1 and "512" in msg
    assert q(FAKE, 128, 512, 0, FAKE, FAKE, None, None, None, None) == 1          # no usage
    assert q(FAKE, 128, 512, 4, FAKE, FAKE, None, None, None, None) == 1          # unknown usage bit
    assert q(FAKE, 128, 512, 2, FAKE, FAKE, None, None, None, None) == 1          # col without buffers
    assert q(FAKE, 128, 512, 1, None, FAKE, None, None, None, None) == 1          # row without data


def test_gemm_rejects(lib):
    g = lib.mxfp8_grouped_gemm
    args = (FAKE, FAKE, FAKE, FAKE, FAKE)
    assert g(3, *args, 0, 128, 512, 512, FAKE, 1, None) == 1                 # bad layout
    st, msg = _status_msg(lib, g(0, *args, 7, 128, 512, 512, FAKE, 1, None))
    assert st == 2 and "dtype" in msg                                        # NotImplemented
    assert g(0, None, FAKE, FAKE, FAKE, FAKE, 0, 128, 512, 512, FAKE, 1, None) == 1
    assert g(0, *args, 0, 129, 512, 512, FAKE, 1, None) == 1                # T % 128
    assert g(0, *args, 0, 128, 500, 512, FAKE, 1, None) == 1                # N % 512
    assert g(0, *args, 0, 128, 512, 256, FAKE, 1, None) == 1                # K % 512
    assert g(0, *args, 0, 128, 512, 512, None, 1, None) == 1                # no splits
    assert g(0, *args, 0, 128, 512, 512, FAKE, 0, None) == 1                # G < 1


def test_gemm_rejects_host_splits(lib):
    splits = np.array([128], dtype=np.int64)
    st, msg = _status_msg(lib, lib.mxfp8_grouped_gemm(
        0, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 128, 512, 512,
        splits.ctypes.data_as(ctypes.c_void_p), 1, None))
    assert st == 1 and "m_splits" in msg


def test_requant_and_dbias_reject(lib):
    r = lib.mxfp8_requant_colwise
    assert r(None, FAKE, 128, 512, FAKE, FAKE, None, 0, None, None, 0, None) == 1
    assert r(FAKE, FAKE, 128, 100, FAKE, FAKE, None, 0, None, None, 0, None) == 1
    # dbias requested without splits / workspace
    assert r(FAKE, FAKE, 128, 512, FAKE, FAKE, None, 1, FAKE, FAKE, 1 << 20, None) == 1
    d = lib.mxfp8_grouped_dbias
    assert d(FAKE, FAKE, 128, 512, None, 1, FAKE, FAKE, 1 << 20, None) == 1
    assert d(FAKE, FAKE, 130, 512, FAKE, 1, FAKE, FAKE, 1 << 20, None) == 1


def test_swiglu_and_validate_reject(lib):
    assert lib.mxfp8_swiglu_fwd(None, 4, 8, FAKE, None) == 1
    assert lib.mxfp8_swiglu_fwd(FAKE, 4, 6, FAKE, None) == 1
    assert lib.mxfp8_swiglu_bwd(FAKE, None, 4, 8, FAKE, None) == 1
    assert lib.mxfp8_validate_splits(FAKE, 1, 128, None, None) == 1
    q = lib.mxfp8_swiglu_quantize
    assert q(None, 128, 512, 3, FAKE, FAKE, FAKE, FAKE, None) == 1        # no h
    assert q(FAKE, 100, 512, 3, FAKE, FAKE, FAKE, FAKE, None) == 1        # T % 128
    assert q(FAKE, 128, 500, 3, FAKE, FAKE, FAKE, FAKE, None) == 1        # F % 512
    assert q(FAKE, 128, 512, 0, FAKE, FAKE, FAKE, FAKE, None) == 1        # usage 0
    assert q(FAKE, 128, 512, 2, FAKE, FAKE, None, FAKE, None) == 1        # COLWISE, no q_col
    assert q(FAKE, 128, 512, 1, None, FAKE, None, None, None) == 1        # ROWWISE, no q_row
    assert q(FAKE, 0, 512, 3, FAKE, FAKE, FAKE, FAKE, None) == 0          # T == 0: nothing enqueued


def test_wgrad_accumulate_rejects(lib):
    f = lib.mxfp8_grouped_gemm_wgrad_accumulate
    assert f(FAKE, FAKE, FAKE, FAKE, None, 128, 512, 512, FAKE, 1, None) == 1      # no main_grad
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 100, 512, 512, FAKE, 1, None) == 1      # T % 128
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 128, 500, 512, FAKE, 1, None) == 1      # N % 512
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 128, 512, 512, FAKE, 2000, None) == 1   # G > 1024


def test_quantize_requant_rejects(lib):
    f = lib.mxfp8_group_quantize_requant
    args = (FAKE, FAKE, FAKE, FAKE)
    assert f(None, 128, 512, *args, None, 0, None, None, 0, None) == 1        # no x
    assert f(FAKE, 100, 512, *args, None, 0, None, None, 0, None) == 1        # T % 128
    assert f(FAKE, 128, 500, *args, None, 0, None, None, 0, None) == 1        # K % 512
    assert f(FAKE, 128, 512, FAKE, None, FAKE, FAKE, None, 0, None, None, 0, None) == 1
    # dbias without splits, or without a workspace
    assert f(FAKE, 128, 512, *args, None, 1, FAKE, FAKE, 1 << 20, None) == 1
    assert f(FAKE, 128, 512, *args, FAKE, 1, FAKE, None, 0, None) == 1
    assert f(None, 0, 512, None, None, None, None, None, 0, None, None, 0, None) == 0  # T == 0


def test_gemm_workspace_entries_reject(lib):
    """The workspace forms check the workspace first, then everything the
    plain forms check."""
    need = lib.mxfp8_grouped_gemm_workspace_bytes()
    assert need >= 4
    g = lib.mxfp8_grouped_gemm_ws
    args = (FAKE, FAKE, FAKE, FAKE, FAKE)
    st, msg = _status_msg(lib, g(2, *args, 0, 128, 512, 512, FAKE, 1, None, need, None))
    assert st == 1 and "workspace" in msg                                    # no workspace
    assert g(2, *args, 0, 128, 512, 512, FAKE, 1, FAKE, need - 1, None) == 1  # too small
    assert g(3, *args, 0, 128, 512, 512, FAKE, 1, FAKE, need, None) == 1     # bad layout
    assert g(2, *args, 0, 129, 512, 512, FAKE, 1, FAKE, need, None) == 1     # T % 128
    f = lib.mxfp8_grouped_gemm_wgrad_accumulate_ws
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 128, 512, 512, FAKE, 1, None, need, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, None, 128, 512, 512, FAKE, 1, FAKE, need, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 128, 512, 512, FAKE, 2000, FAKE, need, None) == 1


def test_scaled_bias_grad_rejects(lib):
    f = lib.mxfp8_grouped_scaled_bias_grad
    big = 1 << 30
    assert f(FAKE, FAKE, 128, 512, FAKE, 1, FAKE, FAKE, None, None, FAKE, big, None) == 1  # no output
    assert f(FAKE, FAKE, 128, 512, FAKE, 1, None, FAKE, FAKE, None, FAKE, big, None) == 1  # no scales
    assert f(FAKE, FAKE, 128, 512, FAKE, 1, FAKE, None, None, FAKE, FAKE, big, None) == 1  # no bias
    assert f(FAKE, FAKE, 100, 512, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == 1  # T % 128
    assert lib.mxfp8_scaled_bias_workspace_bytes(16384, 14336) == (
        512 + 128 * 14336 * 4 + 16384 * 28 * 4)


def test_convert_sweep_sizes_and_rejects(lib):
    assert lib.mxfp8_convert_sweep_bytes(0) == 2 << 24
    assert lib.mxfp8_convert_sweep_bytes(1) == 1 << 24
    assert lib.mxfp8_convert_sweep_bytes(2) == 8 << 16
    assert lib.mxfp8_convert_sweep_bytes(3) == 0
    assert lib.mxfp8_convert_sweep(3, FAKE, 1 << 30, None) == 1
    assert lib.mxfp8_convert_sweep(0, FAKE, (2 << 24) - 1, None) == 1
    assert lib.mxfp8_convert_sweep(2, None, 1 << 20, None) == 1


def test_binding_maps_errors(lib):
    with pytest.raises(ValueError):
        _native.check(1, "x")
    with pytest.raises(NotImplementedError):
        _native.check(2, "x")
    with pytest.raises(RuntimeError):
        _native.check(3, "x")
    assert mx.ROWWISE == 1 and mx.COLWISE == 2


def test_noalloc_quantize_requant_rejects(lib):
    """The allocation-free fused quantize refuses, on the host, dbias partials
    beyond its static scratch, and the usual shape errors."""
    f = lib.mxfp8_group_quantize_requant_noalloc
    assert mx.NOALLOC_SCRATCH_BYTES == 32 << 20
    k = 14336
    t_max = (mx.NOALLOC_SCRATCH_BYTES // (k * 4)) * 128     # 74880
    st, msg = _status_msg(lib, f(FAKE, t_max + 128, k, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE,
                                 None))
    assert st == 1 and "static scratch" in msg
    assert f(FAKE, 100, 512, FAKE, FAKE, FAKE, FAKE, None, 0, None, None) == 1    # T % 128
    assert f(FAKE, 128, 96, FAKE, FAKE, FAKE, FAKE, None, 0, None, None) == 1     # K % 512
    assert f(None, 128, 512, FAKE, FAKE, FAKE, FAKE, None, 0, None, None) == 1    # NULL x


def test_swiglu_gemm_rejects(lib):
    """FC1 with the SwiGLU + quantize epilogue: shape and usage errors on the
    host."""
    f = lib.mxfp8_grouped_gemm_swiglu_quantize
    ops = (FAKE, FAKE, FAKE, FAKE, FAKE)
    outs = (FAKE, FAKE, FAKE, FAKE)
    assert f(*ops, 128, 512, 512, FAKE, 1, 0, *outs, None) == 1            # no usage
    assert f(*ops, 128, 512, 512, FAKE, 1, 4, *outs, None) == 1            # unknown usage bit
    assert f(*ops, 100, 512, 512, FAKE, 1, 3, *outs, None) == 1            # T % 128
    assert f(*ops, 128, 256, 512, FAKE, 1, 3, *outs, None) == 1            # F % 512
    assert f(*ops, 128, 512, 500, FAKE, 1, 3, *outs, None) == 1            # K % 512
    assert f(*ops, 128, 512, 512, FAKE, 1025, 3, *outs, None) == 1         # G > 1024
    st, msg = _status_msg(lib, f(*ops, 128, 512, 512, FAKE, 1, 2, FAKE, FAKE, None, None, None))
    assert st == 1 and "COLWISE" in msg                                    # col without buffers
