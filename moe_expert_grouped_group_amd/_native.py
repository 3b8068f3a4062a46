"""ctypes loader for libmxfp8moe.so (the HIP kernels behind the C ABI).

The library must have been built in-tree (``python -m
moe_expert_grouped_group_amd.build``).  There is no fallback: if it is
missing, or if it would bring a second HIP runtime into the process, loading
fails loudly.
"""

import ctypes
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxfp8moe.so")
_lib = None

c_u8p = ctypes.c_void_p
c_i64 = ctypes.c_int64
c_i32 = ctypes.c_int32
c_u32 = ctypes.c_uint32
c_size = ctypes.c_size_t
c_vp = ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/mxfp8moe.h
SIGNATURES = {
    "mxfp8_last_error": (ctypes.c_char_p, []),
    "mxfp8_abi_version": (c_i32, []),
    "mxfp8_dbias_workspace_bytes": (c_size, [c_i64, c_i64]),
    "mxfp8_group_quantize": (c_i32, [c_vp, c_i64, c_i64, c_u32, c_vp, c_vp, c_vp, c_vp, c_vp,
                                     c_vp]),
    "mxfp8_requant_colwise": (c_i32, [c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_i32, c_vp,
                                      c_vp, c_size, c_vp]),
    "mxfp8_grouped_dbias": (c_i32, [c_vp, c_vp, c_i64, c_i64, c_vp, c_i32, c_vp, c_vp, c_size,
                                    c_vp]),
    "mxfp8_group_quantize_requant": (c_i32, [c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp,
                                             c_i32, c_vp, c_vp, c_size, c_vp]),
    "mxfp8_group_quantize_requant_noalloc": (c_i32, [c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp,
                                                     c_vp, c_i32, c_vp, c_vp]),
    "mxfp8_grouped_gemm_swiglu_quantize": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64,
                                                   c_i64, c_vp, c_i32, c_u32, c_vp, c_vp, c_vp,
                                                   c_vp, c_vp]),
    "mxfp8_grouped_gemm": (c_i32, [c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i64, c_i64,
                                   c_i64, c_vp, c_i32, c_vp]),
    "mxfp8_validate_splits": (c_i32, [c_vp, c_i32, c_i64, c_vp, c_vp]),
    "mxfp8_grouped_gemm_wgrad_accumulate": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64,
                                                    c_i64, c_vp, c_i32, c_vp]),
    "mxfp8_grouped_gemm_workspace_bytes": (c_size, []),
    "mxfp8_grouped_gemm_ws": (c_i32, [c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i64, c_i64,
                                      c_i64, c_vp, c_i32, c_vp, c_size, c_vp]),
    "mxfp8_grouped_gemm_wgrad_accumulate_ws": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64,
                                                       c_i64, c_vp, c_i32, c_vp, c_size, c_vp]),
    "mxfp8_swiglu_fwd": (c_i32, [c_vp, c_i64, c_i64, c_vp, c_vp]),
    "mxfp8_swiglu_bwd": (c_i32, [c_vp, c_vp, c_i64, c_i64, c_vp, c_vp]),
    "mxfp8_swiglu_bwd_quantize": (c_i32, [c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp,
                                          c_i32, c_vp, c_vp, c_size, c_vp]),
    "mxfp8_swiglu_quantize": (c_i32, [c_vp, c_i64, c_i64, c_u32, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "mxfp8_scaled_bias_workspace_bytes": (c_size, [c_i64, c_i64]),
    "mxfp8_grouped_scaled_bias_grad": (c_i32, [c_vp, c_vp, c_i64, c_i64, c_vp, c_i32, c_vp, c_vp,
                                               c_vp, c_vp, c_vp, c_size, c_vp]),
    "mxfp8_convert_sweep_bytes": (c_size, [c_i32]),
    "mxfp8_convert_sweep": (c_i32, [c_i32, c_vp, c_size, c_vp]),
}

ABI_VERSION = 4

MXFP8_OK, MXFP8_EINVAL, MXFP8_ENOTSUP, MXFP8_EHIP = 0, 1, 2, 3


def lib_path():
    return _LIB_PATH


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as f:
            return sorted({l.split()[-1] for l in f if "libamdhip64" in l})
    except OSError:
        return []


def load():
    """Load the library once and declare every entry point's signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python -m moe_expert_grouped_group_amd.build`"
            " (there is no non-HIP fallback)")
    import torch  # noqa: F401  -- bring torch's HIP runtime in first so the library shares it
    lib = ctypes.CDLL(_LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError(f"two HIP runtimes are mapped in this process: {runtimes}")
    if lib.mxfp8_abi_version() != ABI_VERSION:
        raise ImportError("libmxfp8moe.so ABI version mismatch: rebuild it")
    _lib = lib
    return lib


def check(status, fn_name):
    """Raise the exception that the status code maps to."""
    if status == MXFP8_OK:
        return
    msg = _lib.mxfp8_last_error().decode(errors="replace") if _lib else ""
    msg = msg or f"{fn_name} failed with status {status}"
    if status == MXFP8_EINVAL:
        raise ValueError(msg)
    if status == MXFP8_ENOTSUP:
        raise NotImplementedError(msg)
    raise RuntimeError(msg)
