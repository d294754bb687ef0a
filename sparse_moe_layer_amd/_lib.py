"""ctypes binding of libmoe_mi355x.so (the C ABI in include/moe_mi355x.h).

Argument marshalling only: torch tensors are passed as device pointers
(data_ptr()) together with the current HIP stream; every step of the layer
runs in the library's kernels.  Importing this module fails loudly when the
library has not been built.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_MI355X_LIB names another build of the same library (A/B runs); default: the in-tree build
LIB_PATH = os.environ.get("MOE_MI355X_LIB") or os.path.join(_HERE, "libmoe_mi355x.so")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, \
    MOE_ERR_UNSUPPORTED, MOE_ERR_HIP = range(8)
MOE_F32, MOE_BF16, MOE_FP8_E4M3FN = 0, 1, 2
MOE_FLAG_FORCE_GEMM = 1
MOE_FLAG_FORCE_STREAM = 2
MOE_FLAG_GEMM_TILE_128 = 4
MOE_FLAG_GEMM_TILE_256 = 8
MOE_FLAG_PAGE_ROUTING = 16
MOE_NOALLOC_SCRATCH_BYTES = 32 << 20

EXPORTS = ["moe_abi_version", "moe_status_str", "moe_validate", "moe_workspace_bytes", "moe_route",
           "moe_dispatch", "moe_expert_ffn", "moe_expert_gate_up", "moe_expert_down", "moe_combine",
           "moe_layer_forward", "moe_gr_workspace_bytes", "moe_gr_read", "moe_gr_write", "moe_combine_gr_write",
           "moe_audit_workspace_bytes", "moe_weight_audit", "moe_layer_forward_noalloc",
           "moe_hbm_read_probe", "moe_mfma_pipe_probe"]


class moe_problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64), ("E", ctypes.c_int64), ("k", ctypes.c_int64),
                ("I", ctypes.c_int64), ("I_shared", ctypes.c_int64), ("act_dtype", ctypes.c_int32),
                ("w_dtype", ctypes.c_int32), ("scale_block", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class moe_weights(ctypes.Structure):
    _fields_ = [("w_router", ctypes.c_void_p), ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("stride_gate", ctypes.c_int64), ("stride_up", ctypes.c_int64),
                ("stride_down", ctypes.c_int64), ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p),
                ("s_down", ctypes.c_void_p), ("sh_gate", ctypes.c_void_p), ("sh_up", ctypes.c_void_p),
                ("sh_down", ctypes.c_void_p), ("sh_gate_w", ctypes.c_void_p)]


class moe_gr_weights(ctypes.Structure):
    _fields_ = [("norm_w", ctypes.c_void_p), ("w_read", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
                ("rank", ctypes.c_int64), ("eps", ctypes.c_float)]


class moe_audit_stats(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("n_zero", ctypes.c_int64), ("n_nan", ctypes.c_int64),
                ("median", ctypes.c_double), ("mad", ctypes.c_double), ("sigma_rob", ctypes.c_double)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python sparse_moe_layer_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(moe_problem)
    W = ctypes.POINTER(moe_weights)
    G = ctypes.POINTER(moe_gr_weights)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    sig = {
        "moe_abi_version": (i32, []),
        "moe_status_str": (ctypes.c_char_p, [i32]),
        "moe_validate": (i32, [P]),
        "moe_workspace_bytes": (sz, [P]),
        "moe_route": (i32, [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moe_dispatch": (i32, [P, vp, vp, vp, vp, vp, sz, vp]),
        "moe_expert_ffn": (i32, [P, W, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moe_expert_gate_up": (i32, [P, W, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moe_expert_down": (i32, [P, W, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moe_combine": (i32, [P, vp, vp, vp, vp, vp, vp, vp]),
        "moe_layer_forward": (i32, [P, W, vp, vp, vp, vp, vp, sz, vp]),
        "moe_layer_forward_noalloc": (i32, [P, W, vp, vp, vp, vp, vp]),
        "moe_hbm_read_probe": (i32, [vp, sz, vp, vp]),
        "moe_mfma_pipe_probe": (i32, [ctypes.c_int32, ctypes.c_int32, vp, sz, vp, vp]),
        "moe_gr_workspace_bytes": (sz, [P, ctypes.c_int64]),
        "moe_gr_read": (i32, [P, G, vp, vp, vp, vp, sz, vp]),
        "moe_gr_write": (i32, [P, vp, vp, vp, vp, vp]),
        "moe_combine_gr_write": (i32, [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "moe_audit_workspace_bytes": (sz, [ctypes.c_int64]),
        "moe_weight_audit": (i32, [vp, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, vp, vp, sz,
                                   vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()
