"""ctypes loader for ``libmhc.so`` (the gfx950 C-ABI library).

The library is built in-tree by ``birkhoff_projection_amd.build``.  There is
no fallback: if it is missing or fails to load, every op raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmhc.so")

c_void_p = ctypes.c_void_p
c_int64 = ctypes.c_int64
c_int32 = ctypes.c_int32


class ProjOpts(ctypes.Structure):
    """Mirror of ``mhc_proj_opts``."""
    _fields_ = [("solver", ctypes.c_int32), ("max_iters", ctypes.c_int32),
                ("tol", ctypes.c_float), ("warm_sweeps", ctypes.c_int32)]


class LayerArgs(ctypes.Structure):
    """Mirror of ``mhc_layer_args``."""
    _fields_ = [("T", ctypes.c_int64), ("n", ctypes.c_int32), ("C", ctypes.c_int64),
                ("eps", ctypes.c_float), ("proj", ctypes.POINTER(ProjOpts)),
                ("x", c_void_p), ("W", c_void_p), ("f", c_void_p),
                ("u", c_void_p), ("x_out", c_void_p), ("rms", c_void_p), ("logits", c_void_p),
                ("H_pre", c_void_p), ("H_post", c_void_p), ("H_res", c_void_p),
                ("grad_x_out", c_void_p), ("grad_u", c_void_p),
                ("grad_x", c_void_p), ("grad_f", c_void_p), ("grad_W", c_void_p),
                ("grad_logits", c_void_p), ("workspace", c_void_p),
                ("workspace_bytes", ctypes.c_int64)]


# name -> (restype, argtypes), exactly as declared in include/mhc.h
SIGNATURES = {
    "mhc_proj_opts_default": (c_int32, [ctypes.POINTER(ProjOpts)]),
    "mhc_birkhoff_fwd": (c_int32, [c_void_p, c_void_p, c_int64, ctypes.POINTER(ProjOpts),
                                   c_void_p, c_void_p]),
    "mhc_birkhoff_bwd": (c_int32, [c_void_p, c_void_p, c_void_p, c_int64, c_void_p]),
    "mhc_birkhoff_bwd_recompute": (c_int32, [c_void_p, c_void_p, c_void_p, c_int64,
                                             ctypes.POINTER(ProjOpts), c_void_p]),
    "mhc_birkhoff_fwd_bwd": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_int64,
                                       ctypes.POINTER(ProjOpts), c_void_p, c_void_p]),
    "mhc_birkhoff_pipeline_step": (c_int32, [c_void_p, c_void_p, c_int64, ctypes.POINTER(ProjOpts),
                                             c_void_p, c_void_p, c_void_p, c_void_p, c_int64,
                                             c_void_p]),
    "mhc_birkhoff_fwd_n": (c_int32, [c_void_p, c_void_p, c_int64, c_int32,
                                     ctypes.POINTER(ProjOpts), c_void_p, c_void_p]),
    "mhc_birkhoff_bwd_n": (c_int32, [c_void_p, c_void_p, c_void_p, c_int64, c_int32, c_void_p]),
    "mhc_stream_mix": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int32,
                                 c_int64, ctypes.POINTER(ProjOpts), c_void_p]),
    "mhc_stream_mix_bwd": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64,
                                     c_int32, c_int64, c_void_p]),
    "mhc_layer_workspace_bytes": (c_int64, [c_int64, c_int32, c_int64]),
    "mhc_layer_fwd": (c_int32, [ctypes.POINTER(LayerArgs), c_void_p]),
    "mhc_layer_bwd": (c_int32, [ctypes.POINTER(LayerArgs), c_void_p]),
    "mhc_layer_bwd_noalloc": (c_int32, [ctypes.POINTER(LayerArgs), c_void_p]),
    "mhc_status_string": (ctypes.c_char_p, [c_int32]),
    "mhc_last_error": (ctypes.c_char_p, []),
    "mhc_abi_version": (c_int32, []),
}

STATUS = {0: "MHC_OK", 1: "MHC_ERR_INVALID_ARGUMENT", 2: "MHC_ERR_UNSUPPORTED",
          3: "MHC_ERR_LAUNCH"}

_lib = None


class MHCError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def lib():
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m birkhoff_projection_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != 0:
        msg = lib().mhc_last_error().decode(errors="replace")
        raise MHCError(status, msg)
