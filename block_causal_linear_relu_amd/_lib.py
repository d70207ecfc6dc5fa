"""ctypes loader for libsvla.so: symbol table and prototypes (no torch needed).

The library is built in-tree by ``block_causal_linear_relu_amd.build``; this
module never builds it and never falls back to anything else: a missing
library is an error.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsvla.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "svla.h")

# enums of include/svla.h
SVLA_OK = 0
STATUS_NAMES = {0: "SVLA_OK", 1: "SVLA_ERR_NULL", 2: "SVLA_ERR_SHAPE", 3: "SVLA_ERR_DTYPE",
                4: "SVLA_ERR_ALIGN", 5: "SVLA_ERR_UNSUPPORTED", 6: "SVLA_ERR_WORKSPACE",
                7: "SVLA_ERR_VALUE", 8: "SVLA_ERR_HIP"}
SVLA_F32, SVLA_BF16, SVLA_FP8 = 0, 1, 2
(OP_NONCAUSAL, OP_BLOCK_CAUSAL, OP_BLOCK_STEP, OP_STATE_BUILD, OP_STATE_SCAN, OP_APPLY,
 OP_BACKWARD) = range(7)


class SvlaRope(ctypes.Structure):
    _fields_ = [("dt_dims", ctypes.c_int), ("dh_dims", ctypes.c_int),
                ("dw_dims", ctypes.c_int), ("grid_h", ctypes.c_int),
                ("grid_w", ctypes.c_int), ("t0", ctypes.c_int), ("base", ctypes.c_float)]


class SvlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), message))
        self.status = status


_i, _f, _vp, _sz = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
_rp = ctypes.POINTER(SvlaRope)

PROTOTYPES = {
    "svla_abi_version": (_i, []),
    "svla_status_string": (ctypes.c_char_p, [_i]),
    "svla_last_error": (ctypes.c_char_p, []),
    "svla_workspace_size": (_i, [_i, _i, _i, _i, _i, _i, _i, ctypes.POINTER(_sz)]),
    "svla_noncausal": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _f, _vp, _vp, _vp, _sz, _vp]),
    "svla_block_causal": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               _rp, _f, _vp, _sz, _vp]),
    "svla_block_causal_gated": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _vp, _rp, _f, _vp, _sz, _vp]),
    "svla_block_step": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _rp, _f,
                             _vp, _sz, _vp]),
    "svla_block_step_gated": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                   _vp, _rp, _f, _vp, _sz, _vp]),
    "svla_block_step_noalloc": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _rp, _f, _vp]),
    "svla_state_build": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _rp, _vp, _vp, _vp, _sz, _vp]),
    "svla_state_scan": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "svla_apply": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _rp, _f, _vp, _vp, _sz, _vp]),
    "svla_temporal_conv": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "svla_block_causal_backward": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _rp, _f, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "svla_set_timing_events": (_i, [ctypes.POINTER(_vp), _i]),
    "svla_hbm_probe": (_i, [_i, _vp, _vp, _sz, _vp, _i, _vp]),
    "svla_softmax_attention": (_i, [_i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _f, _vp]),
    "svla_describe": (_i, [_i, _i, _i, _i, _i, _i, _i, _rp, ctypes.c_char_p, _sz]),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsvla.so (built in-tree) and declare every prototype."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libsvla.so is not built (%s); run __graft_entry__.build() or "
                          "python -m block_causal_linear_relu_amd.build" % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in PROTOTYPES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.svla_abi_version() != 1:
        raise ImportError("libsvla ABI version %d, expected 1" % lib.svla_abi_version())
    if path == LIB_PATH:
        _lib = lib
    return lib


def check(lib, status: int) -> None:
    if status != SVLA_OK:
        raise SvlaError(status, lib.svla_last_error().decode())


def rope_struct(rope):
    """A svla_rope from any object with dt_dims, dh_dims, dw_dims, grid_h,
    grid_w, t0, base attributes (or a dict with those keys); None -> NULL."""
    if rope is None:
        return None
    get = (lambda k: rope[k]) if isinstance(rope, dict) else (lambda k: getattr(rope, k))
    return SvlaRope(int(get("dt_dims")), int(get("dh_dims")), int(get("dw_dims")),
                    int(get("grid_h")), int(get("grid_w")), int(get("t0")), float(get("base")))
