"""CPU oracle for block-causal ReLU linear attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never imports it and
shares no code with it.

Two independent CPU implementations live here:

* ``forward`` -- the fp64 C oracle (``svla_oracle.c``), which follows the
  method's recurrence block by block: carry the d x d state S and the
  normaliser z, add each block's contribution, read the block's queries
  against the inclusive state.
* ``brute.brute_force`` -- the quadratic form in numpy fp64: every query
  against every key of its own and earlier blocks, no state at all.

Pins of the oracle (closed forms, special cases, invariants, an exact
rational example) are in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time
from typing import Optional

import numpy as np

from .brute import brute_force, rope_apply  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "svla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libsvla_oracle.so")
_lib = None


class _Rope(ctypes.Structure):
    _fields_ = [("dt_dims", ctypes.c_int), ("dh_dims", ctypes.c_int),
                ("dw_dims", ctypes.c_int), ("grid_h", ctypes.c_int),
                ("grid_w", ctypes.c_int), ("t0", ctypes.c_int),
                ("base", ctypes.c_double)]


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-std=c99", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.svlao_forward.restype = ctypes.c_int
        lib.svlao_forward.argtypes = [ctypes.c_int] * 5 + [dp, dp, dp, dp,
                                      ctypes.POINTER(_Rope), dp, dp,
                                      ctypes.c_double, dp, dp, dp, dp, dp,
                                      dp, dp, dp, ctypes.c_int]
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a, shape=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.float64)
    if shape is not None:
        a = a.reshape(shape)
    return a


def forward(Q, K, V, nb: int, *, g=None, rope=None, S0=None, z0=None,
            eps: float = 1e-6, want_blocks: bool = False,
            want_local: bool = False, want_den: bool = False,
            threads: int = 0) -> dict:
    """Run the fp64 oracle.  Q, K, V: [B,H,N,d] (any float dtype, upcast exactly).

    ``g``: [B,H,nb] decay per block or None.  ``rope``: an object with
    dt_dims, dh_dims, dw_dims, grid_h, grid_w, t0, base, or None.
    ``S0``/``z0``: [B,H,d,d] / [B,H,d] carried state or None (zero).
    Returns a dict with O, S, z (final state) and, on request, the inclusive
    per-block states (S_blocks, z_blocks), each block's own contribution
    (S_local, z_local), the denominators (den) and the threads used.
    """
    lib = _load()
    Q = _f64(Q); K = _f64(K); V = _f64(V)
    B, H, N, d = Q.shape
    if K.shape != Q.shape or V.shape != Q.shape:
        raise ValueError("Q, K, V shapes differ")
    if nb <= 0 or N % nb:
        if not (nb == 0 and N == 0):
            raise ValueError("N must be a multiple of nb")
    n = N // nb if nb else 0
    g = _f64(g, (B, H, nb)) if g is not None else None
    S0 = _f64(S0, (B, H, d, d)) if S0 is not None else None
    z0 = _f64(z0, (B, H, d)) if z0 is not None else None
    O = np.zeros((B, H, N, d))
    S = np.zeros((B, H, d, d))
    z = np.zeros((B, H, d))
    Sb = np.zeros((B, H, nb, d, d)) if want_blocks else None
    zb = np.zeros((B, H, nb, d)) if want_blocks else None
    Sl = np.zeros((B, H, nb, d, d)) if want_local else None
    zl = np.zeros((B, H, nb, d)) if want_local else None
    den = np.zeros((B, H, N)) if want_den else None
    r = None
    if rope is not None:
        r = _Rope(int(rope.dt_dims), int(rope.dh_dims), int(rope.dw_dims),
                  int(rope.grid_h), int(rope.grid_w), int(rope.t0),
                  float(rope.base))
    t = time.perf_counter()
    used = lib.svlao_forward(B, H, nb, n, d, _ptr(Q), _ptr(K), _ptr(V),
                             _ptr(g), ctypes.byref(r) if r is not None else None,
                             _ptr(S0), _ptr(z0), float(eps), _ptr(O), _ptr(S),
                             _ptr(z), _ptr(Sb), _ptr(zb), _ptr(Sl), _ptr(zl),
                             _ptr(den), int(threads))
    elapsed = time.perf_counter() - t
    if used < 0:
        raise ValueError("oracle rejected its arguments")
    out = {"O": O, "S": S, "z": z, "threads": used, "seconds": elapsed}
    if want_blocks:
        out["S_blocks"], out["z_blocks"] = Sb, zb
    if want_local:
        out["S_local"], out["z_local"] = Sl, zl
    if want_den:
        out["den"] = den
    return out


def step(Q, K, V, S_in, z_in, *, g=None, rope=None, eps: float = 1e-6) -> dict:
    """One streaming block step: a one-block forward that starts from (S_in, z_in).

    ``g``: [B,H] decay of the carried state for this step, or None.
    """
    Q = np.asarray(Q)
    B, H = Q.shape[:2]
    gg = None if g is None else np.asarray(g, dtype=np.float64).reshape(B, H, 1)
    return forward(Q, K, V, 1, g=gg, rope=rope, S0=S_in, z0=z_in, eps=eps)


def normwise_error(x, ref) -> float:
    """Normwise relative error: max over (b,h) slices of max|x-ref| / max|ref|.

    Arrays are [B,H,...]; every trailing axis belongs to one slice.
    """
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        raise ValueError("shape mismatch %s vs %s" % (x.shape, ref.shape))
    if x.size == 0:
        return 0.0
    B, H = ref.shape[:2]
    xs = x.reshape(B * H, -1)
    rs = ref.reshape(B * H, -1)
    if not np.all(np.isfinite(xs)):
        return float("inf")
    err = np.abs(xs - rs).max(axis=1)
    scale = np.abs(rs).max(axis=1)
    rel = np.where(scale > 0, err / np.where(scale > 0, scale, 1.0), err)
    return float(rel.max())
