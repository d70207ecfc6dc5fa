"""block_causal_linear_relu_amd -- block-causal ReLU linear attention on MI355X.

Python binding of libsvla (``include/svla.h``).  Argument marshalling only:
every step of the computation runs in the library's HIP kernels.  PyTorch
provides device memory (outputs, workspace) and the current stream.

    O = noncausal(Q, K, V)                             # one block, bidirectional
    O, S, z = block_causal(Q, K, V, nb, return_state=True)
    O, S, z = block_causal(Q, K, V, nb, g=g)           # gated (SANA-Video 2.0)
    O, S, z = block_step(Q, K, V, S, z, rope=rope)     # streaming, state carried

Tensors are [B,H,N,d] contiguous CUDA (HIP) tensors of torch.bfloat16 or
torch.float32; states S [B,H,d,d] (S[k][v]) and z [B,H,d] are float32.
A ``rope`` is any object (or dict) with dt_dims, dh_dims, dw_dims, grid_h,
grid_w, t0, base.  Errors of the library raise ``SvlaError``.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import SvlaError, rope_struct  # noqa: F401

__all__ = ["noncausal", "block_causal", "block_step", "state_build", "state_scan", "apply",
           "workspace_size", "describe", "set_timing_events", "SvlaError", "library"]

_DT = {torch.bfloat16: _lib.SVLA_BF16, torch.float32: _lib.SVLA_F32}
_OPS = {"noncausal": _lib.OP_NONCAUSAL, "block_causal": _lib.OP_BLOCK_CAUSAL,
        "block_step": _lib.OP_BLOCK_STEP, "state_build": _lib.OP_STATE_BUILD,
        "state_scan": _lib.OP_STATE_SCAN, "apply": _lib.OP_APPLY}


def library() -> ctypes.CDLL:
    """The loaded libsvla.so (raises ImportError if it is not built)."""
    return _lib.load()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (got %s)" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    return t


def _opt(t, name, dtype=torch.float32):
    return None if t is None else _dev(t, name, dtype)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise ValueError("dtype %s not supported (bfloat16 or float32)" % t.dtype)
    return _DT[t.dtype]


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def workspace_size(op: str, dtype: torch.dtype, B: int, H: int, nb: int, n: int, d: int) -> int:
    lib = library()
    out = ctypes.c_size_t(0)
    _lib.check(lib, lib.svla_workspace_size(_OPS[op], _DT[dtype], B, H, nb, n, d,
                                            ctypes.byref(out)))
    return int(out.value)


def describe(op: str, dtype: torch.dtype, B: int, H: int, nb: int, n: int, d: int, rope=None) -> dict:
    """The launch plan of a fused call (kernel names, grids, splits, workspace)."""
    import json
    lib = library()
    buf = ctypes.create_string_buffer(4096)
    rs = rope_struct(rope)
    _lib.check(lib, lib.svla_describe(_OPS[op], _DT[dtype], B, H, nb, n, d,
                                      ctypes.byref(rs) if rs is not None else None, buf, 4096))
    return json.loads(buf.value.decode())


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _rope_arg(rope):
    s = rope_struct(rope)
    return (ctypes.byref(s), s) if s is not None else (None, None)


def _qkv(Q, K, V):
    _dev(Q, "Q")
    dt = _dtype(Q)
    _dev(K, "K", Q.dtype)
    _dev(V, "V", Q.dtype)
    if Q.dim() != 4 or K.shape != Q.shape or V.shape != Q.shape:
        raise ValueError("Q, K, V must share one [B,H,N,d] shape")
    return dt


def _ws_arg(workspace, op, Q, B, H, nb, n, d):
    if workspace is None:
        workspace = _workspace(workspace_size(op, Q.dtype, B, H, nb, n, d), Q.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return workspace, nbytes


def set_timing_events(events) -> None:
    """Record ``events`` (torch.cuda.Event, each recorded once already) between
    the kernels of every following fused call on this thread; None stops."""
    lib = library()
    if not events:
        _lib.check(lib, lib.svla_set_timing_events(None, 0))
        set_timing_events._keep = None
        return
    arr = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    set_timing_events._keep = arr
    _lib.check(lib, lib.svla_set_timing_events(arr, len(events)))


def noncausal(Q, K, V, eps: float = 1e-6, return_state: bool = False,
              out: Optional[torch.Tensor] = None, workspace=None):
    """Bidirectional linear attention over all N tokens (one block)."""
    dt = _qkv(Q, K, V)
    B, H, N, d = Q.shape
    lib = library()
    O = torch.empty_like(Q) if out is None else _dev(out, "out", Q.dtype)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=Q.device) if return_state else None
    z = torch.empty((B, H, d), dtype=torch.float32, device=Q.device) if return_state else None
    ws, nbytes = _ws_arg(workspace, "noncausal", Q, B, H, 1, N, d)
    _lib.check(lib, lib.svla_noncausal(dt, B, H, N, d, _ptr(Q), _ptr(K), _ptr(V), _ptr(O),
                                       float(eps), _ptr(S), _ptr(z), _ptr(ws), nbytes,
                                       _stream(Q.device)))
    return (O, S, z) if return_state else O


def block_causal(Q, K, V, nb: int, S0=None, z0=None, g=None, rope=None, eps: float = 1e-6,
                 return_state: bool = False, out: Optional[torch.Tensor] = None,
                 workspace=None):
    """Block-causal linear attention over nb blocks of N/nb tokens in one call.

    ``g`` [B,H,nb] float32 selects the gated variant."""
    dt = _qkv(Q, K, V)
    B, H, N, d = Q.shape
    if nb <= 0 or N % nb:
        raise ValueError("N=%d is not a multiple of nb=%d" % (N, nb))
    n = N // nb
    S0, z0, g = _opt(S0, "S0"), _opt(z0, "z0"), _opt(g, "g")
    lib = library()
    O = torch.empty_like(Q) if out is None else _dev(out, "out", Q.dtype)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=Q.device) if return_state else None
    z = torch.empty((B, H, d), dtype=torch.float32, device=Q.device) if return_state else None
    ws, nbytes = _ws_arg(workspace, "block_causal", Q, B, H, nb, n, d)
    rp, _keep = _rope_arg(rope)
    if g is None:
        st = lib.svla_block_causal(dt, B, H, nb, n, d, _ptr(Q), _ptr(K), _ptr(V), _ptr(O),
                                   _ptr(S0), _ptr(z0), _ptr(S), _ptr(z), rp, float(eps),
                                   _ptr(ws), nbytes, _stream(Q.device))
    else:
        st = lib.svla_block_causal_gated(dt, B, H, nb, n, d, _ptr(Q), _ptr(K), _ptr(V), _ptr(O),
                                         _ptr(S0), _ptr(z0), _ptr(S), _ptr(z), _ptr(g), rp,
                                         float(eps), _ptr(ws), nbytes, _stream(Q.device))
    _lib.check(lib, st)
    return (O, S, z) if return_state else O


def block_step(Q, K, V, S_in=None, z_in=None, S_out=None, z_out=None, g=None, rope=None,
               eps: float = 1e-6, out: Optional[torch.Tensor] = None, workspace=None):
    """One streaming block: S_out = g*S_in + phi(K)^T V (g = 1 ungated), O reads S_out.

    ``S_out``/``z_out`` default to new tensors; pass S_out=S_in, z_out=z_in to
    commit in place.  Returns (O, S_out, z_out)."""
    dt = _qkv(Q, K, V)
    B, H, n, d = Q.shape
    S_in, z_in, g = _opt(S_in, "S_in"), _opt(z_in, "z_in"), _opt(g, "g")
    lib = library()
    O = torch.empty_like(Q) if out is None else _dev(out, "out", Q.dtype)
    if S_out is None:
        S_out = torch.empty((B, H, d, d), dtype=torch.float32, device=Q.device)
    if z_out is None:
        z_out = torch.empty((B, H, d), dtype=torch.float32, device=Q.device)
    _dev(S_out, "S_out", torch.float32)
    _dev(z_out, "z_out", torch.float32)
    ws, nbytes = _ws_arg(workspace, "block_step", Q, B, H, 1, n, d)
    rp, _keep = _rope_arg(rope)
    if g is None:
        st = lib.svla_block_step(dt, B, H, n, d, _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(S_in),
                                 _ptr(z_in), _ptr(S_out), _ptr(z_out), rp, float(eps), _ptr(ws),
                                 nbytes, _stream(Q.device))
    else:
        st = lib.svla_block_step_gated(dt, B, H, n, d, _ptr(Q), _ptr(K), _ptr(V), _ptr(O),
                                       _ptr(S_in), _ptr(z_in), _ptr(S_out), _ptr(z_out), _ptr(g),
                                       rp, float(eps), _ptr(ws), nbytes, _stream(Q.device))
    _lib.check(lib, st)
    return O, S_out, z_out


def state_build(K, V, nb: int, rope=None):
    """Each block's own contribution: S_local [B,H,nb,d,d], z_local [B,H,nb,d]."""
    _dev(K, "K")
    dt = _dtype(K)
    _dev(V, "V", K.dtype)
    B, H, N, d = K.shape
    if nb <= 0 or N % nb:
        raise ValueError("N=%d is not a multiple of nb=%d" % (N, nb))
    lib = library()
    S = torch.empty((B, H, nb, d, d), dtype=torch.float32, device=K.device)
    z = torch.empty((B, H, nb, d), dtype=torch.float32, device=K.device)
    rp, _keep = _rope_arg(rope)
    _lib.check(lib, lib.svla_state_build(dt, B, H, nb, N // nb, d, _ptr(K), _ptr(V), rp,
                                         _ptr(S), _ptr(z), None, 0, _stream(K.device)))
    return S, z


def state_scan(S_local, z_local, g=None, S0=None, z0=None):
    """Inclusive (decayed) prefix over blocks of the local states."""
    _dev(S_local, "S_local", torch.float32)
    _dev(z_local, "z_local", torch.float32)
    B, H, nb, d, _ = S_local.shape
    g, S0, z0 = _opt(g, "g"), _opt(S0, "S0"), _opt(z0, "z0")
    lib = library()
    Sp = torch.empty_like(S_local)
    zp = torch.empty_like(z_local)
    _lib.check(lib, lib.svla_state_scan(B, H, nb, d, _ptr(S_local), _ptr(z_local), _ptr(g),
                                        _ptr(S0), _ptr(z0), _ptr(Sp), _ptr(zp),
                                        _stream(S_local.device)))
    return Sp, zp


def apply(Q, S_prefix, z_prefix, nb: int, rope=None, eps: float = 1e-6):
    """O of every token against its block's (given) inclusive state."""
    _dev(Q, "Q")
    dt = _dtype(Q)
    _dev(S_prefix, "S_prefix", torch.float32)
    _dev(z_prefix, "z_prefix", torch.float32)
    B, H, N, d = Q.shape
    if nb <= 0 or N % nb:
        raise ValueError("N=%d is not a multiple of nb=%d" % (N, nb))
    n = N // nb
    lib = library()
    O = torch.empty_like(Q)
    ws = _workspace(workspace_size("apply", Q.dtype, B, H, nb, n, d), Q.device)
    nbytes = 0 if ws is None else ws.numel()
    rp, _keep = _rope_arg(rope)
    _lib.check(lib, lib.svla_apply(dt, B, H, nb, n, d, _ptr(Q), _ptr(S_prefix), _ptr(z_prefix),
                                   rp, float(eps), _ptr(O), _ptr(ws), nbytes,
                                   _stream(Q.device)))
    return O
