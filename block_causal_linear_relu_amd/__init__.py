"""block_causal_linear_relu_amd -- block-causal ReLU linear attention on MI355X.

Python binding of libsvla (``include/svla.h``).  Argument marshalling only:
every step of the computation runs in the library's HIP kernels.  PyTorch
provides device memory (outputs, workspace) and the current stream.

    O = noncausal(Q, K, V)                             # one block, bidirectional
    O, S, z = block_causal(Q, K, V, nb, return_state=True)
    O, S, z = block_causal(Q, K, V, nb, g=g)           # gated (SANA-Video 2.0)
    O, S, z = block_step(Q, K, V, S, z, rope=rope)     # streaming, state carried
    grads = block_causal_backward(Q, K, V, dO, nb)     # dQ, dK, dV (+ dg, dS0, dz0)

Tensors are [B,H,N,d] contiguous CUDA (HIP) tensors of torch.bfloat16,
torch.float32 or torch.float8_e4m3fn (d = 32; O is then bfloat16); states
S [B,H,d,d] (S[k][v]) and z [B,H,d] are float32.
A ``rope`` is any object (or dict) with dt_dims, dh_dims, dw_dims, grid_h,
grid_w, t0, base.  Errors of the library raise ``SvlaError``.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import SvlaError, rope_struct  # noqa: F401

__all__ = ["noncausal", "block_causal", "block_step", "block_step_noalloc", "state_build",
           "state_scan", "apply", "temporal_conv", "block_causal_backward", "softmax_attention",
           "workspace_size", "describe", "set_timing_events", "SvlaError", "library"]

_DT = {torch.bfloat16: _lib.SVLA_BF16, torch.float32: _lib.SVLA_F32,
       torch.float8_e4m3fn: _lib.SVLA_FP8}
_OPS = {"noncausal": _lib.OP_NONCAUSAL, "block_causal": _lib.OP_BLOCK_CAUSAL,
        "block_step": _lib.OP_BLOCK_STEP, "state_build": _lib.OP_STATE_BUILD,
        "state_scan": _lib.OP_STATE_SCAN, "apply": _lib.OP_APPLY,
        "backward": _lib.OP_BACKWARD}


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
        raise ValueError("dtype %s not supported (bfloat16, float32 or float8_e4m3fn)" % t.dtype)
    return _DT[t.dtype]


def _odtype(dtype):
    """The dtype of O for inputs of `dtype` (fp8 inputs give a bf16 output)."""
    return torch.bfloat16 if dtype == torch.float8_e4m3fn else dtype


def _out(out, Q):
    if out is None:
        return torch.empty(Q.shape, dtype=_odtype(Q.dtype), device=Q.device)
    return _dev(out, "out", _odtype(Q.dtype))


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


def _shape(t, shape, name):
    """Raise ValueError unless ``t`` (None allowed) has exactly ``shape``.

    The library reads and writes every tensor through a raw pointer with no
    range check of its own, so the shapes are checked here, before anything
    else (device, dtype) and before any call into the library."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, list(shape), list(t.shape)))


def _qkv_shape(Q, K, V):
    """(B, H, N, d) of Q, K, V, which must share one 4-d shape."""
    for t, name in ((Q, "Q"), (K, "K"), (V, "V")):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % name)
    if Q.dim() != 4 or K.shape != Q.shape or V.shape != Q.shape:
        raise ValueError("Q, K, V must share one [B,H,N,d] shape")
    return tuple(Q.shape)


def _pair(a, b, na, nb_):
    if (a is None) != (b is None):
        raise ValueError("pass both %s and %s, or neither" % (na, nb_))


def _qkv(Q, K, V):
    _qkv_shape(Q, K, V)
    _dev(Q, "Q")
    dt = _dtype(Q)
    _dev(K, "K", Q.dtype)
    _dev(V, "V", Q.dtype)
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
    B, H, N, d = _qkv_shape(Q, K, V)
    _shape(out, Q.shape, "out")
    dt = _qkv(Q, K, V)
    lib = library()
    O = _out(out, Q)
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
    B, H, N, d = _qkv_shape(Q, K, V)
    if nb <= 0 or N % nb:
        raise ValueError("N=%d is not a multiple of nb=%d" % (N, nb))
    n = N // nb
    _shape(S0, (B, H, d, d), "S0")
    _shape(z0, (B, H, d), "z0")
    _shape(g, (B, H, nb), "g")
    _shape(out, Q.shape, "out")
    _pair(S0, z0, "S0", "z0")
    dt = _qkv(Q, K, V)
    S0, z0, g = _opt(S0, "S0"), _opt(z0, "z0"), _opt(g, "g")
    lib = library()
    O = _out(out, Q)
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
    B, H, n, d = _qkv_shape(Q, K, V)
    _shape(S_in, (B, H, d, d), "S_in")
    _shape(z_in, (B, H, d), "z_in")
    _shape(S_out, (B, H, d, d), "S_out")
    _shape(z_out, (B, H, d), "z_out")
    _shape(g, (B, H), "g")
    _shape(out, Q.shape, "out")
    _pair(S_in, z_in, "S_in", "z_in")
    dt = _qkv(Q, K, V)
    S_in, z_in, g = _opt(S_in, "S_in"), _opt(z_in, "z_in"), _opt(g, "g")
    lib = library()
    O = _out(out, Q)
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


def block_step_noalloc(Q, K, V, S_in, z_in, S_out, z_out, out, g=None, rope=None,
                       eps: float = 1e-6):
    """svla_block_step with the library's own scratch: every output (``out``,
    ``S_out``, ``z_out``) is passed in and nothing is allocated, here or in
    the library.  Returns (out, S_out, z_out)."""
    B, H, n, d = _qkv_shape(Q, K, V)
    _shape(S_in, (B, H, d, d), "S_in")
    _shape(z_in, (B, H, d), "z_in")
    _shape(S_out, (B, H, d, d), "S_out")
    _shape(z_out, (B, H, d), "z_out")
    _shape(g, (B, H), "g")
    _shape(out, Q.shape, "out")
    _pair(S_in, z_in, "S_in", "z_in")
    if out is None or S_out is None or z_out is None:
        raise ValueError("out, S_out and z_out are required (nothing is allocated)")
    dt = _qkv(Q, K, V)
    S_in, z_in, g = _opt(S_in, "S_in"), _opt(z_in, "z_in"), _opt(g, "g")
    _dev(out, "out", _odtype(Q.dtype))
    _dev(S_out, "S_out", torch.float32)
    _dev(z_out, "z_out", torch.float32)
    lib = library()
    rp, _keep = _rope_arg(rope)
    _lib.check(lib, lib.svla_block_step_noalloc(dt, B, H, n, d, _ptr(Q), _ptr(K), _ptr(V), _ptr(out),
                                                _ptr(S_in), _ptr(z_in), _ptr(S_out), _ptr(z_out),
                                                _ptr(g), rp, float(eps), _stream(Q.device)))
    return out, S_out, z_out


def temporal_conv(X, w, F: int, bias=None, cache_in=None, cache_out=None, out=None):
    """The FFN's temporal convolution, causal across blocks of F frames.

    X [B,T,P,C] (bf16 or fp32, C % 8 == 0), w [C,3] and bias [C] float32,
    cache_in / cache_out [B,P,C] in X's dtype (cache_out receives X's last
    frame; it may be cache_in itself).  Returns Y (and cache_out if given)."""
    if not isinstance(X, torch.Tensor) or X.dim() != 4:
        raise ValueError("X must be a [B,T,P,C] tensor")
    B, T, P, C = X.shape
    if F <= 0 or T % F:
        raise ValueError("T=%d is not a multiple of F=%d" % (T, F))
    _shape(w, (C, 3), "w")
    _shape(bias, (C,), "bias")
    _shape(cache_in, (B, P, C), "cache_in")
    _shape(cache_out, (B, P, C), "cache_out")
    _shape(out, X.shape, "out")
    _dev(X, "X")
    dt = _dtype(X)
    _dev(w, "w", torch.float32)
    bias = _opt(bias, "bias")
    cache_in = None if cache_in is None else _dev(cache_in, "cache_in", X.dtype)
    cache_out = None if cache_out is None else _dev(cache_out, "cache_out", X.dtype)
    Y = torch.empty_like(X) if out is None else _dev(out, "out", X.dtype)
    lib = library()
    _lib.check(lib, lib.svla_temporal_conv(dt, B, T // F, F, P, C, _ptr(X), _ptr(Y), _ptr(w),
                                           _ptr(bias), _ptr(cache_in), _ptr(cache_out),
                                           _stream(X.device)))
    return Y if cache_out is None else (Y, cache_out)


def state_build(K, V, nb: int, rope=None):
    """Each block's own contribution: S_local [B,H,nb,d,d], z_local [B,H,nb,d]."""
    _qkv_shape(K, K, V)
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
    if not isinstance(S_local, torch.Tensor) or S_local.dim() != 5 or \
            S_local.shape[3] != S_local.shape[4]:
        raise ValueError("S_local must be a [B,H,nb,d,d] tensor")
    B, H, nb, d, _ = S_local.shape
    _shape(z_local, (B, H, nb, d), "z_local")
    _shape(g, (B, H, nb), "g")
    _shape(S0, (B, H, d, d), "S0")
    _shape(z0, (B, H, d), "z0")
    _pair(S0, z0, "S0", "z0")
    _dev(S_local, "S_local", torch.float32)
    _dev(z_local, "z_local", torch.float32)
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
    B, H, N, d = _qkv_shape(Q, Q, Q)
    if nb <= 0 or N % nb:
        raise ValueError("N=%d is not a multiple of nb=%d" % (N, nb))
    _shape(S_prefix, (B, H, nb, d, d), "S_prefix")
    _shape(z_prefix, (B, H, nb, d), "z_prefix")
    _dev(Q, "Q")
    dt = _dtype(Q)
    _dev(S_prefix, "S_prefix", torch.float32)
    _dev(z_prefix, "z_prefix", torch.float32)
    n = N // nb
    lib = library()
    O = _out(None, Q)
    ws = _workspace(workspace_size("apply", Q.dtype, B, H, nb, n, d), Q.device)
    nbytes = 0 if ws is None else ws.numel()
    rp, _keep = _rope_arg(rope)
    _lib.check(lib, lib.svla_apply(dt, B, H, nb, n, d, _ptr(Q), _ptr(S_prefix), _ptr(z_prefix),
                                   rp, float(eps), _ptr(O), _ptr(ws), nbytes,
                                   _stream(Q.device)))
    return O


def block_causal_backward(Q, K, V, dO, nb: int, S0=None, z0=None, g=None, rope=None,
                          eps: float = 1e-6, need_dg: bool = False, need_dstate: bool = False,
                          workspace=None, out: Optional[dict] = None) -> dict:
    """Gradients of ``block_causal`` (same arguments) given dO = dLoss/dO.

    Returns {"dQ", "dK", "dV"} in Q's dtype, plus "dg" [B,H,nb] when
    ``need_dg`` and "dS0" [B,H,d,d], "dz0" [B,H,d] when ``need_dstate``
    (float32).  ``out`` may bring any of these tensors preallocated."""
    B, H, N, d = _qkv_shape(Q, K, V)
    if nb <= 0 or N % nb:
        raise ValueError("N=%d is not a multiple of nb=%d" % (N, nb))
    n = N // nb
    _shape(dO, Q.shape, "dO")
    _shape(S0, (B, H, d, d), "S0")
    _shape(z0, (B, H, d), "z0")
    _shape(g, (B, H, nb), "g")
    _pair(S0, z0, "S0", "z0")
    dt = _qkv(Q, K, V)
    _dev(dO, "dO", Q.dtype)
    S0, z0, g = _opt(S0, "S0"), _opt(z0, "z0"), _opt(g, "g")
    lib = library()
    given = dict(out or {})
    shapes = {"dQ": tuple(Q.shape), "dK": tuple(Q.shape), "dV": tuple(Q.shape), "dg": (B, H, nb),
              "dS0": (B, H, d, d), "dz0": (B, H, d)}
    for k, t in given.items():
        if k not in shapes:
            raise ValueError("unknown output %s" % k)
        _shape(t, shapes[k], k)
    wanted = ["dQ", "dK", "dV"] + (["dg"] if need_dg or "dg" in given else []) + \
        (["dS0", "dz0"] if need_dstate or "dS0" in given or "dz0" in given else [])
    out = {}
    for k in wanted:
        dtype = Q.dtype if k in ("dQ", "dK", "dV") else torch.float32
        out[k] = _dev(given[k], k, dtype) if k in given else \
            torch.empty(shapes[k], dtype=dtype, device=Q.device)
    ws, nbytes = _ws_arg(workspace, "backward", Q, B, H, nb, n, d)
    rp, _keep = _rope_arg(rope)
    st = lib.svla_block_causal_backward(
        dt, B, H, nb, n, d, _ptr(Q), _ptr(K), _ptr(V), _ptr(dO), _ptr(S0), _ptr(z0), _ptr(g), rp,
        float(eps), _ptr(out["dQ"]), _ptr(out["dK"]), _ptr(out["dV"]), _ptr(out.get("dg")),
        _ptr(out.get("dS0")), _ptr(out.get("dz0")), _ptr(ws), nbytes, _stream(Q.device))
    _lib.check(lib, st)
    return out


def softmax_attention(Q, K, V, nb: int, scale: Optional[float] = None,
                      out: Optional[torch.Tensor] = None):
    """Block-causal softmax attention (the 2.0 hybrid's anchor layers): Q
    [B,H,nb*n,d] against K, V [B,H,Nk,d], Nk >= nb*n (the first Nk - nb*n keys
    are a cache of earlier blocks); query i of block c sees keys
    0 .. Nk - nb*n + (c+1)*n - 1.  scale defaults to 1/sqrt(d).  bf16."""
    for t, name in ((Q, "Q"), (K, "K"), (V, "V")):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % name)
    if Q.dim() != 4 or K.dim() != 4 or V.shape != K.shape:
        raise ValueError("Q must be [B,H,Nq,d] and K, V one [B,H,Nk,d] shape")
    B, H, Nq, d = Q.shape
    Nk = K.shape[2]
    if tuple(K.shape[:2]) != (B, H) or K.shape[3] != d:
        raise ValueError("K, V must be [B,H,Nk,d] with Q's B, H and d")
    if nb <= 0 or Nq % nb:
        raise ValueError("Nq=%d is not a multiple of nb=%d" % (Nq, nb))
    if Nk < Nq:
        raise ValueError("Nk=%d is smaller than Nq=%d" % (Nk, Nq))
    _shape(out, Q.shape, "out")
    _dev(Q, "Q", torch.bfloat16)
    _dev(K, "K", torch.bfloat16)
    _dev(V, "V", torch.bfloat16)
    lib = library()
    O = torch.empty(Q.shape, dtype=torch.bfloat16, device=Q.device) if out is None else _dev(out, "out", torch.bfloat16)
    s = (1.0 / float(d) ** 0.5) if scale is None else float(scale)
    st = lib.svla_softmax_attention(_lib.SVLA_BF16, B, H, nb, Nq // nb, Nk, d, _ptr(Q), _ptr(K), _ptr(V),
                                    _ptr(O), s, _stream(Q.device))
    _lib.check(lib, st)
    return O
