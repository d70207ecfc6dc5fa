"""C-ABI contract on the CPU: the library loads, exports every declared symbol,
and rejects bad arguments before any HIP call (nothing is launched)."""
import ctypes
import os
import re

import pytest

from block_causal_linear_relu_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def _declared():
    text = open(os.path.join(ROOT, "include", "svla.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(svla_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 12
    for name in names:
        assert hasattr(lib, name), name
        assert name in _lib.PROTOTYPES, name


def test_version_and_strings(lib):
    assert lib.svla_abi_version() == 1
    assert lib.svla_status_string(0) == b"SVLA_OK"
    assert lib.svla_status_string(6) == b"SVLA_ERR_WORKSPACE"


def _ws(lib, *args):
    out = ctypes.c_size_t(12345)
    st = lib.svla_workspace_size(*args, ctypes.byref(out))
    return st, out.value


def test_workspace_size(lib):
    st, n1 = _ws(lib, _lib.OP_BLOCK_STEP, _lib.SVLA_BF16, 1, 70, 1, 1170, 32)
    assert st == 0 and n1 > 0
    # the state is the only thing carried: the step's workspace does not grow
    st, n2 = _ws(lib, _lib.OP_BLOCK_STEP, _lib.SVLA_BF16, 1, 70, 1, 1170, 32)
    assert n2 == n1
    st, n3 = _ws(lib, _lib.OP_STATE_BUILD, _lib.SVLA_BF16, 1, 70, 7, 2640, 32)
    assert st == 0 and n3 == 0
    st, _ = _ws(lib, _lib.OP_BLOCK_CAUSAL, _lib.SVLA_BF16, 1, 70, 7, 2640, 48)
    assert st == 5
    st, _ = _ws(lib, _lib.OP_BLOCK_CAUSAL, 7, 1, 70, 7, 2640, 32)
    assert st == 3
    st, _ = _ws(lib, 99, _lib.SVLA_BF16, 1, 70, 7, 2640, 32)
    assert st == 7
    st, n = _ws(lib, _lib.OP_NONCAUSAL, _lib.SVLA_BF16, 0, 70, 1, 10, 32)
    assert st == 0


# Fake, aligned, never dereferenced "device" addresses: every case below
# must fail validation before any HIP call.
A = ctypes.c_void_p(0x10000)
A2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10004)


def _bc(lib, **kw):
    a = dict(dt=_lib.SVLA_BF16, B=1, H=2, nb=2, n=64, d=32, Q=A, K=A, V=A, O=A2, S0=None,
             z0=None, Sf=None, zf=None, rope=None, eps=1e-6, ws=A, wsb=1 << 30)
    a.update(kw)
    st = lib.svla_block_causal(a["dt"], a["B"], a["H"], a["nb"], a["n"], a["d"], a["Q"], a["K"],
                               a["V"], a["O"], a["S0"], a["z0"], a["Sf"], a["zf"], a["rope"],
                               a["eps"], a["ws"], a["wsb"], None)
    return st, lib.svla_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), 1),
    (dict(O=None), 1),
    (dict(ws=None), 1),
    (dict(S0=A), 1),                      # S0 without z0
    (dict(Sf=A), 1),                      # S_final without z_final
    (dict(B=-1), 2),
    (dict(n=-5), 2),
    (dict(nb=1, n=(1 << 31) // 64), 2),   # one slice >= 2 GiB
    (dict(dt=5), 3),
    (dict(Q=MIS), 4),
    (dict(O=MIS), 4),
    (dict(d=16), 5),
    (dict(d=256), 5),
    (dict(wsb=16), 6),
    (dict(eps=-1.0), 7),
    (dict(eps=float("nan")), 7),
    (dict(eps=float("inf")), 7),
])
def test_block_causal_rejects(lib, kw, status):
    st, msg = _bc(lib, **kw)
    assert st == status, msg
    assert msg.startswith("svla_block_causal:")


@pytest.mark.parametrize("rope,status", [
    (_lib.SvlaRope(7, 12, 12, 15, 26, 0, 1e4), 7),      # odd split
    (_lib.SvlaRope(8, 12, 14, 15, 26, 0, 1e4), 7),      # 34 > d
    (_lib.SvlaRope(8, 12, 12, 0, 26, 0, 1e4), 7),       # empty grid
    (_lib.SvlaRope(8, 12, 12, 15, 26, -3, 1e4), 7),     # negative t0
    (_lib.SvlaRope(8, 12, 12, 15, 26, 0, 0.0), 7),      # base 0
    (_lib.SvlaRope(8, 12, 12, 4000, 4000, 0, 1e4), 5),  # table too large
])
def test_rope_rejects(lib, rope, status):
    st, msg = _bc(lib, rope=ctypes.byref(rope))
    assert st == status, msg


def test_empty_is_ok_without_launch(lib):
    st, msg = _bc(lib, B=0, Q=None, K=None, V=None, O=None, ws=None, wsb=0)
    assert st == 0, msg


def test_gated_needs_g(lib):
    st = lib.svla_block_causal_gated(_lib.SVLA_BF16, 1, 2, 2, 64, 32, A, A, A, A2, None, None,
                                     None, None, None, None, 1e-6, A, 1 << 30, None)
    assert st == 1


def test_step_needs_state_out(lib):
    st = lib.svla_block_step(_lib.SVLA_BF16, 1, 2, 64, 32, A, A, A, A2, None, None, None, None,
                             None, 1e-6, A, 1 << 30, None)
    assert st == 1


def test_other_entry_points_validate(lib):
    assert lib.svla_noncausal(_lib.SVLA_BF16, 1, 2, 100, 32, A, A, A, A2, -1.0, None, None, A,
                              1 << 30, None) == 7
    assert lib.svla_state_build(_lib.SVLA_BF16, 1, 2, 2, 64, 32, A, A, None, None, A, None, 0,
                                None) == 1
    assert lib.svla_state_scan(1, 2, 2, 32, A, A, None, A, None, A, A, None) == 1
    assert lib.svla_state_scan(1, 2, 2, 32, MIS, A, None, None, None, A, A, None) == 4
    assert lib.svla_apply(_lib.SVLA_BF16, 1, 2, 2, 64, 32, A, A, A, None, 1e-6, A2, A, 8,
                          None) == 6


def test_workspace_covers_every_plan():
    """svla_workspace_size takes no RoPE argument, so the workspace it gives
    must hold the partials of whichever build the call picks, RoPE or not;
    the plan the library describes (svla_describe, host logic only) must fit."""
    import torch
    import block_causal_linear_relu_amd as svla
    from workloads import Rope
    shapes = [
        ("block_step", 1, 70, 1, 1170, 32), ("block_causal", 1, 70, 80, 1170, 32),
        ("noncausal", 2, 70, 1, 8190, 32), ("block_causal", 1, 70, 7, 2640, 32),
        ("block_causal", 1, 20, 8, 1760, 128), ("block_step", 1, 20, 1, 1760, 128),
        ("block_causal", 1, 3, 3, 333, 32), ("block_step", 2, 5, 1, 77, 64),
        ("block_causal", 1, 40, 30, 37, 32),
    ]
    for op, B, H, nb, n, d in shapes:
        ws = svla.workspace_size(op, torch.bfloat16, B, H, nb, n, d)
        rope = Rope(8, 12, 12, 5, 7, 3, 1e4)
        plain = svla.describe(op, torch.bfloat16, B, H, nb, n, d)
        rot = svla.describe(op, torch.bfloat16, B, H, nb, n, d, rope=rope)
        assert plain["workspace"] == ws and rot["workspace"] == ws, (op, B, H, nb, n, d)
        # one-block bf16 d = 32 calls fold the scan into the apply (with RoPE
        # as long as the block's splits fit the apply's partial count: the
        # minute-long block step does)
        if nb == 1 and d == 32:
            # up to 3072 tokens: one launch, or (new state over the old one)
            # build and apply
            short = n <= 3072
            key = "in_place_kernels" if short else "kernels"
            assert plain["fused"] is short and rot["fused"] is short
            assert [k["slot"] for k in plain[key]] == ["build", "apply"]
            if short:
                assert [k["slot"] for k in plain["kernels"]] == ["step"]
                assert [k["slot"] for k in rot["kernels"]] == ["step"]
            if op == "block_step" and n == 1170:
                assert [k["slot"] for k in rot["in_place_kernels"]] == ["build", "apply"]
                assert rot["step_tiles"] * rot["step_tile"] >= n
        else:
            assert plain["fused"] is False and "in_place_kernels" not in plain


def test_noalloc_step_validates_before_any_hip_call(lib):
    """The no-alloc block step rejects a step whose workspace exceeds the
    library's scratch, and bad arguments, on the host (no GPU here)."""
    A = ctypes.c_void_p(4096)        # aligned stand-ins; never dereferenced on a rejection
    MIS = ctypes.c_void_p(4100)
    f = lib.svla_block_step_noalloc
    # 40 heads of 8192 tokens at d = 128 need about 34 MiB of scratch (> 32 MiB)
    assert f(_lib.SVLA_BF16, 1, 40, 8192, 128, A, A, A, A, None, None, A, A, None, None,
             1e-6, None) == 6
    assert b"scratch" in lib.svla_last_error()
    assert f(_lib.SVLA_BF16, 1, 2, 64, 32, A, A, A, A, None, None, None, None, None, None,
             1e-6, None) == 1                                  # S_out, z_out required
    assert f(_lib.SVLA_BF16, 1, 2, 64, 32, A, A, A, MIS, None, None, A, A, None, None,
             1e-6, None) == 4                                  # misaligned O
    assert f(_lib.SVLA_BF16, 1, 2, 64, 48, A, A, A, A, None, None, A, A, None, None,
             1e-6, None) == 5                                  # d = 48
    assert f(_lib.SVLA_BF16, 1, 2, 64, 32, A, A, A, A, None, None, A, A, None, None,
             -1.0, None) == 7                                  # eps < 0
    assert f(_lib.SVLA_BF16, 0, 2, 64, 32, None, None, None, None, None, None, None, None,
             None, None, 1e-6, None) == 0                      # empty: nothing to do


def test_temporal_conv_rejects(lib):
    A, MIS = ctypes.c_void_p(4096), ctypes.c_void_p(4100)
    f = lib.svla_temporal_conv
    bf = _lib.SVLA_BF16
    assert f(bf, 1, 2, 3, 4, 12, A, ctypes.c_void_p(1 << 20), A, None, None, None, None) == 5   # C % 8
    assert f(bf, 1, 2, 0, 4, 16, A, ctypes.c_void_p(1 << 20), A, None, None, None, None) == 2   # F = 0
    assert f(7, 1, 2, 3, 4, 16, A, ctypes.c_void_p(1 << 20), A, None, None, None, None) == 3
    assert f(bf, 1, 2, 3, 4, 16, None, A, A, None, None, None, None) == 1
    assert f(bf, 1, 2, 3, 4, 16, A, MIS, A, None, None, None, None) == 4
    # Y overlapping X
    assert f(bf, 1, 2, 3, 4, 16, A, ctypes.c_void_p(4096 + 64), A, None, None, None, None) == 7
    # one batch's frames past 2 GiB
    assert f(bf, 1, 1000, 3, 1000, 1024, A, ctypes.c_void_p(1 << 40), A, None, None, None, None) == 2
    # nothing to do
    assert f(bf, 0, 2, 3, 4, 16, None, None, None, None, None, None, None) == 0


def test_fp8_is_d32_only(lib):
    st, _ = _ws(lib, _lib.OP_BLOCK_CAUSAL, _lib.SVLA_FP8, 1, 70, 7, 2640, 64)
    assert st == 5 and b"fp8" in lib.svla_last_error()
    st, n = _ws(lib, _lib.OP_BLOCK_CAUSAL, _lib.SVLA_FP8, 1, 70, 7, 2640, 32)
    assert st == 0 and n > 0


def _bwd(lib, **kw):
    a = dict(dt=_lib.SVLA_BF16, B=1, H=2, nb=2, n=64, d=32, Q=A, K=A, V=A, dO=A,
             S0=None, z0=None, g=None, rope=None, eps=1e-6,
             dQ=ctypes.c_void_p(1 << 30), dK=ctypes.c_void_p(2 << 30), dV=ctypes.c_void_p(3 << 30),
             dg=None, dS0=None, dz0=None, ws=ctypes.c_void_p(4 << 30), wsb=1 << 30)
    a.update(kw)
    return lib.svla_block_causal_backward(
        a["dt"], a["B"], a["H"], a["nb"], a["n"], a["d"], a["Q"], a["K"], a["V"], a["dO"],
        a["S0"], a["z0"], a["g"], a["rope"], a["eps"], a["dQ"], a["dK"], a["dV"], a["dg"],
        a["dS0"], a["dz0"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dO=None), 1),
    (dict(dV=None), 1),
    (dict(ws=None), 1),
    (dict(S0=A), 1),                      # S0 without z0
    (dict(dS0=A), 1),                     # dS0 without dz0
    (dict(n=-1), 2),
    (dict(dt=_lib.SVLA_FP8), 5),          # no backward for fp8 inputs
    (dict(d=128), 5),
    (dict(d=48), 5),
    (dict(dQ=MIS), 4),
    (dict(dg=MIS), 4),
    (dict(wsb=64), 6),
    (dict(eps=-1.0), 7),
    (dict(dQ=A), 7),                      # dQ overlapping the inputs
    (dict(dK=ctypes.c_void_p((1 << 30) + 64)), 7),   # dK overlapping dQ
])
def test_backward_rejects(lib, kw, status):
    assert _bwd(lib, **kw) == status, lib.svla_last_error()


def test_backward_empty_and_workspace(lib):
    assert _bwd(lib, B=0, Q=None, K=None, V=None, dO=None, dQ=None, dK=None, dV=None,
                ws=None) == 0
    st, n = _ws(lib, _lib.OP_BACKWARD, _lib.SVLA_BF16, 1, 70, 7, 2640, 32)
    assert st == 0
    # at least the rebuilt prefix states, the query partials and G, H
    assert n >= 70 * 7 * (32 * 32 + 32) * 4 * 3
    assert _bwd(lib, B=1, H=70, nb=7, n=2640, wsb=n - 1) == 6
    st, _ = _ws(lib, _lib.OP_BACKWARD, _lib.SVLA_BF16, 1, 20, 8, 1760, 128)
    assert st == 5


def test_hbm_probe_rejects(lib):
    f = lib.svla_hbm_probe
    S = ctypes.c_void_p(0x20000)
    assert f(2, A, A2, 1 << 24, S, 16, None) == 7           # mode
    assert f(0, A, None, 1 << 24, S, 0, None) == 7          # no workgroups
    assert f(0, None, None, 1 << 24, S, 16, None) == 1      # src
    assert f(0, A, None, 1 << 24, None, 16, None) == 1      # sink for the read
    assert f(1, A, None, 1 << 24, None, 16, None) == 1      # dst for the copy
    assert f(0, A, None, (1 << 24) + 16, S, 16, None) == 2  # not whole 16 KiB chunks
    assert f(1, MIS, A2, 1 << 24, None, 16, None) == 4


def test_softmax_attention_rejects(lib):
    f = lib.svla_softmax_attention
    bf = _lib.SVLA_BF16
    assert f(_lib.SVLA_F32, 1, 2, 2, 64, 128, 128, A, A, A, A2, 0.1, None) == 3
    assert f(bf, 1, 2, 2, 64, 128, 32, A, A, A, A2, 0.1, None) == 5          # d
    assert f(bf, 1, 2, 2, 64, 100, 128, A, A, A, A2, 0.1, None) == 2         # Nk < nb*n
    assert f(bf, 1, 2, 2, 64, 128, 128, A, A, A, A2, 0.0, None) == 7         # scale
    assert f(bf, 1, 2, 2, 64, 128, 128, A, A, None, A2, 0.1, None) == 1
    assert f(bf, 1, 2, 2, 64, 128, 128, MIS, A, A, A2, 0.1, None) == 4
    assert f(bf, 1, 2, 2, 64, 128, 128, A, A, A, A, 0.1, None) == 7          # O overlaps Q
    assert f(bf, 0, 2, 2, 64, 128, 128, None, None, None, None, 0.1, None) == 0
    assert f(bf, 1, 2, 1, 1 << 24, 1 << 24, 128, A, A, A, A2, 0.1, None) == 2  # a K slice past 2 GiB
