"""GPU parity of the backward pass (svla_block_causal_backward through the C
ABI) against the numpy fp64 oracle (oracle.backward, pinned by finite
differences of the forward oracle).

Tolerances (normwise per (b, h) slice, the oracle's measure).  Every step
of the kernels is fp32 arithmetic on exact inputs: the rebuilt states are sums
of at most n products per entry, each gradient a sum of at most d (features) or
n (tokens) fp32 products, so the relative error before the final rounding is a
small multiple of 2^-24 times sqrt(n d), below 1e-5 at these sizes.
  * dQ, dK, dV in bf16: dominated by the final rounding, at most 2^-9 of the
    largest element; tested at 2^-8.
  * fp32 outputs (dQ, dK, dV for fp32 inputs; dg, dS0, dz0 always): 1e-4.
"""
import numpy as np
import pytest
import torch

from oracle import normwise_error as nerr
from oracle.backward import backward
from workloads import CONFIGS, Rope, make_grad_output, make_inputs, scaled_config

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_BF16, TOL_F32 = 2.0 ** -8, 1e-4


@pytest.fixture(scope="module")
def svla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_causal_linear_relu_amd as m
    m.library()
    return m


def _t(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dtype)


def _case(dtype, B, H, d, nb, n, gate, state, seed):
    base = CONFIGS["c5"] if gate else CONFIGS["c3"]
    cfg = scaled_config(base, d=d, dtype=dtype, seed=seed, rope=None)
    x = make_inputs(cfg, B=B, H=H, nb=nb, n=n)
    dO = make_grad_output(x, seed + 1000)
    S0 = z0 = None
    if state:
        rng = np.random.default_rng(seed + 2000)
        S0 = (rng.standard_normal((B, H, d, d)) * 30).astype(np.float32)
        z0 = np.abs(rng.standard_normal((B, H, d)) * 100).astype(np.float32)
    return x, dO, S0, z0


def _run(svla, x, dO, S0, z0, rope, eps):
    dt = torch.bfloat16 if x["dtype"] == "bf16" else torch.float32
    Q, K, V, dOt = (_t(a, dt) for a in (x["Q"], x["K"], x["V"], dO))
    g = None if x["g"] is None else _t(x["g"], torch.float32)
    S0t = None if S0 is None else _t(S0, torch.float32)
    z0t = None if z0 is None else _t(z0, torch.float32)
    out = svla.block_causal_backward(Q, K, V, dOt, x["nb"], S0=S0t, z0=z0t, g=g, rope=rope,
                                     eps=eps, need_dg=True, need_dstate=True)
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy() for k, v in out.items()}


def _check(got, ref, dtype, names=("dQ", "dK", "dV", "dg", "dS0", "dz0")):
    errs = {}
    for k in names:
        tol = TOL_BF16 if (dtype == "bf16" and k in ("dQ", "dK", "dV")) else TOL_F32
        errs[k] = nerr(got[k], ref[k])
        assert np.all(np.isfinite(got[k])), k
        assert errs[k] <= tol, "%s: normwise error %.3e > %.1e (all: %s)" % (k, errs[k], tol, errs)
    return errs


CASES = [
    # name, dtype, B, H, d, nb, n, gate, rope, carried state, eps
    ("f32_d32_ragged_tail", "f32", 1, 2, 32, 4, 200, False, None, False, 1e-6),
    ("bf16_d32_rope_gate_state", "bf16", 1, 3, 32, 3, 180, True,
     Rope(8, 12, 12, 6, 10, 2, 10000.0), True, 1e-6),
    ("bf16_d32_four_splits", "bf16", 1, 1, 32, 2, 1000, False, None, False, 1e-6),
    ("bf16_d32_one_token_blocks", "bf16", 1, 2, 32, 9, 1, True, None, True, 1e-6),
    ("bf16_d64_gate_state", "bf16", 2, 2, 64, 5, 300, True, None, True, 1e-6),
    ("f32_d64_rope", "f32", 1, 2, 64, 2, 257, False, Rope(16, 24, 24, 5, 7, 0, 10000.0), False, 1e-6),
    ("bf16_d64_rope_partial_dims", "bf16", 1, 2, 64, 3, 96, True,
     Rope(8, 12, 12, 4, 6, 1, 500.0), False, 1e-3),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(svla, case):
    name, dtype, B, H, d, nb, n, gate, rope, state, eps = case
    print("backward case %s: B=%d H=%d d=%d nb=%d n=%d" % (name, B, H, d, nb, n), flush=True)
    x, dO, S0, z0 = _case(dtype, B, H, d, nb, n, gate, state, seed=70 + len(name))
    got = _run(svla, x, dO, S0, z0, rope, eps)
    ref = backward(x["Q"], x["K"], x["V"], nb, dO, g=x["g"], rope=rope, S0=S0, z0=z0, eps=eps)
    _check(got, ref, dtype)


def test_dead_tokens_pass_no_gradient(svla):
    """eps = 0: tokens whose phi(q) is zero have a zero denominator and pass
    no gradient; a block whose keys are all negative adds nothing to z."""
    x, dO, _, _ = _case("f32", 1, 2, 32, 3, 64, False, False, seed=91)
    x["Q"][:, :, 5:40:3, :] = -np.abs(x["Q"][:, :, 5:40:3, :]) - 0.25
    x["K"][:, :, 0:64, :] = -np.abs(x["K"][:, :, 0:64, :]) - 0.25
    got = _run(svla, x, dO, None, None, None, 0.0)
    ref = backward(x["Q"], x["K"], x["V"], 3, dO, eps=0.0)
    _check(got, ref, "f32")
    assert np.all(got["dQ"][:, :, 5:40:3, :] == 0.0)
    assert np.all(got["dQ"][:, :, 0:64, :] == 0.0)     # block 0: z_0 = 0, every denominator 0


def test_no_tokens(svla):
    """n = 0: nothing reaches the carried state or the gates."""
    B, H, d, nb = 1, 2, 32, 3
    e = torch.empty((B, H, 0, d), dtype=torch.bfloat16, device=DEV)
    S0 = torch.ones((B, H, d, d), dtype=torch.float32, device=DEV)
    z0 = torch.ones((B, H, d), dtype=torch.float32, device=DEV)
    g = torch.full((B, H, nb), 0.5, dtype=torch.float32, device=DEV)
    out = svla.block_causal_backward(e, e, e, e, nb, S0=S0, z0=z0, g=g, need_dg=True,
                                     need_dstate=True)
    torch.cuda.synchronize()
    for k in ("dg", "dS0", "dz0"):
        assert torch.count_nonzero(out[k]).item() == 0, k


def test_full_size_720p_every_head(svla):
    """The 720p block-causal workload (7 blocks of 2640 tokens, 70 heads, bf16,
    d = 32) in the launch plan the benchmark times, every head against the
    oracle."""
    cfg = CONFIGS["c3"]
    print("backward full size c3", flush=True)
    x = make_inputs(cfg)
    dO = make_grad_output(x, 1003)
    got = _run(svla, x, dO, None, None, None, cfg.eps)
    for h0 in range(0, cfg.H, 14):
        sl = slice(h0, h0 + 14)
        ref = backward(x["Q"][:, sl], x["K"][:, sl], x["V"][:, sl], cfg.nb, dO[:, sl], eps=cfg.eps)
        _check({k: v[:, sl] for k, v in got.items()}, ref, "bf16")


def test_repeatable(svla):
    """Two calls on the same inputs give the same bits (fixed summation order)."""
    x, dO, S0, z0 = _case("bf16", 1, 2, 32, 3, 500, True, True, seed=95)
    a = _run(svla, x, dO, S0, z0, None, 1e-6)
    b = _run(svla, x, dO, S0, z0, None, 1e-6)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
