"""GPU parity with OCP FP8 E4M3 inputs (Q, K, V one byte per element, O in
bf16), through the C ABI, against the fp64 oracle on the decoded values.

Tolerances are those of the bf16 path: products of fp8 values are exact in
fp32 as products of bf16 values are, the state enters the read-out's matrix
cores rounded to bf16 and O is rounded to bf16, so the error budget is the
bf16 path's (O <= 2e-2, S and z <= 1e-3, normwise per (b,h) slice).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import normwise_error as nerr
from workloads import CONFIGS, Rope, fp8_bits, fp8_from_bits, make_inputs, scaled_config

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
F8 = torch.float8_e4m3fn
TOL_O, TOL_S = 2e-2, 1e-3


@pytest.fixture(scope="module")
def svla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_causal_linear_relu_amd as m
    m.library()
    return m


def _f8(bits):
    """uint8 bit patterns -> a device float8_e4m3fn tensor with those bits."""
    return torch.from_numpy(np.ascontiguousarray(bits)).to(DEV).view(F8)


def _inputs(B, H, nb, n, seed=7, cfg="c3"):
    return make_inputs(scaled_config(CONFIGS[cfg], dtype="fp8", seed=seed), B=B, H=H, nb=nb, n=n)


def test_every_finite_code_decodes_exactly(svla):
    """Block j of one token holds code j in every V feature and 1.0 in every K
    feature, so the block's local state is decode(code j) in every entry: the
    kernels' fp8 decoding against the format's definition, bit for bit."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    nb = len(codes)
    K = np.full((1, 1, nb, 32), fp8_bits(np.array([1.0], dtype=np.float32))[0], dtype=np.uint8)
    V = np.repeat(codes[None, None, :, None], 32, axis=3)
    S, z = svla.state_build(_f8(K), _f8(V), nb)
    torch.cuda.synchronize()
    want = fp8_from_bits(codes)
    got = S[0, 0].cpu().numpy()                        # [nb, 32, 32]
    assert np.array_equal(got, np.broadcast_to(want[:, None, None], got.shape))
    assert torch.all(z == 1.0)


CASES = [
    # name, B, H, nb, n, rope, gate, state_in
    ("ragged", 2, 3, 3, 333, None, False, False),
    ("rope", 1, 3, 3, 333, Rope(8, 12, 12, 5, 7, 0, 1e4), False, False),
    ("gate_state", 1, 3, 4, 200, None, True, True),
    ("rope_gate_state", 1, 2, 3, 390, Rope(8, 12, 12, 15, 26, 6, 1e4), True, True),
    ("token_causal", 1, 2, 40, 1, None, False, False),
    ("noncausal_long", 2, 3, 1, 3000, None, False, False),
    ("noncausal_short", 2, 3, 1, 1000, None, False, True),
    ("long_chain", 1, 3, 17, 70, Rope(8, 12, 12, 5, 7, 1, 1e4), True, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_block_causal(svla, case):
    name, B, H, nb, n, rope, gate, state_in = case
    x = _inputs(B, H, nb, n)
    rng = np.random.default_rng(99)
    g = rng.uniform(0.3, 1.0, (B, H, nb)).astype(np.float32) if gate else None
    S0 = z0 = None
    if state_in:
        S0 = (rng.standard_normal((B, H, 32, 32)) * 30).astype(np.float32)
        z0 = np.abs(rng.standard_normal((B, H, 32)) * 100).astype(np.float32)
    t = lambda a: None if a is None else torch.from_numpy(a).to(DEV)
    O, S, z = svla.block_causal(_f8(x["Q_bits"]), _f8(x["K_bits"]), _f8(x["V_bits"]), nb, S0=t(S0),
                                z0=t(z0), g=t(g), rope=rope, return_state=True)
    torch.cuda.synchronize()
    assert O.dtype == torch.bfloat16
    ref = oracle.forward(x["Q"], x["K"], x["V"], nb, g=g, rope=rope, S0=S0, z0=z0, eps=x["eps"])
    eo = nerr(O.float().cpu().numpy(), ref["O"])
    es, ez = nerr(S.cpu().numpy(), ref["S"]), nerr(z.cpu().numpy(), ref["z"])
    assert eo <= TOL_O and es <= TOL_S and ez <= TOL_S, (eo, es, ez)


@pytest.mark.parametrize("rope", [None, Rope(8, 12, 12, 5, 7, 3, 1e4)])
def test_kernels_one_by_one(svla, rope):
    x = _inputs(1, 2, 3, 211)
    S, z = svla.state_build(_f8(x["K_bits"]), _f8(x["V_bits"]), 3, rope=rope)
    ref = oracle.forward(x["Q"], x["K"], x["V"], 3, rope=rope, want_local=True, want_blocks=True)
    torch.cuda.synchronize()
    assert nerr(S.cpu().numpy(), ref["S_local"]) <= 1e-5
    assert nerr(z.cpu().numpy(), ref["z_local"]) <= 1e-6
    O = svla.apply(_f8(x["Q_bits"]), torch.from_numpy(ref["S_blocks"].astype(np.float32)).to(DEV),
                   torch.from_numpy(ref["z_blocks"].astype(np.float32)).to(DEV), 3, rope=rope)
    torch.cuda.synchronize()
    assert nerr(O.float().cpu().numpy(), ref["O"]) <= TOL_O


@pytest.mark.parametrize("commit", ["in_place", "double_buffer"])
@pytest.mark.parametrize("with_rope,gate", [(True, False), (False, True)])
def test_chained_steps(svla, commit, with_rope, gate):
    """fp8 block steps (the one-launch step double-buffered, the two-kernel
    step in place) chained over 6 blocks against the oracle."""
    gh, gw, frames, nb, H = 5, 6, 2, 6, 3
    n = frames * gh * gw
    x = _inputs(1, H, nb, n, seed=21)
    rope = Rope(8, 12, 12, gh, gw, 0, 1e4) if with_rope else None
    g = np.random.default_rng(3).uniform(0.5, 1.0, (1, H, nb)).astype(np.float32) if gate else None
    Q, K, V = (_f8(x[k + "_bits"]) for k in "QKV")
    bufs = [(torch.zeros((1, H, 32, 32), device=DEV), torch.zeros((1, H, 32), device=DEV)) for _ in range(2)]
    nbuf = 2 if commit == "double_buffer" else 1
    outs = []
    for s in range(nb):
        sl = slice(s * n, (s + 1) * n)
        S, z = bufs[s % nbuf]
        Sn, zn = bufs[(s + 1) % nbuf]
        gs = None if g is None else torch.from_numpy(np.ascontiguousarray(g[:, :, s])).to(DEV)
        O, _, _ = svla.block_step(Q[:, :, sl].contiguous(), K[:, :, sl].contiguous(),
                                  V[:, :, sl].contiguous(), S, z, S_out=Sn, z_out=zn, g=gs,
                                  rope=Rope(8, 12, 12, gh, gw, frames * s, 1e4) if with_rope else None)
        outs.append(O)
    S, z = bufs[nb % nbuf]
    torch.cuda.synchronize()
    ref = oracle.forward(x["Q"], x["K"], x["V"], nb, g=g, rope=rope)
    eo = nerr(torch.cat(outs, 2).float().cpu().numpy(), ref["O"])
    assert eo <= TOL_O and nerr(S.cpu().numpy(), ref["S"]) <= TOL_S and nerr(z.cpu().numpy(), ref["z"]) <= TOL_S


@pytest.mark.parametrize("with_rope", [False, True])
def test_one_launch_step_four_q_groups(svla, with_rope):
    """An fp8 block step of 70 heads x 2640 tokens: one launch whose waves
    read out four 16-token Q groups each, against the oracle's step."""
    H, n = 70, 2640
    x = _inputs(1, H, 1, n, seed=27)
    rng = np.random.default_rng(28)
    S_in = (rng.standard_normal((1, H, 32, 32)) * 20).astype(np.float32)
    z_in = np.abs(rng.standard_normal((1, H, 32)) * 80).astype(np.float32)
    rope = Rope(8, 12, 12, 5, 7, 4, 1e4) if with_rope else None
    plan = svla.describe("block_step", F8, 1, H, 1, n, 32, rope=rope)
    assert [k["slot"] for k in plan["kernels"]] == ["step"] and plan["step_tile"] > 16 * 16 * 2, plan
    Q, K, V = (_f8(x[k + "_bits"]) for k in "QKV")
    O, S, z = svla.block_step(Q, K, V, torch.from_numpy(S_in).to(DEV), torch.from_numpy(z_in).to(DEV),
                              rope=rope)
    torch.cuda.synchronize()
    ref = oracle.step(x["Q"], x["K"], x["V"], S_in, z_in, rope=rope, eps=x["eps"])
    assert nerr(O.float().cpu().numpy(), ref["O"]) <= TOL_O
    assert nerr(S.cpu().numpy(), ref["S"]) <= TOL_S and nerr(z.cpu().numpy(), ref["z"]) <= TOL_S


@pytest.mark.parametrize("name", ["c2", "c3", "c4"])
def test_full_size_every_head(svla, name):
    """The 480p, 720p and minute-long shapes with fp8 inputs (the minute-long
    one as one call), every head against the oracle."""
    cfg = scaled_config(CONFIGS[name], dtype="fp8")
    x = make_inputs(cfg)
    Q, K, V = (_f8(x[k + "_bits"]) for k in "QKV")
    O, S, z = svla.block_causal(Q, K, V, cfg.nb, rope=cfg.rope, return_state=True)
    torch.cuda.synchronize()
    O, S, z = O.float().cpu().numpy(), S.cpu().numpy(), z.cpu().numpy()
    worst = [0.0, 0.0, 0.0]
    for h0 in range(0, cfg.H, 14):
        hs = slice(h0, min(h0 + 14, cfg.H))
        sub = lambda a: np.ascontiguousarray(a[:, hs])
        ref = oracle.forward(sub(x["Q"]), sub(x["K"]), sub(x["V"]), cfg.nb, rope=cfg.rope, eps=cfg.eps)
        worst = [max(w, e) for w, e in zip(worst, (nerr(O[:, hs], ref["O"]), nerr(S[:, hs], ref["S"]),
                                                   nerr(z[:, hs], ref["z"])))]
    print("%s fp8 all %d heads: O %.2e S %.2e z %.2e" % (name, cfg.H, *worst))
    assert worst[0] <= TOL_O and worst[1] <= TOL_S and worst[2] <= TOL_S
