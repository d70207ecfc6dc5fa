"""GPU parity: libsvla (through the C ABI) against the fp64 CPU oracle.

Tolerances (normwise per (b,h) slice: max|x - ref| / max|ref|):
  O      <= 2e-2 for bf16 inputs, <= 1e-4 for fp32 inputs
  S, z   <= 1e-3
Small cases compare every element and span several stages/tiles plus a
ragged tail; full-size workloads compare every element of every head (the
oracle runs over groups of heads to bound host memory; heads are
independent, so the per-slice measure is the same).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import brute_force
from oracle import normwise_error as nerr
from workloads import CONFIGS, Rope, make_inputs, scaled_config

pytestmark = pytest.mark.gpu

TOL_O = {"bf16": 2e-2, "f32": 1e-4}
TOL_S = 1e-3


@pytest.fixture(scope="module")
def svla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_causal_linear_relu_amd as m
    m.library()          # fails loudly if the HIP library is missing
    return m


DEV = "cuda:0"


def _t(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dtype)


def _tdt(x):
    return torch.bfloat16 if x["dtype"] == "bf16" else torch.float32


def _np(t):
    return t.float().cpu().numpy()


def _run_gpu(svla, x, g=None, S0=None, z0=None, rope=None):
    dt = _tdt(x)
    Q, K, V = _t(x["Q"], dt), _t(x["K"], dt), _t(x["V"], dt)
    gt = None if g is None else _t(g, torch.float32)
    S0t = None if S0 is None else _t(S0, torch.float32)
    z0t = None if z0 is None else _t(z0, torch.float32)
    O, S, z = svla.block_causal(Q, K, V, x["nb"], S0=S0t, z0=z0t, g=gt, rope=rope,
                                eps=x["eps"], return_state=True)
    torch.cuda.synchronize()
    return _np(O), S.cpu().numpy(), z.cpu().numpy()


def _check(x, got, ref, heads=None):
    O, S, z = got
    if heads is not None:
        O, S, z = O[:, heads], S[:, heads], z[:, heads]
    eo, es, ez = nerr(O, ref["O"]), nerr(S, ref["S"]), nerr(z, ref["z"])
    tol = TOL_O[x["dtype"]]
    assert eo <= tol and es <= TOL_S and ez <= TOL_S, (eo, es, ez)
    return eo, es, ez


def _small(dtype, B, H, nb, n, d, seed=7):
    base = CONFIGS["c1"] if dtype == "f32" else CONFIGS["c3"]
    cfg = scaled_config(base, d=d, seed=seed)
    return make_inputs(cfg, B=B, H=H, nb=nb, n=n)


SMALL = [
    # name, dtype, B, H, nb, n, d, rope, gate, state_in
    ("f32_tiny_shape_seed7", "f32", 1, 2, 4, 256, 32, None, False, False),
    ("f32_d64_ragged", "f32", 1, 2, 3, 100, 64, None, True, False),
    ("f32_d128_rope_gate", "f32", 1, 1, 2, 77, 128, Rope(8, 12, 12, 5, 7, 2, 1e4), True, True),
    ("bf16_d32_ragged", "bf16", 2, 3, 3, 333, 32, None, False, False),
    ("bf16_d32_rope", "bf16", 1, 3, 3, 333, 32, Rope(8, 12, 12, 5, 7, 0, 1e4), False, False),
    ("bf16_d32_gate_state", "bf16", 1, 3, 4, 200, 32, None, True, True),
    ("bf16_d32_rope_gate", "bf16", 1, 2, 3, 390, 32, Rope(8, 12, 12, 15, 26, 6, 1e4), True, False),
    ("bf16_d64_rope_gate", "bf16", 1, 3, 2, 300, 64, Rope(16, 24, 24, 6, 10, 1, 1e4), True, False),
    ("bf16_d128_gate", "bf16", 1, 2, 3, 257, 128, None, True, False),
    ("bf16_d128_rope", "bf16", 1, 2, 2, 300, 128, Rope(40, 44, 44, 6, 10, 0, 1e4), False, True),
    ("bf16_d32_token_causal", "bf16", 1, 2, 40, 1, 32, None, False, False),
    ("bf16_d32_noncausal", "bf16", 2, 3, 1, 1000, 32, None, False, False),
    # over a thousand short ragged blocks (one-stage and two-stage blocks)
    ("bf16_d32_many_blocks", "bf16", 1, 40, 30, 37, 32, None, False, False),
    ("bf16_d32_many_blocks_rope_gate_state", "bf16", 2, 50, 12, 100, 32, Rope(8, 12, 12, 5, 7, 3, 1e4), True, True),
    # an angle table of over a thousand entries (wide latent grid)
    ("bf16_d32_rope_wide_grid", "bf16", 1, 2, 3, 300, 32, Rope(8, 12, 12, 100, 100, 0, 1e4), False, False),
    # chains of 16 blocks or more take the segmented scan (four waves, each a
    # quarter of the blocks, composed through LDS): with a gate and a state in
    ("bf16_d128_long_chain_gate_state", "bf16", 1, 2, 20, 64, 128, None, True, True),
    ("f32_d64_long_chain_gate_state", "f32", 1, 2, 18, 50, 64, None, True, True),
    ("bf16_d64_long_chain_gate_state", "bf16", 1, 3, 17, 90, 64, None, True, True),
    ("bf16_d32_long_chain_rope_gate_state", "bf16", 1, 3, 17, 70, 32, Rope(8, 12, 12, 5, 7, 1, 1e4), True, True),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_block_causal_small(svla, case):
    name, dtype, B, H, nb, n, d, rope, gate, state_in = case
    x = _small(dtype, B, H, nb, n, d)
    rng = np.random.default_rng(99)
    g = rng.uniform(0.3, 1.0, (B, H, nb)).astype(np.float32) if gate else None
    S0 = z0 = None
    if state_in:
        S0 = (rng.standard_normal((B, H, d, d)) * 30).astype(np.float32)
        z0 = np.abs(rng.standard_normal((B, H, d)) * 100).astype(np.float32)
    got = _run_gpu(svla, x, g=g, S0=S0, z0=z0, rope=rope)
    ref = oracle.forward(x["Q"], x["K"], x["V"], nb, g=g, rope=rope, S0=S0, z0=z0, eps=x["eps"])
    _check(x, got, ref)


def test_tiny_workload_on_its_own_inputs(svla):
    """The tiny fp32 workload's own seeded inputs (the ones the CPU tests check
    the oracle on against the quadratic brute force) through the GPU, compared
    with the oracle and with the brute force."""
    x = make_inputs(CONFIGS["c1"])
    got = _run_gpu(svla, x)
    ref = oracle.forward(x["Q"], x["K"], x["V"], x["nb"], eps=x["eps"])
    _check(x, got, ref)
    bf = brute_force(x["Q"], x["K"], x["V"], x["nb"], eps=x["eps"])
    assert nerr(got[0], bf) <= TOL_O["f32"]


def test_noncausal_entry_point(svla):
    x = _small("bf16", 2, 3, 1, 1000, 32)
    Q, K, V = (_t(x[k], torch.bfloat16) for k in "QKV")
    O, S, z = svla.noncausal(Q, K, V, eps=x["eps"], return_state=True)
    torch.cuda.synchronize()
    ref = oracle.forward(x["Q"], x["K"], x["V"], 1, eps=x["eps"])
    _check(x, (_np(O), S.cpu().numpy(), z.cpu().numpy()), ref)


# --- the three kernels one by one ------------------------------------------------

@pytest.mark.parametrize("dtype,d,rope", [("bf16", 32, Rope(8, 12, 12, 5, 7, 3, 1e4)),
                                          ("bf16", 128, None), ("f32", 64, None),
                                          ("bf16", 64, Rope(16, 24, 24, 4, 9, 0, 1e4)),
                                          ("bf16", 32, None), ("bf16", 64, None),
                                          ("bf16", 128, Rope(32, 48, 48, 4, 9, 1, 1e4))])
def test_state_build(svla, dtype, d, rope):
    x = _small(dtype, 1, 2, 3, 211, d)
    dt = _tdt(x)
    S, z = svla.state_build(_t(x["K"], dt), _t(x["V"], dt), x["nb"], rope=rope)
    torch.cuda.synchronize()
    ref = oracle.forward(x["Q"], x["K"], x["V"], x["nb"], rope=rope, want_local=True)
    assert nerr(S.cpu().numpy(), ref["S_local"]) <= 1e-5
    assert nerr(z.cpu().numpy(), ref["z_local"]) <= 1e-6


@pytest.mark.parametrize("nb", [5, 20])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_state_scan(svla, d, nb):
    """nb = 20 takes the segmented scan (chains of 16 blocks or more)."""
    x = _small("bf16", 2, 2, nb, 50, d)
    rng = np.random.default_rng(5)
    g = rng.uniform(0.2, 1.0, (2, 2, nb)).astype(np.float32)
    S0 = rng.standard_normal((2, 2, d, d)).astype(np.float32)
    z0 = np.abs(rng.standard_normal((2, 2, d))).astype(np.float32)
    ref = oracle.forward(x["Q"], x["K"], x["V"], nb, g=g, S0=S0, z0=z0, want_local=True,
                         want_blocks=True)
    Sl = _t(ref["S_local"].astype(np.float32), torch.float32)
    zl = _t(ref["z_local"].astype(np.float32), torch.float32)
    Sp, zp = svla.state_scan(Sl, zl, g=_t(g, torch.float32), S0=_t(S0, torch.float32),
                             z0=_t(z0, torch.float32))
    torch.cuda.synchronize()
    assert nerr(Sp.cpu().numpy(), ref["S_blocks"]) <= 1e-6
    assert nerr(zp.cpu().numpy(), ref["z_blocks"]) <= 1e-6


@pytest.mark.parametrize("dtype,d,rope", [("bf16", 32, None), ("bf16", 32, Rope(8, 12, 12, 5, 7, 0, 1e4)),
                                          ("bf16", 128, None), ("f32", 32, None), ("f32", 128, None),
                                          ("bf16", 64, None)])
def test_apply(svla, dtype, d, rope):
    x = _small(dtype, 1, 3, 2, 299, d)
    ref = oracle.forward(x["Q"], x["K"], x["V"], 2, rope=rope, want_blocks=True)
    dt = _tdt(x)
    O = svla.apply(_t(x["Q"], dt), _t(ref["S_blocks"].astype(np.float32), torch.float32),
                   _t(ref["z_blocks"].astype(np.float32), torch.float32), 2, rope=rope,
                   eps=x["eps"])
    torch.cuda.synchronize()
    assert nerr(_np(O), ref["O"]) <= TOL_O[dtype]


# --- streaming steps ------------------------------------------------------------

CHAIN = [("f32", False, 32, True), ("bf16", True, 32, True), ("bf16", False, 32, True),
         ("bf16", True, 128, True), ("bf16", False, 64, True),
         ("bf16", True, 32, False), ("bf16", True, 64, False), ("bf16", False, 128, False),
         ("f32", True, 128, False)]


@pytest.mark.parametrize("commit", ["in_place", "double_buffer"])
@pytest.mark.parametrize("dtype,gate,d,with_rope", CHAIN)
def test_chained_steps_equal_one_shot(svla, dtype, gate, d, with_rope, commit):
    """nb block steps with the state carried == the one-shot call (and the oracle).
    Committed in place (S_out = S_in: the two-kernel step) or into the other of
    two state buffers (the one-launch step at bf16, d = 32)."""
    gh, gw, frames = 5, 6, 2
    n = frames * gh * gw
    nb = 6
    x = _small(dtype, 1, 3, nb, n, d)
    rope = Rope(8, 12, 12, gh, gw, 0, 1e4) if with_rope else None
    rng = np.random.default_rng(3)
    g = rng.uniform(0.5, 1.0, (1, 3, nb)).astype(np.float32) if gate else None
    dt = _tdt(x)
    Q, K, V = (_t(x[k], dt) for k in "QKV")
    gt = None if g is None else _t(g, torch.float32)
    O1, S1, z1 = svla.block_causal(Q, K, V, nb, g=gt, rope=rope, return_state=True)
    bufs = [(torch.zeros((1, 3, d, d), device=DEV), torch.zeros((1, 3, d), device=DEV))
            for _ in range(2)]
    outs = []
    for s in range(nb):
        sl = slice(s * n, (s + 1) * n)
        gs = None if g is None else gt[:, :, s].contiguous()
        S, z = bufs[s % 2] if commit == "double_buffer" else bufs[0]
        S_next, z_next = bufs[(s + 1) % 2] if commit == "double_buffer" else bufs[0]
        O, S, z = svla.block_step(Q[:, :, sl].contiguous(), K[:, :, sl].contiguous(),
                                  V[:, :, sl].contiguous(), S, z, S_out=S_next, z_out=z_next,
                                  g=gs,
                                  rope=Rope(8, 12, 12, gh, gw, frames * s, 1e4) if with_rope else None)
        outs.append(O)
    Oc = torch.cat(outs, dim=2)
    torch.cuda.synchronize()
    tol_chain = 1e-5 if dtype == "f32" else 1e-2
    assert nerr(_np(Oc), _np(O1)) <= tol_chain
    assert nerr(S.cpu().numpy(), S1.cpu().numpy()) <= 1e-5
    ref = oracle.forward(x["Q"], x["K"], x["V"], nb, g=g, rope=rope)
    _check(x, (_np(Oc), S.cpu().numpy(), z.cpu().numpy()), ref)


@pytest.mark.parametrize("B,H,n,rope,gate", [
    (1, 3, 1, False, False),        # one token
    (1, 3, 15, True, True),         # less than one 16-token group
    (2, 5, 2048, True, False),      # many tiles of few groups
    (1, 70, 2640, False, True),     # the 720p step: four Q groups per wave
    (1, 70, 2640, True, False),     # ... with RoPE
    (1, 200, 3000, False, False),   # 200 heads, three tiles of up to four groups per wave
    (2, 5, 3072, True, False),      # the longest one-launch block
    (1, 2, 3073, True, True),       # one token longer: the two-kernel step
    (1, 70, 1170, True, True),      # the minute-long step's shape
    (3, 100, 333, False, True),     # 300 heads: one workgroup per head
    (1, 7, 512 * 5 + 17, False, False)])
def test_one_launch_step_sizes(svla, B, H, n, rope, gate):
    """The one-launch step (state double-buffered) against the oracle, at the
    edges of its tiling and of its length limit."""
    x = _small("bf16", B, H, 1, n, 32, seed=23)
    rp = Rope(8, 12, 12, 5, 7, 9, 1e4) if rope else None
    rng = np.random.default_rng(24)
    S_in = (rng.standard_normal((B, H, 32, 32)) * 20).astype(np.float32)
    z_in = np.abs(rng.standard_normal((B, H, 32)) * 80).astype(np.float32)
    g = rng.uniform(0.3, 1.0, (B, H)).astype(np.float32) if gate else None
    Q, K, V = (_t(x[k], torch.bfloat16) for k in "QKV")
    O, S, z = svla.block_step(Q, K, V, _t(S_in, torch.float32), _t(z_in, torch.float32),
                              g=None if g is None else _t(g, torch.float32), rope=rp)
    torch.cuda.synchronize()
    ref = oracle.step(x["Q"], x["K"], x["V"], S_in, z_in, g=g, rope=rp, eps=x["eps"])
    _check(x, (_np(O), S.cpu().numpy(), z.cpu().numpy()), ref)


@pytest.mark.parametrize("H,n,d,gate,commit,slots", [
    # the 720p step committed in place: build, then a read-out that sums the
    # block's six split partials and the carried state itself (7 partials)
    (70, 2640, 32, False, "in_place", ["build", "apply"]),
    # the same into a second buffer: one launch, four Q groups per wave
    (70, 2640, 32, True, "double_buffer", ["step"]),
    # the gated d = 128 step: ten 192-token splits, scanned, read out
    (20, 1760, 128, True, "in_place", ["build", "scan", "apply"]),
    (20, 1760, 128, True, "double_buffer", ["build", "scan", "apply"])])
def test_block_step_at_workload_shapes(svla, H, n, d, gate, commit, slots):
    """One block step at the 720p (d = 32) and gated 2.0 (d = 128) block
    shapes, with a carried state, against the oracle; the launch plan is the
    one the shape is meant to take."""
    x = _small("bf16", 1, H, 1, n, d, seed=31)
    rng = np.random.default_rng(32)
    S_in = (rng.standard_normal((1, H, d, d)) * 20).astype(np.float32)
    z_in = np.abs(rng.standard_normal((1, H, d)) * 80).astype(np.float32)
    g = rng.uniform(0.3, 1.0, (1, H)).astype(np.float32) if gate else None
    plan = svla.describe("block_step", torch.bfloat16, 1, H, 1, n, d)
    key = "in_place_kernels" if (commit == "in_place" and plan.get("fused")) else "kernels"
    assert [k["slot"] for k in plan[key]] == slots, plan
    Q, K, V = (_t(x[k], torch.bfloat16) for k in "QKV")
    S, z = _t(S_in, torch.float32), _t(z_in, torch.float32)
    gt = None if g is None else _t(g, torch.float32)
    if commit == "in_place":
        O, S_o, z_o = svla.block_step(Q, K, V, S, z, S_out=S, z_out=z, g=gt)
    else:
        O, S_o, z_o = svla.block_step(Q, K, V, S, z, g=gt)
    torch.cuda.synchronize()
    ref = oracle.step(x["Q"], x["K"], x["V"], S_in, z_in, g=g, eps=x["eps"])
    _check(x, (_np(O), S_o.cpu().numpy(), z_o.cpu().numpy()), ref)


def test_step_without_commit_leaves_state(svla):
    """S_out != S_in: a denoising loop can evaluate a block several times."""
    x = _small("bf16", 1, 2, 1, 300, 32)
    Q, K, V = (_t(x[k], torch.bfloat16) for k in "QKV")
    rng = np.random.default_rng(1)
    S_in = _t(rng.standard_normal((1, 2, 32, 32)).astype(np.float32), torch.float32)
    z_in = _t(np.abs(rng.standard_normal((1, 2, 32))).astype(np.float32) * 10, torch.float32)
    keep = S_in.clone(), z_in.clone()
    O_a, S_a, z_a = svla.block_step(Q, K, V, S_in, z_in)
    O_b, S_b, z_b = svla.block_step(Q, K, V, S_in, z_in)
    torch.cuda.synchronize()
    assert torch.equal(S_in, keep[0]) and torch.equal(z_in, keep[1])
    assert torch.equal(O_a, O_b) and torch.equal(S_a, S_b)
    ref = oracle.step(x["Q"], x["K"], x["V"], keep[0].cpu().numpy(), keep[1].cpu().numpy(),
                      eps=x["eps"])
    _check(x, (_np(O_a), S_a.cpu().numpy(), z_a.cpu().numpy()), ref)


# --- degenerate and edge cases ------------------------------------------------------

def test_zero_queries_and_keys(svla):
    x = _small("bf16", 1, 2, 2, 100, 32)
    Qn = -np.abs(x["Q"])
    Qn[:, :, 1::3] = x["Q"][:, :, 1::3]            # some tokens keep positive features
    dt = torch.bfloat16
    O, S, z = svla.block_causal(_t(Qn, dt), _t(x["K"], dt), _t(x["V"], dt), 2, return_state=True)
    O2 = svla.block_causal(_t(x["Q"], dt), _t(-np.abs(x["K"]), dt), _t(x["V"], dt), 2)
    torch.cuda.synchronize()
    Of = _np(O)
    assert np.all(np.isfinite(Of))
    assert np.all(Of[:, :, 0::3] == 0.0)
    assert torch.count_nonzero(O2).item() == 0
    ref = oracle.forward(Qn, x["K"], x["V"], 2)
    assert nerr(Of, ref["O"]) <= TOL_O["bf16"]


def test_empty_inputs(svla):
    e = torch.empty((0, 3, 64, 32), dtype=torch.bfloat16, device=DEV)
    O = svla.block_causal(e, e, e, 2)
    assert O.shape == e.shape
    e2 = torch.empty((1, 2, 0, 32), dtype=torch.bfloat16, device=DEV)
    S_in = torch.randn((1, 2, 32, 32), device=DEV)
    z_in = torch.rand((1, 2, 32), device=DEV)
    g = torch.full((1, 2), 0.5, device=DEV)
    O, S, z = svla.block_step(e2, e2, e2, S_in, z_in, g=g)
    torch.cuda.synchronize()
    assert torch.allclose(S, 0.5 * S_in) and torch.allclose(z, 0.5 * z_in)


@pytest.mark.parametrize("name", ["c3", "c5"])
def test_repeatable_bit_for_bit(svla, name):
    """Fixed reduction order: runs give identical bits (a race shows up here).
    At full size, so the LDS rings run with every CU loaded."""
    x = make_inputs(CONFIGS[name])
    Q, K, V = (_t(x[k], torch.bfloat16) for k in "QKV")
    g = None if x["g"] is None else torch.from_numpy(x["g"]).to(DEV)
    runs = [svla.block_causal(Q, K, V, x["nb"], g=g, return_state=True) for _ in range(3)]
    torch.cuda.synchronize()
    for r in runs[1:]:
        assert all(torch.equal(p, q) for p, q in zip(runs[0], r))


# --- full-size workloads, every head -------------------------------------------------

def _all_heads_errors(x, cfg, got, group=14):
    """Normwise errors of (O, S, z) against the oracle over every head, with
    the oracle run on groups of `group` heads (its fp64 copies of a whole
    minute-long workload would take about 7 GB of host memory)."""
    O, S, z = got
    worst = [0.0, 0.0, 0.0]
    for h0 in range(0, cfg.H, group):
        hs = slice(h0, min(h0 + group, cfg.H))
        sub = lambda a: None if a is None else np.ascontiguousarray(a[:, hs])
        ref = oracle.forward(sub(x["Q"]), sub(x["K"]), sub(x["V"]), x["nb"], g=sub(x["g"]),
                             rope=cfg.rope, eps=x["eps"])
        errs = (nerr(O[:, hs], ref["O"]), nerr(S[:, hs], ref["S"]), nerr(z[:, hs], ref["z"]))
        worst = [max(a, b) for a, b in zip(worst, errs)]
        del ref
    return worst


def _assert_tol(x, errs):
    eo, es, ez = errs
    assert eo <= TOL_O[x["dtype"]] and es <= TOL_S and ez <= TOL_S, (eo, es, ez)


@pytest.mark.parametrize("name", ["c2", "c3", "c5"])
def test_full_size_one_shot(svla, name):
    cfg = CONFIGS[name]
    x = make_inputs(cfg)
    got = _run_gpu(svla, x, g=x["g"])
    errs = _all_heads_errors(x, cfg, got)
    print("%s all %d heads: O %.2e S %.2e z %.2e" % (name, cfg.H, *errs))
    _assert_tol(x, errs)


def test_full_size_c4_streaming_and_one_shot(svla):
    """Minute-long 480p: 80 block steps with RoPE (t0 = 3 frames per step), the
    state double-buffered (the one-launch step) and committed in place (the
    two-kernel step); device memory in use is the same after step 1 and step 80;
    the streams equal each other and the one-shot call over the same 80 blocks;
    the double-buffered stream and the one-shot call against the oracle on
    every head."""
    cfg = CONFIGS["c4"]
    x = make_inputs(cfg)
    n, nb = cfg.n, cfg.nb
    frames = n // (cfg.rope.grid_h * cfg.rope.grid_w)
    Q, K, V = (_t(x[k], torch.bfloat16) for k in "QKV")
    steps = [tuple(t[:, :, s * n:(s + 1) * n].contiguous() for t in (Q, K, V)) for s in range(nb)]
    ws = torch.empty(svla.workspace_size("block_step", torch.bfloat16, 1, cfg.H, 1, n, 32),
                     dtype=torch.uint8, device=DEV)

    def stream_pass(nbuf):
        """80 steps; the state committed in place (nbuf = 1: the two-kernel
        step) or into the other of two buffers (nbuf = 2: the one-launch step)."""
        bufs = [(torch.zeros((1, cfg.H, 32, 32), device=DEV), torch.zeros((1, cfg.H, 32), device=DEV))
                for _ in range(nbuf)]
        outs = [torch.empty_like(steps[0][0]) for _ in range(nb)]
        torch.cuda.synchronize()
        mem = []
        for s in range(nb):
            S, z = bufs[s % nbuf]
            S_next, z_next = bufs[(s + 1) % nbuf]
            svla.block_step(*steps[s], S, z, S_out=S_next, z_out=z_next,
                            rope=cfg.rope.with_t0(frames * s), out=outs[s], workspace=ws)
            if s in (0, nb - 1):
                torch.cuda.synchronize()
                mem.append(torch.cuda.memory_allocated())
        assert mem[0] == mem[1]
        S, z = bufs[nb % nbuf]
        return torch.cat(outs, dim=2), S, z

    Oc, S, z = stream_pass(2)
    Oi, Si, zi = stream_pass(1)
    torch.cuda.synchronize()
    assert nerr(_np(Oi), _np(Oc)) <= 1e-2
    assert nerr(Si.cpu().numpy(), S.cpu().numpy()) <= 1e-5
    del Oi, steps
    O1, S1, z1 = svla.block_causal(Q, K, V, nb, rope=cfg.rope, return_state=True)
    torch.cuda.synchronize()
    assert nerr(_np(Oc), _np(O1)) <= 1e-2
    assert nerr(S.cpu().numpy(), S1.cpu().numpy()) <= 1e-5
    stream = (_np(Oc), S.cpu().numpy(), z.cpu().numpy())
    del Oc
    one = (_np(O1), S1.cpu().numpy(), z1.cpu().numpy())
    del O1
    e_stream = _all_heads_errors(x, cfg, stream)
    e_one = _all_heads_errors(x, cfg, one)
    print("c4 all %d heads, 80 steps: O %.2e S %.2e z %.2e; one shot: O %.2e S %.2e z %.2e"
          % (cfg.H, *e_stream, *e_one))
    _assert_tol(x, e_stream)
    _assert_tol(x, e_one)


@pytest.mark.parametrize("dtype,d", [("bf16", 32), ("bf16", 64), ("bf16", 128), ("f32", 128)])
def test_largest_slice(svla, dtype, d):
    """The largest call the size check admits: two blocks of 2^k - 1 tokens per
    (b,h), so one slice is two rows short of 2 GiB and the second head's
    slice starts 2 GiB into each tensor.  The inputs are sparse: zero rows of K
    and V add nothing to the state and a zero query gives a zero output, so the
    rows that are set (at both ends of every block, the slice's last token
    among them, and random rows between) form a small dense problem with the
    same block structure, which the oracle solves."""
    B, H, nb = 1, 2, 2
    es = 2 if dtype == "bf16" else 4
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    n = (1 << 31) // (nb * d * es) - 1
    N = nb * n
    assert nb * n * d * es < (1 << 31) <= nb * (n + 1) * d * es
    rng = np.random.default_rng(29)
    rows = []
    for b in range(nb):
        inner = rng.choice(np.arange(b * n + 1, (b + 1) * n - 1), size=62, replace=False)
        rows.append(np.sort(np.concatenate([[b * n], inner, [(b + 1) * n - 1]])))
    m = max(len(r) for r in rows)
    vals = {k: torch.from_numpy(rng.standard_normal((B, H, nb * m, d)).astype(np.float32)).to(tdt)
            for k in "QKV"}
    g = rng.uniform(0.5, 1.0, (B, H, nb)).astype(np.float32)

    big = {k: torch.zeros((B, H, N, d), dtype=tdt, device=DEV) for k in "QKV"}
    for b in range(nb):
        idx = torch.from_numpy(rows[b]).to(DEV)
        for k in "QKV":
            big[k][:, :, idx] = vals[k][:, :, b * m:b * m + len(rows[b])].to(DEV)
    O, S, z = svla.block_causal(big["Q"], big["K"], big["V"], nb, g=_t(g, torch.float32),
                                return_state=True)
    torch.cuda.synchronize()
    del big

    ref = oracle.forward(vals["Q"].float().numpy(), vals["K"].float().numpy(),
                         vals["V"].float().numpy(), nb, g=g)
    got = np.concatenate([_np(O[:, :, torch.from_numpy(rows[b]).to(DEV)]) for b in range(nb)], axis=2)
    want = np.concatenate([ref["O"][:, :, b * m:b * m + len(rows[b])] for b in range(nb)], axis=2)
    eo = nerr(got, want)
    es_, ez = nerr(S.cpu().numpy(), ref["S"]), nerr(z.cpu().numpy(), ref["z"])
    assert eo <= TOL_O[dtype] and es_ <= TOL_S and ez <= TOL_S, (eo, es_, ez)
    # rows whose query is zero, sampled across the slice (the last rows included)
    zero = np.setdiff1d(np.concatenate([rng.integers(0, N, 4000), np.arange(N - 200, N)]),
                        np.concatenate(rows))
    assert torch.count_nonzero(O[:, :, torch.from_numpy(zero).to(DEV)]).item() == 0
    print("largest slice %s d=%d: O %.2e S %.2e z %.2e" % (dtype, d, eo, es_, ez))


@pytest.mark.parametrize("d,with_rope,gate,commit", [(32, True, False, "in_place"),
                                                     (64, False, True, "in_place"),
                                                     (32, True, True, "double_buffer"),
                                                     (32, False, False, "double_buffer")])
def test_graph_replay_matches_eager(svla, d, with_rope, gate, commit):
    """A pass of block steps captured in a HIP graph, as a streaming caller
    replays it: every replay, with eager work and a synchronization between
    replays, gives the eager pass's outputs and final state bit for bit."""
    gh, gw, frames, nb, H = 5, 6, 2, 5, 3
    n = frames * gh * gw
    x = _small("bf16", 1, H, nb, n, d, seed=13)
    Q, K, V = (_t(x[k], torch.bfloat16) for k in "QKV")
    steps = [tuple(t[:, :, s * n:(s + 1) * n].contiguous() for t in (Q, K, V)) for s in range(nb)]
    rng = np.random.default_rng(17)
    gs = ([_t(rng.uniform(0.5, 1.0, (1, H)).astype(np.float32), torch.float32) for _ in range(nb)]
          if gate else [None] * nb)
    ropes = [Rope(8, 12, 12, gh, gw, frames * s, 1e4) if with_rope else None for s in range(nb)]
    bufs = [(torch.zeros((1, H, d, d), device=DEV), torch.zeros((1, H, d), device=DEV))
            for _ in range(2)]
    nbuf = 2 if commit == "double_buffer" else 1
    outs = [torch.empty_like(steps[0][0]) for _ in range(nb)]
    ws = torch.empty(svla.workspace_size("block_step", torch.bfloat16, 1, H, 1, n, d),
                     dtype=torch.uint8, device=DEV)

    def run_pass():
        for s in range(nb):
            S, z = bufs[s % nbuf]
            S_next, z_next = bufs[(s + 1) % nbuf]
            svla.block_step(*steps[s], S if s else None, z if s else None, S_out=S_next,
                            z_out=z_next, g=gs[s], rope=ropes[s], out=outs[s], workspace=ws)

    S, z = bufs[nb % nbuf]          # the final state
    run_pass()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs] + [S.clone(), z.clone()]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_pass()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_pass()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        for S_, z_ in bufs:
            S_.fill_(float("nan"))
            z_.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = outs + [S, z]
        assert all(torch.equal(a, b) for a, b in zip(got, want)), "replay %d differs" % rep


def test_side_stream_matches_default_stream(svla):
    """Every call launches on the caller's current stream: the same calls on a
    side stream, with inputs produced on that stream, give the same bits."""
    x = _small("bf16", 1, 4, 3, 330, 32, seed=19)
    rope = Rope(8, 12, 12, 5, 6, 0, 1e4)
    Q, K, V = (_t(x[k], torch.bfloat16) for k in "QKV")
    ref = svla.block_causal(Q, K, V, 3, rope=rope, return_state=True)
    S0 = torch.randn((1, 4, 32, 32), device=DEV)
    z0 = torch.rand((1, 4, 32), device=DEV) * 10
    ref_step = svla.block_step(Q[:, :, :330].contiguous(), K[:, :, :330].contiguous(),
                               V[:, :, :330].contiguous(), S0, z0, rope=rope)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        Q2, K2, V2 = (t * 1 for t in (Q, K, V))      # produced on the side stream
        got = svla.block_causal(Q2, K2, V2, 3, rope=rope, return_state=True)
        got_step = svla.block_step(Q2[:, :, :330].contiguous(), K2[:, :, :330].contiguous(),
                                   V2[:, :, :330].contiguous(), S0, z0, rope=rope)
    side.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(got, ref))
    assert all(torch.equal(a, b) for a, b in zip(got_step, ref_step))
