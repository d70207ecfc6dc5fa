"""The no-alloc block step (svla_block_step_noalloc, through the C ABI)
against the workspace entry point on the same inputs: bit for bit, on two
calls in a row, the second smaller than the first."""
import ctypes

import numpy as np
import pytest
import torch

from workloads import CONFIGS, Rope, make_inputs, scaled_config

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def svla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_causal_linear_relu_amd as m
    m.library()
    return m


def _case(B, H, n, d, seed):
    x = make_inputs(scaled_config(CONFIGS["c3"], d=d, seed=seed), B=B, H=H, nb=1, n=n)
    Q, K, V = (torch.from_numpy(x[k]).to(DEV).to(torch.bfloat16) for k in "QKV")
    rng = np.random.default_rng(seed)
    S = torch.from_numpy((rng.standard_normal((B, H, d, d)) * 10).astype(np.float32)).to(DEV)
    z = torch.from_numpy(np.abs(rng.standard_normal((B, H, d)) * 50).astype(np.float32)).to(DEV)
    g = torch.from_numpy(rng.uniform(0.3, 1.0, (B, H)).astype(np.float32)).to(DEV)
    return Q, K, V, S, z, g


def _noalloc(svla, Q, K, V, S_in, z_in, S_out, z_out, O, g, rope):
    lib = svla.library()
    B, H, n, d = Q.shape
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    rs = svla.rope_struct(rope)
    st = lib.svla_block_step_noalloc(svla._DT[Q.dtype], B, H, n, d, p(Q), p(K), p(V), p(O),
                                     p(S_in), p(z_in), p(S_out), p(z_out), p(g),
                                     ctypes.byref(rs) if rs is not None else None, 1e-6,
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.svla_last_error()


CASES = [
    # B, H, n, d, gated, rope, commit in place (the two-kernel step, which uses the scratch)
    (1, 70, 1170, 32, False, Rope(8, 12, 12, 15, 26, 30, 1e4), True),
    (1, 3, 300, 128, True, None, True),
]


def test_noalloc_matches_workspace_entry_point(svla):
    """Two no-alloc calls in a row (the minute-long step shape, then a smaller
    gated d = 128 step), each against svla_block_step / svla_block_step_gated
    with a workspace; then a double-buffered step (the one-launch path)."""
    for i, (B, H, n, d, gated, rope, in_place) in enumerate(CASES):
        Q, K, V, S, z, g = _case(B, H, n, d, seed=40 + i)
        gg = g if gated else None
        # the workspace entry point, committing in place
        S_ref, z_ref = S.clone(), z.clone()
        O_ref = torch.empty_like(Q)
        svla.block_step(Q, K, V, S_ref, z_ref, S_out=S_ref, z_out=z_ref, g=gg, rope=rope, out=O_ref)
        # the no-alloc entry point, the same
        S_na, z_na = S.clone(), z.clone()
        O_na = torch.full_like(Q, float("nan"))
        _noalloc(svla, Q, K, V, S_na, z_na, S_na, z_na, O_na, gg, rope)
        torch.cuda.synchronize()
        assert torch.equal(O_na, O_ref), "call %d: O differs" % i
        assert torch.equal(S_na, S_ref) and torch.equal(z_na, z_ref), "call %d: state differs" % i
    # a double-buffered step through the no-alloc entry point (no scratch used)
    Q, K, V, S, z, g = _case(1, 5, 500, 32, seed=50)
    O_ref, S_ref, z_ref = svla.block_step(Q, K, V, S, z, g=g)
    S2, z2, O2 = torch.empty_like(S), torch.empty_like(z), torch.empty_like(Q)
    svla.block_step_noalloc(Q, K, V, S, z, S2, z2, O2, g=g)
    torch.cuda.synchronize()
    assert torch.equal(O2, O_ref) and torch.equal(S2, S_ref) and torch.equal(z2, z_ref)
