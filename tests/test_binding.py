"""Python binding, CPU only: every state, gate and output tensor is checked
against the shape its entry point implies before anything reaches the library
(which reads them through raw pointers, without range checks of its own)."""
import pytest
import torch

import block_causal_linear_relu_amd as svla

B, H, N, d, nb = 1, 3, 40, 32, 4


def qkv(n=N):
    return [torch.zeros((B, H, n, d), dtype=torch.bfloat16) for _ in range(3)]


def _raises(match, fn, *args, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*args, **kw)


@pytest.mark.parametrize("kw,name", [
    (dict(g=torch.zeros(B, H)), "g"),                               # a step's gate, not [B,H,nb]
    (dict(g=torch.zeros(B, H, nb + 1)), "g"),
    (dict(S0=torch.zeros(B, H, d, d + 1), z0=torch.zeros(B, H, d)), "S0"),
    (dict(S0=torch.zeros(B, H, d, d), z0=torch.zeros(B, H, d, 1)), "z0"),
    (dict(S0=torch.zeros(B, H, d, d)), "S0 and z0"),
    (dict(out=torch.zeros(B, H, N + 1, d, dtype=torch.bfloat16)), "out"),
])
def test_block_causal_shapes(kw, name):
    _raises(name, svla.block_causal, *qkv(), nb, **kw)


@pytest.mark.parametrize("kw,name", [
    (dict(g=torch.zeros(B, H, 1)), "g"),                            # a one-shot gate, not [B,H]
    (dict(S_in=torch.zeros(B, H + 1, d, d), z_in=torch.zeros(B, H, d)), "S_in"),
    (dict(S_in=torch.zeros(B, H, d, d), z_in=torch.zeros(B, H)), "z_in"),
    (dict(S_out=torch.zeros(B, H, d * d)), "S_out"),
    (dict(z_out=torch.zeros(B, H, d + 4)), "z_out"),
    (dict(z_in=torch.zeros(B, H, d)), "S_in and z_in"),
    (dict(out=torch.zeros(B, H, N, d // 2, dtype=torch.bfloat16)), "out"),
])
def test_block_step_shapes(kw, name):
    _raises(name, svla.block_step, *qkv(), **kw)


def test_qkv_must_agree():
    Q, K, V = qkv()
    _raises("shape", svla.block_causal, Q, K[:, :, :-1], V, nb)
    _raises("shape", svla.noncausal, Q[0], K[0], V[0])
    _raises("multiple", svla.block_causal, Q, K, V, 3)
    _raises("out", svla.noncausal, Q, K, V, out=torch.zeros(1))


def test_kernel_entry_points_shapes():
    Sl = torch.zeros(B, H, nb, d, d)
    zl = torch.zeros(B, H, nb, d)
    _raises("z_local", svla.state_scan, Sl, zl[:, :, :-1])
    _raises("g", svla.state_scan, Sl, zl, g=torch.zeros(B, H))
    _raises("S0", svla.state_scan, Sl, zl, S0=torch.zeros(B, H, nb, d, d), z0=torch.zeros(B, H, d))
    _raises("S0 and z0", svla.state_scan, Sl, zl, z0=torch.zeros(B, H, d))
    _raises("S_local", svla.state_scan, torch.zeros(B, H, nb, d), zl)
    Q = qkv()[0]
    _raises("S_prefix", svla.apply, Q, Sl[:, :, :-1], zl, nb)
    _raises("z_prefix", svla.apply, Q, Sl, zl[..., :-1], nb)
    K, V = qkv()[:2]
    _raises("shape", svla.state_build, K, V[:, :1], nb)


def test_right_shapes_reach_the_device_check():
    """With every shape right, the first complaint is that the tensors are not
    on the GPU: shape checks come first and pass."""
    Q, K, V = qkv()
    with pytest.raises(ValueError, match="GPU"):
        svla.block_causal(Q, K, V, nb, g=torch.zeros(B, H, nb),
                          S0=torch.zeros(B, H, d, d), z0=torch.zeros(B, H, d))
    with pytest.raises(ValueError, match="GPU"):
        svla.block_step(Q, K, V, torch.zeros(B, H, d, d), torch.zeros(B, H, d),
                        g=torch.zeros(B, H))


@pytest.mark.parametrize("kw,name", [
    (dict(dO=torch.zeros(B, H, N + 1, d, dtype=torch.bfloat16)), "dO"),
    (dict(g=torch.zeros(B, H)), "g"),
    (dict(S0=torch.zeros(B, H, d, d), z0=torch.zeros(B, H)), "z0"),
    (dict(z0=torch.zeros(B, H, d)), "S0 and z0"),
])
def test_backward_shapes(kw, name):
    args = dict(dO=torch.zeros(B, H, N, d, dtype=torch.bfloat16))
    args.update(kw)
    dO = args.pop("dO")
    _raises(name, svla.block_causal_backward, *qkv(), dO, nb, **args)


def test_backward_block_count():
    _raises("multiple", svla.block_causal_backward, *qkv(), qkv()[0], 3)


def test_softmax_attention_shapes():
    Q = torch.zeros(B, H, N, 64, dtype=torch.bfloat16)
    K = torch.zeros(B, H, N + 8, 64, dtype=torch.bfloat16)
    _raises("multiple", svla.softmax_attention, Q, K, K, 3)
    _raises("smaller", svla.softmax_attention, Q, K[:, :, :N - 4], K[:, :, :N - 4], 4)
    _raises("one", svla.softmax_attention, Q, K, K[:, :, :N], 4)
    _raises("out", svla.softmax_attention, Q, K, K, 4, out=torch.zeros(B, H, N, 32))
