"""Pins of the backward oracle (CPU only): directional derivatives of the
loss L = sum(dO * O) by central differences of the forward oracle (the fp64
C implementation, which shares no code with oracle.backward), for every
gradient, with and without gate, RoPE and a carried state; and the linearity
of the gradients in dO."""
import numpy as np
import pytest

import oracle
from oracle.backward import backward
from workloads import Rope


def _inputs(seed, B=1, H=2, nb=3, n=5, d=8):
    rng = np.random.default_rng(seed)
    # magnitudes kept away from the ReLU's kink, where a difference quotient
    # would straddle it
    def away(shape):
        x = rng.standard_normal(shape)
        return np.sign(x) * (np.abs(x) + 0.05)
    Q, K = away((B, H, nb * n, d)), away((B, H, nb * n, d))
    V = rng.standard_normal((B, H, nb * n, d))
    dO = rng.standard_normal((B, H, nb * n, d))
    g = rng.uniform(0.3, 0.95, (B, H, nb))
    S0 = rng.standard_normal((B, H, d, d))
    z0 = np.abs(rng.standard_normal((B, H, d))) + 0.5
    return Q, K, V, dO, g, S0, z0


def _loss(Q, K, V, nb, dO, **kw):
    return float(np.sum(dO * oracle.forward(Q, K, V, nb, **kw)["O"]))


VARIANTS = {
    "plain": dict(),
    "gate": dict(gate=True),
    "rope": dict(rope=Rope(2, 2, 4, 2, 3, 1, 10000.0)),
    "gate_rope_state": dict(gate=True, state=True, rope=Rope(2, 2, 4, 2, 3, 5, 10000.0)),
}


@pytest.mark.parametrize("name", list(VARIANTS))
def test_directional_derivatives(name):
    v = VARIANTS[name]
    Q, K, V, dO, g, S0, z0 = _inputs(1)
    nb = 3
    kw = dict(eps=1e-3, rope=v.get("rope"), g=g if v.get("gate") else None,
              S0=S0 if v.get("state") else None, z0=z0 if v.get("state") else None)
    grads = backward(Q, K, V, nb, dO, **kw)
    rng = np.random.default_rng(2)
    h = 1e-5
    args = {"Q": Q, "K": K, "V": V}
    for key, gname in (("Q", "dQ"), ("K", "dK"), ("V", "dV")):
        for _ in range(3):
            D = rng.standard_normal(args[key].shape)
            plus = dict(args); plus[key] = args[key] + h * D
            minus = dict(args); minus[key] = args[key] - h * D
            fd = (_loss(plus["Q"], plus["K"], plus["V"], nb, dO, **kw) -
                  _loss(minus["Q"], minus["K"], minus["V"], nb, dO, **kw)) / (2 * h)
            an = float(np.sum(grads[gname] * D))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, key, fd, an)
    if kw["g"] is not None:
        D = rng.standard_normal(g.shape)
        fd = (_loss(Q, K, V, nb, dO, **dict(kw, g=g + h * D)) -
              _loss(Q, K, V, nb, dO, **dict(kw, g=g - h * D))) / (2 * h)
        assert abs(fd - float(np.sum(grads["dg"] * D))) <= 1e-6 * max(1.0, abs(fd))
    if kw["S0"] is not None:
        D = rng.standard_normal(S0.shape)
        fd = (_loss(Q, K, V, nb, dO, **dict(kw, S0=S0 + h * D)) -
              _loss(Q, K, V, nb, dO, **dict(kw, S0=S0 - h * D))) / (2 * h)
        assert abs(fd - float(np.sum(grads["dS0"] * D))) <= 1e-6 * max(1.0, abs(fd))
        D = rng.standard_normal(z0.shape)
        fd = (_loss(Q, K, V, nb, dO, **dict(kw, z0=z0 + h * D)) -
              _loss(Q, K, V, nb, dO, **dict(kw, z0=z0 - h * D))) / (2 * h)
        assert abs(fd - float(np.sum(grads["dz0"] * D))) <= 1e-6 * max(1.0, abs(fd))


def test_single_entries_by_difference():
    """A few individual entries of dQ, dK, dV against one-coordinate differences."""
    Q, K, V, dO, g, _, _ = _inputs(3, H=1, nb=2, n=4, d=4)
    kw = dict(eps=1e-3, g=g)
    grads = backward(Q, K, V, 2, dO, **kw)
    h = 1e-6
    for key, gname, idx in (("Q", "dQ", (0, 0, 1, 2)), ("K", "dK", (0, 0, 5, 0)),
                            ("V", "dV", (0, 0, 0, 3)), ("K", "dK", (0, 0, 0, 1))):
        args = {"Q": Q, "K": K, "V": V}
        p, m = {k: a.copy() for k, a in args.items()}, {k: a.copy() for k, a in args.items()}
        p[key][idx] += h
        m[key][idx] -= h
        fd = (_loss(p["Q"], p["K"], p["V"], 2, dO, **kw) - _loss(m["Q"], m["K"], m["V"], 2, dO, **kw)) / (2 * h)
        assert abs(fd - grads[gname][idx]) <= 1e-6 * max(1.0, abs(fd)), (key, idx, fd, grads[gname][idx])


def test_linear_in_dO_and_causal():
    """The gradients are linear in dO; and causality backwards: a dO confined
    to block 0 gives no gradient to the queries, keys or values of blocks 1
    and 2 (their tokens never reach block 0's outputs)."""
    Q, K, V, dO, g, _, _ = _inputs(4)
    a = backward(Q, K, V, 3, dO, g=g)
    b = backward(Q, K, V, 3, 2.5 * dO, g=g)
    for k in ("dQ", "dK", "dV", "dg"):
        np.testing.assert_allclose(b[k], 2.5 * a[k], rtol=1e-12, atol=1e-12)
    d0 = np.zeros_like(dO)
    d0[:, :, :5] = dO[:, :, :5]
    c = backward(Q, K, V, 3, d0, g=g)
    assert np.all(c["dK"][:, :, 5:] == 0) and np.all(c["dV"][:, :, 5:] == 0)
    assert np.all(c["dQ"][:, :, 5:] == 0)
