"""Pins of the CPU oracle against things other than itself (CPU only).

Each test ties the fp64 oracle to something it cannot share a mistake with:
hand-worked examples, exact rational arithmetic, the quadratic brute force,
textbook special cases computed with plain matrix products or cumulative
sums, closed forms and invariants of the method.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import brute_force, normwise_error
from workloads import CONFIGS, Rope, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _tiny(seed, B=1, H=2, N=64, d=32, dtype=np.float64):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, N, d)).astype(dtype) for _ in range(3)]


# --- hand-worked examples ---------------------------------------------------

@pytest.mark.parametrize("ex", json.load(open(GOLDEN))["examples"], ids=lambda e: e["name"])
def test_hand_examples(ex):
    shape = (1, 1, ex["nb"] * ex["n"], ex["d"])
    Q = np.array(ex["Q"], dtype=np.float64).reshape(shape)
    K = np.array(ex["K"], dtype=np.float64).reshape(shape)
    V = np.array(ex["V"], dtype=np.float64).reshape(shape)
    g = None if ex["g"] is None else np.array(ex["g"]).reshape(1, 1, ex["nb"])
    out = oracle.forward(Q, K, V, ex["nb"], g=g, eps=ex["eps"])
    np.testing.assert_allclose(out["O"].reshape(-1, ex["d"]), np.array(ex["O"]),
                               rtol=1e-15, atol=1e-6 * ex["eps"] + 1e-15)


# --- exact rational arithmetic ---------------------------------------------

def _exact_brute(Qi, Ki, Vi, nb, g, eps):
    """Quadratic form in exact Fractions, pure Python (tiny sizes only)."""
    N, d = len(Qi), len(Qi[0])
    n = N // nb
    relu = lambda x: x if x > 0 else Fraction(0)
    out = []
    for i in range(N):
        ci = i // n
        num = [Fraction(0)] * d
        den = Fraction(eps)
        p = [relu(x) for x in Qi[i]]
        for j in range(N):
            cj = j // n
            if cj > ci:
                continue
            w = Fraction(1)
            for c in range(cj + 1, ci + 1):
                w *= g[c]
            a = [relu(x) for x in Ki[j]]
            s = sum(pk * ak for pk, ak in zip(p, a)) * w
            den += s
            for v in range(d):
                num[v] += s * Vi[j][v]
        out.append([x / den if den != 0 else Fraction(0) for x in num])
    return out


@pytest.mark.parametrize("gated", [False, True])
def test_exact_rational(gated):
    rng = np.random.default_rng(11)
    nb, n, d = 3, 2, 3
    N = nb * n
    Qi = rng.integers(-3, 4, size=(N, d))
    Ki = rng.integers(-3, 4, size=(N, d))
    Vi = rng.integers(-5, 6, size=(N, d))
    g = [Fraction(1, 2), Fraction(3, 4), Fraction(1, 8)] if gated else [Fraction(1)] * nb
    eps = Fraction(1, 1000)
    F = lambda m: [[Fraction(int(x)) for x in row] for row in m]
    exact = _exact_brute(F(Qi), F(Ki), F(Vi), nb, g, eps)
    shape = (1, 1, N, d)
    gg = np.array([float(x) for x in g]).reshape(1, 1, nb) if gated else None
    out = oracle.forward(Qi.reshape(shape), Ki.reshape(shape), Vi.reshape(shape), nb,
                         g=gg, eps=float(eps))["O"].reshape(N, d)
    ref = np.array([[float(x) for x in row] for row in exact])
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)


# --- quadratic brute force ---------------------------------------------------

def _c1_inputs():
    return make_inputs(CONFIGS["c1"])


def test_c1_vs_brute_force():
    x = _c1_inputs()
    out = oracle.forward(x["Q"], x["K"], x["V"], x["nb"], eps=x["eps"])
    ref = brute_force(x["Q"], x["K"], x["V"], x["nb"], eps=x["eps"])
    assert normwise_error(out["O"], ref) < 1e-12


C1_ROPE = Rope(8, 12, 12, 16, 16, 0, 10000.0)   # one 16x16 frame per 256-token block


@pytest.mark.parametrize("variant", ["rope", "gate", "rope_gate", "state_in"])
def test_c1_variants_vs_brute_force(variant):
    x = _c1_inputs()
    B, H, nb, d = x["B"], x["H"], x["nb"], x["d"]
    rng = np.random.default_rng(101)
    rope = C1_ROPE if "rope" in variant else None
    g = None
    if "gate" in variant:
        g = 1.0 / (1.0 + np.exp(-(rng.standard_normal((B, H, nb)) + 2.0)))
    S0 = z0 = None
    if variant == "state_in":
        S0 = rng.standard_normal((B, H, d, d)) * 10
        z0 = np.abs(rng.standard_normal((B, H, d))) * 50
        g = rng.uniform(0.2, 1.0, (B, H, nb))
    out = oracle.forward(x["Q"], x["K"], x["V"], nb, g=g, rope=rope, S0=S0, z0=z0, eps=x["eps"])
    ref = brute_force(x["Q"], x["K"], x["V"], nb, g=g, rope=rope, S0=S0, z0=z0, eps=x["eps"])
    assert normwise_error(out["O"], ref) < 1e-12


# --- special cases that reduce to textbook forms ------------------------------

def test_one_block_is_plain_linear_attention():
    """nb = 1: O = phi(Q) (phi(K)^T V) / (phi(Q) phi(K)^T 1 + eps), by matmul."""
    Q, K, V = _tiny(3, N=96)
    eps = 1e-6
    out = oracle.forward(Q, K, V, 1, eps=eps)
    P, A = np.maximum(Q, 0), np.maximum(K, 0)
    S = np.matmul(np.swapaxes(A, -1, -2), V)
    z = A.sum(axis=2)
    ref = np.matmul(P, S) / (np.einsum("bhnd,bhd->bhn", P, z)[..., None] + eps)
    assert normwise_error(out["O"], ref) < 1e-12
    assert normwise_error(out["S"], S) < 1e-13
    assert normwise_error(out["z"], z) < 1e-13


def test_one_token_blocks_are_token_causal():
    """n = 1: classic causal linear attention, by cumulative sums."""
    Q, K, V = _tiny(4, N=50)
    eps = 1e-6
    out = oracle.forward(Q, K, V, 50, eps=eps)
    P, A = np.maximum(Q, 0), np.maximum(K, 0)
    Scum = np.cumsum(A[..., :, None] * V[..., None, :], axis=2)     # [B,H,N,d,d]
    zcum = np.cumsum(A, axis=2)
    num = np.einsum("bhnk,bhnkv->bhnv", P, Scum)
    den = np.einsum("bhnk,bhnk->bhn", P, zcum) + eps
    assert normwise_error(out["O"], num / den[..., None]) < 1e-12


# --- invariants ----------------------------------------------------------------

def test_chained_steps_equal_one_shot_and_brute_force():
    """80 steps of 8 tokens, d=32, state carried: equals one-shot and brute force,
    with a carried state of exactly d*d + d numbers per head."""
    Q, K, V = _tiny(5, B=1, H=2, N=640)
    nb, n, d = 80, 8, 32
    one = oracle.forward(Q, K, V, nb)
    S = np.zeros((1, 2, d, d)); z = np.zeros((1, 2, d))
    outs = []
    for s in range(nb):
        sl = slice(s * n, (s + 1) * n)
        r = oracle.step(Q[:, :, sl], K[:, :, sl], V[:, :, sl], S, z)
        assert r["S"].shape == (1, 2, d, d) and r["z"].shape == (1, 2, d)
        S, z = r["S"], r["z"]
        outs.append(r["O"])
    chained = np.concatenate(outs, axis=2)
    assert normwise_error(chained, one["O"]) < 1e-12
    assert normwise_error(S, one["S"]) < 1e-12
    ref = brute_force(Q, K, V, nb)
    assert normwise_error(chained, ref) < 1e-11


def test_checkpoint_resume():
    """40 steps, state through a host round trip (bytes), 40 more == 80 steps."""
    Q, K, V = _tiny(6, B=1, H=1, N=80 * 4)
    n = 4
    S = np.zeros((1, 1, 32, 32)); z = np.zeros((1, 1, 32))
    straight = []
    for s in range(80):
        sl = slice(s * n, (s + 1) * n)
        r = oracle.step(Q[:, :, sl], K[:, :, sl], V[:, :, sl], S, z)
        S, z = r["S"], r["z"]
        straight.append(r["O"])
    S2 = np.zeros((1, 1, 32, 32)); z2 = np.zeros((1, 1, 32))
    resumed = []
    for s in range(80):
        if s == 40:
            blob = S2.tobytes() + z2.tobytes()
            S2 = np.frombuffer(blob[:S2.nbytes]).reshape(S2.shape).copy()
            z2 = np.frombuffer(blob[S2.nbytes:]).reshape(z2.shape).copy()
        sl = slice(s * n, (s + 1) * n)
        r = oracle.step(Q[:, :, sl], K[:, :, sl], V[:, :, sl], S2, z2)
        S2, z2 = r["S"], r["z"]
        resumed.append(r["O"])
    assert np.array_equal(np.concatenate(straight, 2), np.concatenate(resumed, 2))
    assert np.array_equal(S, S2) and np.array_equal(z, z2)


def test_gate_one_is_ungated_and_gate_zero_is_per_block():
    Q, K, V = _tiny(7, N=4 * 24)
    nb = 4
    ones = np.ones((1, 2, nb))
    a = oracle.forward(Q, K, V, nb)
    b = oracle.forward(Q, K, V, nb, g=ones)
    assert np.array_equal(a["O"], b["O"]) and np.array_equal(a["S"], b["S"])
    c = oracle.forward(Q, K, V, nb, g=np.zeros((1, 2, nb)))
    for blk in range(nb):
        sl = slice(blk * 24, (blk + 1) * 24)
        ref = oracle.forward(Q[:, :, sl], K[:, :, sl], V[:, :, sl], 1)
        assert normwise_error(c["O"][:, :, sl], ref["O"]) < 1e-13


def test_gate_scan_is_associative():
    """(g1,S1) then (g2,S2) == one combined step (g1*g2, g2*S1 + S2) on the state."""
    Q, K, V = _tiny(8, N=2 * 16)
    rng = np.random.default_rng(9)
    S0 = rng.standard_normal((1, 2, 32, 32)); z0 = np.abs(rng.standard_normal((1, 2, 32)))
    g = rng.uniform(0.1, 0.9, (1, 2, 2))
    full = oracle.forward(Q, K, V, 2, g=g, S0=S0, z0=z0, want_local=True)
    Sl, zl = full["S_local"], full["z_local"]
    g1, g2 = g[..., 0], g[..., 1]
    comb_S = (g1 * g2)[..., None, None] * S0 + g2[..., None, None] * Sl[:, :, 0] + Sl[:, :, 1]
    comb_z = (g1 * g2)[..., None] * z0 + g2[..., None] * zl[:, :, 0] + zl[:, :, 1]
    assert normwise_error(full["S"], comb_S) < 1e-13
    assert normwise_error(full["z"], comb_z) < 1e-13


def test_closed_forms():
    Q, K, V = _tiny(10, N=3 * 20)
    nb, eps = 3, 1e-6
    # constant V: O_i = c * (p.z) / (p.z + eps)
    c = np.linspace(-2, 2, 32)
    Vc = np.broadcast_to(c, V.shape).copy()
    out = oracle.forward(Q, K, Vc, nb, eps=eps, want_den=True)
    den = out["den"]
    ref = c[None, None, None, :] * ((den - eps) / den)[..., None]
    assert normwise_error(out["O"], ref) < 1e-13
    # K <= 0 everywhere: nothing enters the state, O = 0, no NaN
    out = oracle.forward(Q, -np.abs(K), V, nb, eps=eps)
    assert np.all(out["O"] == 0.0) and np.all(out["S"] == 0.0)
    # phi(q) = 0: O = 0 exactly
    out = oracle.forward(-np.abs(Q), K, V, nb, eps=eps)
    assert np.all(out["O"] == 0.0)


def test_positive_homogeneity_in_k():
    Q, K, V = _tiny(12, N=2 * 32)
    a = oracle.forward(Q, K, V, 2, eps=0.0)
    b = oracle.forward(Q, 3.5 * K, V, 2, eps=0.0)
    assert normwise_error(b["O"], a["O"]) < 1e-13


# --- RoPE ---------------------------------------------------------------------

def _one_hot_case(rope, f_q, f_k, i, j, N, d=32, eps=0.0):
    """Only key j is active (phi(k_j) = e_fk, v_j = e_0); query i has phi(q_i) = e_fq."""
    Q = -np.ones((1, 1, N, d)); K = -np.ones((1, 1, N, d)); V = np.zeros((1, 1, N, d))
    Q[0, 0, i, f_q] = 1.0
    K[0, 0, j, f_k] = 1.0
    V[0, 0, j, 0] = 1.0
    return oracle.forward(Q, K, V, 1, rope=rope, eps=eps)["O"][0, 0, i, 0]


def _slice_of(f):
    """(axis, pair index m, slice width) of feature f under the 8/12/12 split."""
    if f < 8:
        return 0, f // 2, 8
    if f < 20:
        return 1, (f - 8) // 2, 12
    return 2, (f - 20) // 2, 12


@pytest.mark.parametrize("f", [0, 1, 6, 8, 13, 19, 20, 25, 31])
def test_rope_closed_form_same_feature(f):
    """Numerator of a one-hot pair = cos(theta_m * (pos_j - pos_i)) on f's axis,
    theta_m = 10000^(-2m/width); computed here with math.cos from the formula."""
    gh, gw = 5, 7
    rope = Rope(8, 12, 12, gh, gw, 3, 10000.0)
    N = 3 * gh * gw
    i, j = 4, 2 * gh * gw + 3 * gw + 6          # query at (t0+0,0,4), key at (t0+2,3,6)
    pos_i = (3 + i // (gh * gw), (i // gw) % gh, i % gw)
    pos_j = (3 + j // (gh * gw), (j // gw) % gh, j % gw)
    axis, m, width = _slice_of(f)
    theta = 10000.0 ** (-2.0 * m / width)
    expect = math.cos(theta * (pos_j[axis] - pos_i[axis]))
    got = _one_hot_case(rope, f, f, i, j, N)
    assert abs(got - expect) < 1e-13


@pytest.mark.parametrize("m_axis", [(0, 1), (1, 4), (2, 5)])
def test_rope_closed_form_cross_pair(m_axis):
    """phi(q_i) = e_{2m}, phi(k_j) = e_{2m+1}: numerator = sin(a_i - a_j)
    (rotation by +angle, adjacent pairs).  phi(q).z = 0 here, so eps = 1 makes
    the denominator exactly 1."""
    axis, m = m_axis
    off = [0, 8, 20][axis]
    width = [8, 12, 12][axis]
    gh, gw = 4, 6
    rope = Rope(8, 12, 12, gh, gw, 0, 10000.0)
    N = 2 * gh * gw
    i, j = 1 * gh * gw + 2 * gw + 5, 3
    pos_i = (i // (gh * gw), (i // gw) % gh, i % gw)
    pos_j = (j // (gh * gw), (j // gw) % gh, j % gw)
    theta = 10000.0 ** (-2.0 * m / width)
    expect = math.sin(theta * (pos_i[axis] - pos_j[axis]))
    got = _one_hot_case(rope, off + 2 * m, off + 2 * m + 1, i, j, N, eps=1.0)
    assert abs(got - expect) < 1e-13


def test_rope_time_shift_invariance_and_denominator():
    """A global shift of t0 leaves O unchanged; the denominator never rotates."""
    Q, K, V = _tiny(13, N=2 * 48)
    r0 = Rope(8, 12, 12, 4, 6, 0, 10000.0)
    r1 = Rope(8, 12, 12, 4, 6, 1000, 10000.0)
    a = oracle.forward(Q, K, V, 2, rope=r0, want_den=True)
    b = oracle.forward(Q, K, V, 2, rope=r1, want_den=True)
    c = oracle.forward(Q, K, V, 2, want_den=True)
    assert normwise_error(b["O"], a["O"]) < 1e-10
    assert np.array_equal(a["den"], c["den"])
    assert np.array_equal(a["z"], c["z"])
    assert normwise_error(a["O"], c["O"]) > 1e-3      # RoPE does change the numerator


def test_rope_one_position_grid_is_identity_on_first_token():
    """Token 0 at t0 = 0 sits at position (0,0,0): its rotation is the identity,
    so a one-token call equals the call without RoPE."""
    Q, K, V = _tiny(14, N=1)
    r = Rope(8, 12, 12, 3, 3, 0, 10000.0)
    a = oracle.forward(Q, K, V, 1, rope=r)
    b = oracle.forward(Q, K, V, 1)
    assert np.array_equal(a["O"], b["O"]) and np.array_equal(a["S"], b["S"])


def test_brute_force_rope_rotation_preserves_norm():
    x = np.random.default_rng(15).standard_normal((1, 1, 60, 32))
    y = oracle.rope_apply(x[0, 0], Rope(8, 12, 12, 3, 4, 7, 10000.0), 32)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x[0, 0], axis=-1), rtol=1e-14)


# --- workload generator ----------------------------------------------------------

def test_generator_is_seeded_and_bf16_exact():
    a = make_inputs(CONFIGS["c3"], nb=2, n=40, H=3)
    b = make_inputs(CONFIGS["c3"], nb=2, n=40, H=3)
    assert np.array_equal(a["Q_bits"], b["Q_bits"])
    # bf16-exact: the low 16 bits of every float32 are zero
    assert np.all((a["K"].view(np.uint32) & 0xFFFF) == 0)
    g = make_inputs(CONFIGS["c5"], nb=8, n=4, H=2)["g"]
    assert g.shape == (1, 2, 8) and np.all((g > 0) & (g < 1))


# --- the error measure behind every parity assertion -------------------------
# normwise_error(x, ref): per (b,h) slice, max|x - ref| / max|ref| (the scale
# taken from the reference), then the largest slice value.  Each case below has
# an answer worked out by hand that a plausible slip in the measure (one global
# scale, a mean, a scale from the result) gets wrong.

def test_normwise_error_scale_is_per_slice():
    """Two slices whose scales differ by 12000x, the error in the small one:
    a per-slice measure reports 0.25; one global scale would report 0.25/12000."""
    ref = np.zeros((1, 2, 4, 3))
    ref[0, 0] = 1000.0 * np.arange(1, 13).reshape(4, 3)      # max |ref| = 12000
    ref[0, 1] = np.arange(1, 13).reshape(4, 3) / 12.0        # max |ref| = 1
    x = ref.copy()
    x[0, 1, 2, 1] += 0.25
    assert normwise_error(x, ref) == pytest.approx(0.25, rel=1e-12)
    # the same error in the large slice is small at that slice's scale
    y = ref.copy()
    y[0, 0, 2, 1] += 0.25
    assert normwise_error(y, ref) == pytest.approx(0.25 / 12000.0, rel=1e-12)


def test_normwise_error_is_a_max_not_a_mean():
    """One element of eight off by 0.5 at scale 1: 0.5 (a mean would give 0.0625);
    two slices at 0.1 and 0.3: 0.3 (a mean over slices would give 0.2)."""
    ref = np.ones((1, 1, 8, 1))
    x = ref.copy()
    x[0, 0, 3, 0] = 1.5
    assert normwise_error(x, ref) == 0.5
    ref2 = np.ones((2, 1, 5, 2))
    x2 = ref2.copy()
    x2[0, 0, 1, 1] += 0.1
    x2[1, 0, 4, 0] -= 0.3
    assert normwise_error(x2, ref2) == pytest.approx(0.3, rel=1e-12)


def test_normwise_error_scale_comes_from_the_reference():
    """ref max 1, x max 3: error (3 - 1) / 1 = 2, not (3 - 1) / 3; the measure is
    not symmetric in its arguments."""
    ref = np.ones((1, 1, 4, 1))
    x = ref.copy()
    x[0, 0, 0, 0] = 3.0
    assert normwise_error(x, ref) == 2.0
    assert normwise_error(ref, x) == pytest.approx(2.0 / 3.0, rel=1e-15)


def test_normwise_error_zero_reference_and_non_finite():
    """A slice whose reference is all zero is measured by its absolute error
    (zero when the result is zero too); any NaN or inf in the result is inf."""
    ref = np.zeros((1, 2, 3, 2))
    ref[0, 0] = 2.0
    assert normwise_error(ref.copy(), ref) == 0.0
    x = ref.copy()
    x[0, 1, 1, 1] = -1e-3
    assert normwise_error(x, ref) == pytest.approx(1e-3, rel=1e-15)
    for bad in (np.nan, np.inf, -np.inf):
        y = ref.copy()
        y[0, 0, 2, 0] = bad
        assert normwise_error(y, ref) == float("inf")
    with pytest.raises(ValueError):
        normwise_error(np.zeros((1, 1, 2)), np.zeros((1, 1, 3)))


def test_normwise_error_is_scale_invariant():
    rng = np.random.default_rng(21)
    ref = rng.standard_normal((2, 3, 10, 4))
    x = ref + 1e-3 * rng.standard_normal(ref.shape)
    e = normwise_error(x, ref)
    assert 1e-4 < e < 1e-2
    assert normwise_error(1024.0 * x, 1024.0 * ref) == pytest.approx(e, rel=1e-12)


# --- the per-block states the per-kernel parity tests compare against ----------

@pytest.mark.parametrize("variant", ["plain", "gate", "gate_state_in", "rope"])
def test_block_states_are_the_states_of_truncated_calls(variant):
    """Exported block state c (inclusive) == the final state of the same call
    cut after block c; the last one == the call's final state.  Exported local
    state c == phi(K_c)^T V_c (rotated keys with RoPE) and sum phi(K_c), by
    matrix products and the brute force's own rotation."""
    nb, n, d = 5, 12, 32
    Q, K, V = _tiny(31, N=nb * n)
    rng = np.random.default_rng(32)
    g = rng.uniform(0.2, 0.9, (1, 2, nb)) if "gate" in variant else None
    S0 = z0 = None
    if "state_in" in variant:
        S0 = rng.standard_normal((1, 2, d, d)) * 5
        z0 = np.abs(rng.standard_normal((1, 2, d))) * 20
    rope = Rope(8, 12, 12, 2, 3, 4, 10000.0) if variant == "rope" else None
    full = oracle.forward(Q, K, V, nb, g=g, rope=rope, S0=S0, z0=z0, want_blocks=True,
                          want_local=True)
    for c in range(nb):
        cut = slice(0, (c + 1) * n)
        part = oracle.forward(Q[:, :, cut], K[:, :, cut], V[:, :, cut], c + 1,
                              g=None if g is None else g[:, :, :c + 1], rope=rope,
                              S0=S0, z0=z0)
        assert normwise_error(full["S_blocks"][:, :, c], part["S"]) < 1e-14
        assert normwise_error(full["z_blocks"][:, :, c], part["z"]) < 1e-14
        blk = slice(c * n, (c + 1) * n)
        A = np.maximum(K[:, :, blk], 0.0)
        if rope is None:
            Ar = A
        else:
            # the brute force rotates call tokens 0 .. N-1: block c's keys sit at c*n ..
            padded = np.concatenate([np.zeros((1, 2, c * n, d)), A], axis=2)
            Ar = np.stack([oracle.rope_apply(padded[0, h], rope, d)[c * n:] for h in range(2)])[None]
        assert normwise_error(full["S_local"][:, :, c], np.swapaxes(Ar, -1, -2) @ V[:, :, blk]) < 1e-13
        assert normwise_error(full["z_local"][:, :, c], A.sum(axis=2)) < 1e-14
    assert np.array_equal(full["S_blocks"][:, :, -1], full["S"])
    assert np.array_equal(full["z_blocks"][:, :, -1], full["z"])
    if nb > 1 and g is not None:
        # inclusive, decayed: block 1 = g_1 * block 0 + local 1
        want = g[:, :, 1, None, None] * full["S_blocks"][:, :, 0] + full["S_local"][:, :, 1]
        assert normwise_error(full["S_blocks"][:, :, 1], want) < 1e-14
