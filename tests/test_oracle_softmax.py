"""Pins of the softmax-anchor oracle (CPU only): the definition written out
entry by entry on tiny inputs, closed forms (equal logits give the mean of the
visible values, one dominant logit gives its value), the block-causal
visibility, a streaming step equal to the rows of its block in one call,
invariance under a common logit shift and under a joint permutation of the
visible keys, and convexity."""
import math

import numpy as np
import pytest

from oracle.softmax import softmax_attention, visible_keys


def _rand(seed, B=1, H=2, Nq=12, Nk=None, d=8):
    rng = np.random.default_rng(seed)
    Nk = Nq if Nk is None else Nk
    return (rng.standard_normal((B, H, Nq, d)), rng.standard_normal((B, H, Nk, d)),
            rng.standard_normal((B, H, Nk, d)))


def test_entry_by_entry_on_tiny_inputs():
    Q, K, V = _rand(1, B=1, H=2, Nq=6, Nk=8, d=4)
    nb, n, scale = 3, 2, 0.7
    O = softmax_attention(Q, K, V, nb, scale=scale)
    for h in range(2):
        for i in range(6):
            c = i // n
            m = 8 - 6 + (c + 1) * n
            w = [math.exp(scale * sum(Q[0, h, i, f] * K[0, h, j, f] for f in range(4))) for j in range(m)]
            tot = sum(w)
            for f in range(4):
                ref = sum(w[j] * V[0, h, j, f] for j in range(m)) / tot
                assert abs(O[0, h, i, f] - ref) < 1e-12


def test_equal_logits_give_the_mean_of_visible_values():
    Q, K, V = _rand(2, Nq=12, d=8)
    K[:] = 0.0
    O = softmax_attention(Q, K, V, nb=3)
    for c in range(3):
        m = visible_keys(12, 12, 3, c)
        assert np.allclose(O[:, :, 4 * c:4 * c + 4], V[:, :, :m].mean(axis=2, keepdims=True), atol=1e-13)


def test_one_dominant_logit_gives_its_value():
    Q, K, V = _rand(3, Nq=8, d=8)
    Q[:] = 0.0
    Q[..., 0] = 1.0
    K[..., 0] = 0.0
    K[:, :, 1, 0] = 800.0            # key 1 is visible to every block and dominates (exp(800) overflows fp64 unless the row max is taken out first)
    O = softmax_attention(Q, K, V, nb=4, scale=1.0)
    assert np.allclose(O, np.broadcast_to(V[:, :, 1:2], O.shape), atol=1e-12)


def test_block_causal_visibility():
    Q, K, V = _rand(4, Nq=12, d=8)
    O = softmax_attention(Q, K, V, nb=3)
    K2, V2 = K.copy(), V.copy()
    K2[:, :, 8:] += 5.0              # block 2 only
    V2[:, :, 8:] -= 3.0
    O2 = softmax_attention(Q, K2, V2, nb=3)
    assert np.array_equal(O[:, :, :8], O2[:, :, :8])
    assert not np.allclose(O[:, :, 8:], O2[:, :, 8:])
    K3 = K.copy()
    K3[:, :, 5] += 2.0               # block 1 is seen by blocks 1 and 2, not 0
    O3 = softmax_attention(Q, K3, V, nb=3)
    assert np.array_equal(O[:, :, :4], O3[:, :, :4])
    assert not np.allclose(O[:, :, 4:], O3[:, :, 4:])


def test_streaming_step_equals_its_rows_of_one_call():
    Q, K, V = _rand(5, Nq=15, d=8)
    O = softmax_attention(Q, K, V, nb=5)
    for c in range(5):
        n = 3
        step = softmax_attention(Q[:, :, c * n:(c + 1) * n], K[:, :, :(c + 1) * n], V[:, :, :(c + 1) * n], nb=1)
        assert np.allclose(step, O[:, :, c * n:(c + 1) * n], atol=1e-13)


def test_common_logit_shift_changes_nothing():
    Q, K, V = _rand(6, Nq=10, d=6)
    s = 0.4
    Qa = np.concatenate([Q, np.ones(Q.shape[:3] + (1,))], axis=3)
    Ka = np.concatenate([K, np.full(K.shape[:3] + (1,), 7.5)], axis=3)   # + 7.5 s on every logit
    Va = np.concatenate([V, np.zeros(V.shape[:3] + (1,))], axis=3)
    assert np.allclose(softmax_attention(Qa, Ka, Va, nb=2, scale=s)[..., :6],
                       softmax_attention(Q, K, V, nb=2, scale=s), atol=1e-13)


def test_permuting_visible_keys_and_values_jointly_changes_nothing():
    Q, K, V = _rand(7, Nq=12, d=8)
    p = np.random.default_rng(0).permutation(12)
    O = softmax_attention(Q, K, V, nb=1)
    assert np.allclose(softmax_attention(Q, K[:, :, p], V[:, :, p], nb=1), O, atol=1e-13)


def test_outputs_are_convex_combinations():
    Q, K, V = _rand(8, Nq=16, d=8)
    O = softmax_attention(Q * 3.0, K, V, nb=4)
    for c in range(4):
        m = 4 * (c + 1)
        lo = V[:, :, :m].min(axis=2, keepdims=True)
        hi = V[:, :, :m].max(axis=2, keepdims=True)
        blk = O[:, :, 4 * c:4 * c + 4]
        assert np.all(blk >= lo - 1e-12) and np.all(blk <= hi + 1e-12)


@pytest.mark.parametrize("bad", [dict(nb=0), dict(nb=5), dict(Nk=8)])
def test_rejects_bad_shapes(bad):
    Q, K, V = _rand(9, Nq=12, Nk=bad.get("Nk", 12), d=4)
    with pytest.raises(ValueError):
        softmax_attention(Q, K, V, nb=bad.get("nb", 3))
