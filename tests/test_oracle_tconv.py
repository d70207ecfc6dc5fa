"""Pins of the temporal-convolution oracle (CPU only).

Each test ties oracle.tconv.temporal_conv to something it cannot share a
mistake with: the talk's training construction (cached token and zero padding
around each block, a plain convolution, padding dropped), numpy's own
convolution where the blocks reduce to textbook cases, a hand-worked example,
and the streaming invariant (block steps with the cache carried equal one
call)."""
import numpy as np
import pytest

from oracle.tconv import temporal_conv, temporal_conv_training_form


def _draw(seed, B=2, T=6, P=5, C=4):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, T, P, C)), rng.standard_normal((C, 3)),
            rng.standard_normal(C), rng.standard_normal((B, P, C)))


@pytest.mark.parametrize("F", [1, 2, 3, 6])
@pytest.mark.parametrize("with_cache", [False, True])
def test_equals_the_training_construction(F, with_cache):
    X, w, b, cache = _draw(1)
    c = cache if with_cache else None
    Y, _ = temporal_conv(X, w, F, bias=b, cache_in=c)
    Z = temporal_conv_training_form(X, w, F, bias=b, cache_in=c)
    np.testing.assert_allclose(Y, Z, rtol=0, atol=1e-12)


def test_one_block_is_a_plain_same_convolution():
    """F = T (one block, no cache): numpy's convolution with zero padding at
    both ends, channel by channel (np.convolve flips the kernel)."""
    X, w, b, _ = _draw(2, T=7)
    Y, _ = temporal_conv(X, w, 7, bias=b)
    B, T, P, C = X.shape
    for bb in range(B):
        for p in range(P):
            for c in range(C):
                ref = np.convolve(X[bb, :, p, c], w[c, ::-1], mode="same") + b[c]
                np.testing.assert_allclose(Y[bb, :, p, c], ref, rtol=0, atol=1e-12)


def test_one_frame_blocks_are_a_causal_convolution():
    """F = 1: every frame is its own block, so only taps t-1 and t remain:
    numpy's full convolution with the two causal taps, cut to the first T."""
    X, w, b, _ = _draw(3, T=5)
    Y, _ = temporal_conv(X, w, 1, bias=b)
    B, T, P, C = X.shape
    for bb in range(B):
        for p in range(P):
            for c in range(C):
                ref = np.convolve(X[bb, :, p, c], np.array([w[c, 1], w[c, 0]]), mode="full")[:T] + b[c]
                np.testing.assert_allclose(Y[bb, :, p, c], ref, rtol=0, atol=1e-12)


def test_hand_example():
    """One position, one channel, two blocks of two frames, x = 1, 2 | 3, 4,
    taps (1, 10, 100), bias 0.5, cache 7:
      frame 0: 7 + 10*1 + 100*2 = 217.5 with the bias
      frame 1: 1 + 20 + 0 (end of block) = 21.5
      frame 2: 2 + 30 + 400 = 432.5
      frame 3: 3 + 40 + 0 = 43.5"""
    X = np.array([1.0, 2.0, 3.0, 4.0]).reshape(1, 4, 1, 1)
    w = np.array([[1.0, 10.0, 100.0]])
    Y, cache = temporal_conv(X, w, 2, bias=np.array([0.5]), cache_in=np.array([7.0]).reshape(1, 1, 1))
    assert Y.reshape(-1).tolist() == [217.5, 21.5, 432.5, 43.5]
    assert cache.reshape(-1).tolist() == [4.0]


def test_streaming_steps_equal_one_call():
    """Block by block with the cache carried (a frame per position and
    channel: constant size) == one call over all blocks."""
    X, w, b, cache = _draw(4, T=12)
    F = 3
    Y, last = temporal_conv(X, w, F, bias=b, cache_in=cache)
    c = cache
    outs = []
    for blk in range(4):
        y, c = temporal_conv(X[:, blk * F:(blk + 1) * F], w, F, bias=b, cache_in=c)
        assert c.shape == cache.shape
        outs.append(y)
    np.testing.assert_array_equal(np.concatenate(outs, axis=1), Y)
    np.testing.assert_array_equal(c, last)


def test_no_future_block_reaches_a_frame():
    """Changing block k+1 leaves every output of blocks 0..k unchanged, and
    changing the last frame of block k changes block k+1's first output."""
    X, w, b, _ = _draw(5, T=9)
    F = 3
    Y, _ = temporal_conv(X, w, F, bias=b)
    X2 = X.copy()
    X2[:, 6:] += 100.0
    Y2, _ = temporal_conv(X2, w, F, bias=b)
    np.testing.assert_array_equal(Y2[:, :6], Y[:, :6])
    X3 = X.copy()
    X3[:, 2] += 1.0
    Y3, _ = temporal_conv(X3, w, F, bias=b)
    np.testing.assert_allclose(Y3[:, 3] - Y[:, 3], np.broadcast_to(w[:, 0], Y[:, 3].shape), atol=1e-12)


def test_tiny_workload_training_construction():
    """The tiny fp32 conv workload's own seeded inputs: oracle == the talk's
    training construction, with and without the cache."""
    from workloads import CONV_CONFIGS, make_conv_inputs
    x = make_conv_inputs(CONV_CONFIGS["t1"])
    for c in (None, x["cache"]):
        Y, _ = temporal_conv(x["X"], x["w"], x["F"], bias=x["bias"], cache_in=c)
        Z = temporal_conv_training_form(x["X"], x["w"], x["F"], bias=x["bias"], cache_in=c)
        np.testing.assert_allclose(Y, Z, rtol=0, atol=1e-12)
