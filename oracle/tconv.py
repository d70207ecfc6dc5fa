"""Causal temporal convolution across blocks, numpy fp64 -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It shares no code with the HIP library.

What it computes follows the SANA-Video talk's account of the causal FFN: the
Mix-FFN carries a 1-D convolution over time; when video is generated block by
block, a block may not see the next block, so a zero token separates the two
blocks during training, while a block must still see the previous block, so
the previous block's last token is kept (cached) and placed in front of the
block; the padding and the cached token are dropped from the output.
Readings where the talk says nothing (documented in the design notes of the
repository): the convolution is depthwise (one 3-tap kernel per channel),
centred (taps at t-1, t, t+1), over latent frames for each grid position and
channel; a token of that passage is one latent frame at one grid position;
the frame before the first block is zero unless a cache is passed in.

Layout: X, Y [B, T, P, C] (T frames of P = grid_h * grid_w positions, C
channels, C fastest); frames are grouped into blocks of F consecutive frames;
w [C, 3] (taps for t-1, t, t+1), bias [C] or None; cache [B, P, C].

    y[t,p,c] = bias[c] + w[c,0] x[t-1,p,c] + w[c,1] x[t,p,c] + w[c,2] x[t+1,p,c]
      x[t-1] for t = 0 is the cache (zero without one);
      x[t+1] is zero when frame t is the last frame of its block.
"""
from __future__ import annotations

import numpy as np


def temporal_conv(X, w, F: int, bias=None, cache_in=None):
    """The block-causal temporal convolution of every frame of X, frame by
    frame.  Returns (Y, cache_out) with cache_out = the last frame of X (what
    the next call needs as its cache)."""
    X = np.asarray(X, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, T, P, C = X.shape
    if F <= 0 or T % F:
        raise ValueError("T must be a multiple of the block length F")
    if w.shape != (C, 3):
        raise ValueError("w must be [C, 3]")
    b = np.zeros(C) if bias is None else np.asarray(bias, dtype=np.float64)
    prev_frame = (np.zeros((B, P, C)) if cache_in is None
                  else np.asarray(cache_in, dtype=np.float64).reshape(B, P, C))
    Y = np.zeros_like(X)
    for t in range(T):
        before = prev_frame if t == 0 else X[:, t - 1]
        last_of_block = (t % F) == F - 1
        after = np.zeros((B, P, C)) if last_of_block else X[:, t + 1]
        Y[:, t] = b + w[:, 0] * before + w[:, 1] * X[:, t] + w[:, 2] * after
    cache_out = X[:, T - 1].copy() if T > 0 else prev_frame.copy()
    return Y, cache_out


def temporal_conv_training_form(X, w, F: int, bias=None, cache_in=None):
    """The same result built the way the talk describes training: each block
    is preceded by the previous block's last frame (the cached token; the
    cache, or zero, for the first block) and followed by a zero frame; a plain
    centred 3-tap convolution runs over that sequence, one channel at a time,
    by explicit loops; the outputs at the cached and padding positions are
    dropped."""
    X = np.asarray(X, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, T, P, C = X.shape
    nb = T // F
    first_prev = (np.zeros((B, P, C)) if cache_in is None
                  else np.asarray(cache_in, dtype=np.float64).reshape(B, P, C))
    seq, keep = [], []
    for blk in range(nb):
        prev = first_prev if blk == 0 else X[:, blk * F - 1]
        seq.append(prev)
        keep.append(False)                       # the cached token
        for f in range(F):
            seq.append(X[:, blk * F + f])
            keep.append(True)
        seq.append(np.zeros((B, P, C)))          # the zero padding token
        keep.append(False)
    S = np.stack(seq, axis=1)                    # [B, L, P, C]
    L = S.shape[1]
    out = np.zeros_like(S)
    for c in range(C):
        for i in range(L):
            acc = 0.0 if bias is None else float(bias[c])
            for tap, off in enumerate((-1, 0, 1)):
                j = i + off
                if 0 <= j < L:                   # "same" padding at the ends of the sequence
                    acc = acc + w[c, tap] * S[:, j, :, c]
            out[:, i, :, c] = acc
    return out[:, np.array(keep)]
