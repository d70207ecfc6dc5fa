"""Softmax attention anchors, block-causal, numpy fp64 -- TEST INFRASTRUCTURE
(only tests/, __graft_entry__.smoke() and bench.py's CPU baseline may import
it; it shares no code with the HIP library).

The SANA-Video 2.0 pages describe a hybrid stack: gated linear attention in
three layers of four and dense softmax attention "anchors" in the fourth
(the 2.0 news page, the hybrid linear-softmax attention paragraph; the
comfyui-wiki model page, the 2.0 section).  Readings, where the pages say no
more: an anchor is plain scaled dot-product softmax attention over the same
tokens, on the same block schedule as the linear layers -- bidirectional
inside a block, causal across blocks (the talk's block-causal generation) --
with scale 1/sqrt(d) unless given, and no RoPE.  A streaming step reads the
cached keys and values of every earlier block plus its own block, so a call
takes queries of nb blocks (Nq = nb * n) against Nk >= Nq keys, the first
Nk - Nq of which come before the queries' first block:

    query i (block c = i // n) sees keys 0 .. Nk - Nq + (c + 1) n - 1
    O_i = sum_j softmax_j(scale * q_i . k_j) v_j   over the keys it sees.

One call over all blocks is Nk = Nq; one step of block c is nb = 1 with
Nk = (c + 1) n.
"""
from __future__ import annotations

import numpy as np


def visible_keys(Nq: int, Nk: int, nb: int, block: int) -> int:
    """Number of keys the queries of `block` see."""
    n = Nq // nb
    return Nk - Nq + (block + 1) * n


def softmax_attention(Q, K, V, nb: int, scale=None):
    """O [B,H,Nq,d] (fp64) for Q [B,H,Nq,d], K, V [B,H,Nk,d]."""
    Q, K, V = (np.asarray(t, dtype=np.float64) for t in (Q, K, V))
    B, H, Nq, d = Q.shape
    Nk = K.shape[2]
    if nb <= 0 or Nq % nb or Nk < Nq or K.shape != (B, H, Nk, d) or V.shape != K.shape:
        raise ValueError("bad shapes")
    n = Nq // nb
    s = 1.0 / np.sqrt(d) if scale is None else float(scale)
    O = np.zeros_like(Q)
    for b in range(B):
        for h in range(H):
            for c in range(nb):
                rows = slice(c * n, (c + 1) * n)
                m = visible_keys(Nq, Nk, nb, c)
                logits = s * (Q[b, h, rows] @ K[b, h, :m].T)          # [n, m]
                logits = logits - logits.max(axis=1, keepdims=True)
                w = np.exp(logits)
                O[b, h, rows] = (w @ V[b, h, :m]) / w.sum(axis=1, keepdims=True)
    return O
