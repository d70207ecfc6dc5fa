"""Quadratic brute force for block-causal ReLU linear attention (numpy fp64).

TEST INFRASTRUCTURE.  No state, no recurrence: every query is compared with
every key its block may see, with the block mask of the SANA-Video talk
(its description of the hybrid schedule: causal over blocks, bidirectional
diffusion inside each block) and, for
the gated variant of SANA-Video 2.0, the product of the decays of the blocks
in between.  For token i in block c(i) and token j in block c(j):

    w_ij = prod_{c = c(j)+1 .. c(i)} g_c   if c(j) <= c(i), else 0
    O_i  = sum_j w_ij (R_i phi(q_i) . R_j phi(k_j)) v_j
           / (sum_j w_ij (phi(q_i) . phi(k_j)) + eps)

plus, when a state (S0, z0) is carried in, the terms
w0_i (R_i phi(q_i))^T S0 and w0_i phi(q_i) . z0 with w0_i = prod_{c<=c(i)} g_c.
Without gate and RoPE, this is the block-masked form
O_i = sum_{j in blocks <= c(i)} (phi q_i . phi k_j) v_j / sum_j (phi q_i . phi k_j).
"""
from __future__ import annotations

import numpy as np


def rope_apply(x: np.ndarray, rope, d: int) -> np.ndarray:
    """Rotate x [..., N, d] by the 3D positions of tokens 0..N-1 (vectorised).

    Written independently of the C oracle's per-token loop.
    """
    N = x.shape[-2]
    p = np.arange(N)
    hw = rope.grid_h * rope.grid_w
    positions = [rope.t0 + p // hw, (p // rope.grid_w) % rope.grid_h, p % rope.grid_w]
    widths = [rope.dt_dims, rope.dh_dims, rope.dw_dims]
    y = np.array(x, dtype=np.float64, copy=True)
    start = 0
    for pos, width in zip(positions, widths):
        half = width // 2
        if half:
            freq = float(rope.base) ** (-(2.0 * np.arange(half)) / width)
            ang = pos[:, None].astype(np.float64) * freq[None, :]   # [N, half]
            c, s = np.cos(ang), np.sin(ang)
            ev = x[..., start:start + width:2].astype(np.float64)
            od = x[..., start + 1:start + width:2].astype(np.float64)
            y[..., start:start + width:2] = ev * c - od * s
            y[..., start + 1:start + width:2] = ev * s + od * c
        start += width
    return y


def _block_weights(nb: int, g) -> np.ndarray:
    """W[ci, cj] = prod_{c = cj+1..ci} g_c for cj <= ci, else 0 (g None -> 1)."""
    W = np.zeros((nb, nb))
    for ci in range(nb):
        for cj in range(ci + 1):
            w = 1.0
            if g is not None:
                for c in range(cj + 1, ci + 1):
                    w *= float(g[c])
            W[ci, cj] = w
    return W


def brute_force(Q, K, V, nb: int, *, g=None, rope=None, S0=None, z0=None,
                eps: float = 1e-6) -> np.ndarray:
    """O of shape [B,H,N,d] by the quadratic form (fp64)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, H, N, d = Q.shape
    n = N // nb
    blk = np.arange(N) // n
    O = np.zeros_like(Q)
    for b in range(B):
        for h in range(H):
            P = np.maximum(Q[b, h], 0.0)
            A = np.maximum(K[b, h], 0.0)
            Pr = rope_apply(P, rope, d) if rope is not None else P
            Ar = rope_apply(A, rope, d) if rope is not None else A
            gb = None if g is None else np.asarray(g, dtype=np.float64)[b, h]
            Wb = _block_weights(nb, gb)
            W = Wb[blk[:, None], blk[None, :]]                 # [N, N]
            num = ((Pr @ Ar.T) * W) @ V[b, h]
            den = ((P @ A.T) * W).sum(axis=1) + eps
            if S0 is not None or z0 is not None:
                w0 = np.ones(nb)
                for c in range(nb):
                    w0[c] = np.prod(gb[:c + 1]) if gb is not None else 1.0
                wi = w0[blk]
                if S0 is not None:
                    num = num + wi[:, None] * (Pr @ np.asarray(S0, dtype=np.float64)[b, h])
                if z0 is not None:
                    den = den + wi * (P @ np.asarray(z0, dtype=np.float64)[b, h])
            with np.errstate(invalid="ignore", divide="ignore"):
                o = num / den[:, None]
            o[den == 0.0] = 0.0
            O[b, h] = o
    return O
