"""Backward pass of block-causal ReLU linear attention, numpy fp64 -- TEST
INFRASTRUCTURE (only tests/, __graft_entry__.smoke() and bench.py's CPU
baseline may import it; it shares no code with the HIP library).

The gradients of the forward that oracle.forward computes, for the
block-causal training the SANA-Video talk describes (during causal training a
block cannot see the next one).  Per (b, h), with p = phi(q), a = phi(k) (phi =
ReLU), p~ = R p, a~ = R a (R: the 3D RoPE rotation of the token, the identity
without RoPE), block c's inclusive state S_c = g_c S_{c-1} + sum_{j in c} a~_j
v_j^T, z_c = g_c z_{c-1} + sum_{j in c} a_j, and for token i of block c

    num_i = S_c^T p~_i,  den_i = p_i . z_c + eps,  O_i = num_i / den_i.

Given dO (the gradient of a loss with respect to O), by the chain rule:

    dnum_i = dO_i / den_i,   dden_i = -(dO_i . O_i) / den_i
    dq_i   = [q_i > 0] * (R_i^T S_c dnum_i + dden_i z_c)
    G_c    = sum_{i in c} p~_i dnum_i^T + g_{c+1} G_{c+1}        (gradient reaching S_c)
    H_c    = sum_{i in c} dden_i p_i    + g_{c+1} H_{c+1}        (gradient reaching z_c)
    dv_j   = G_c^T a~_j
    dk_j   = [k_j > 0] * (R_j^T G_c v_j + H_c)                  (j in block c)
    dg_c   = <G_c, S_{c-1}> + <H_c, z_{c-1}>,  dS0 = g_0 G_0, dz0 = g_0 H_0

(G_nb = H_nb = 0; g = 1 without a gate; S_{-1} = S0, z_{-1} = z0, zero when
absent).  A token whose denominator is zero has O = 0 and passes no gradient;
the ReLU's derivative at 0 is taken as 0.
"""
from __future__ import annotations

import numpy as np


def _rotate(x, rope, sign: float):
    """R x (sign = +1) or R^T x (sign = -1) for tokens 0 .. N-1 of a call, x [N, d]."""
    if rope is None:
        return x
    N, d = x.shape
    p = np.arange(N)
    hw = rope.grid_h * rope.grid_w
    pos = [rope.t0 + p // hw, (p // rope.grid_w) % rope.grid_h, p % rope.grid_w]
    y = x.copy()
    start = 0
    for axis_pos, width in zip(pos, (rope.dt_dims, rope.dh_dims, rope.dw_dims)):
        for m in range(width // 2):
            theta = float(rope.base) ** (-2.0 * m / width)
            ang = sign * axis_pos * theta
            c, s = np.cos(ang), np.sin(ang)
            x0, x1 = x[:, start + 2 * m], x[:, start + 2 * m + 1]
            y[:, start + 2 * m] = x0 * c - x1 * s
            y[:, start + 2 * m + 1] = x0 * s + x1 * c
        start += width
    return y


def backward(Q, K, V, nb: int, dO, *, g=None, rope=None, S0=None, z0=None,
             eps: float = 1e-6) -> dict:
    """dQ, dK, dV [B,H,N,d], dg [B,H,nb], dS0 [B,H,d,d], dz0 [B,H,d] (fp64)."""
    Q, K, V, dO = (np.asarray(t, dtype=np.float64) for t in (Q, K, V, dO))
    B, H, N, d = Q.shape
    n = N // nb
    out = {k: np.zeros_like(Q) for k in ("dQ", "dK", "dV")}
    out["dg"] = np.zeros((B, H, nb))
    out["dS0"] = np.zeros((B, H, d, d))
    out["dz0"] = np.zeros((B, H, d))
    for b in range(B):
        for h in range(H):
            gg = np.ones(nb) if g is None else np.asarray(g, dtype=np.float64)[b, h]
            P, A = np.maximum(Q[b, h], 0.0), np.maximum(K[b, h], 0.0)
            Pr, Ar = _rotate(P, rope, +1.0), _rotate(A, rope, +1.0)
            # forward: every block's state and the state before it
            S = np.zeros((d, d)) if S0 is None else np.asarray(S0, dtype=np.float64)[b, h].copy()
            z = np.zeros(d) if z0 is None else np.asarray(z0, dtype=np.float64)[b, h].copy()
            Sb, zb, Sprev, zprev = [], [], [], []
            for c in range(nb):
                blk = slice(c * n, (c + 1) * n)
                Sprev.append(S.copy())
                zprev.append(z.copy())
                S = gg[c] * S + Ar[blk].T @ V[b, h, blk]
                z = gg[c] * z + A[blk].sum(axis=0)
                Sb.append(S.copy())
                zb.append(z.copy())
            # the queries' side, block by block
            dS_loc, dz_loc = [], []
            dPr = np.zeros((N, d))
            dPz = np.zeros((N, d))
            for c in range(nb):
                blk = slice(c * n, (c + 1) * n)
                num = Pr[blk] @ Sb[c]
                den = P[blk] @ zb[c] + eps
                live = den != 0.0
                safe = np.where(live, den, 1.0)
                Oc = np.where(live[:, None], num / safe[:, None], 0.0)
                dnum = np.where(live[:, None], dO[b, h, blk] / safe[:, None], 0.0)
                dden = np.where(live, -(dO[b, h, blk] * Oc).sum(axis=1) / safe, 0.0)
                dPr[blk] = dnum @ Sb[c].T
                dPz[blk] = dden[:, None] * zb[c][None, :]
                dS_loc.append(Pr[blk].T @ dnum)
                dz_loc.append(P[blk].T @ dden)
            dP = _rotate(dPr, rope, -1.0) + dPz
            out["dQ"][b, h] = dP * (Q[b, h] > 0)
            # the gradient reaching each block's state, from the last block back
            G = np.zeros((d, d))
            Hh = np.zeros(d)
            dAr = np.zeros((N, d))
            dAz = np.zeros((N, d))
            for c in range(nb - 1, -1, -1):
                nxt = gg[c + 1] if c + 1 < nb else 0.0
                G = dS_loc[c] + nxt * G
                Hh = dz_loc[c] + nxt * Hh
                blk = slice(c * n, (c + 1) * n)
                out["dg"][b, h, c] = np.sum(G * Sprev[c]) + np.dot(Hh, zprev[c])
                dAr[blk] = V[b, h, blk] @ G.T
                dAz[blk] = Hh[None, :]
                out["dV"][b, h, blk] = Ar[blk] @ G
                if c == 0:
                    out["dS0"][b, h] = gg[0] * G
                    out["dz0"][b, h] = gg[0] * Hh
            dA = _rotate(dAr, rope, -1.0) + dAz
            out["dK"][b, h] = dA * (K[b, h] > 0)
    return out
