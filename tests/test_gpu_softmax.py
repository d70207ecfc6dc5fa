"""GPU parity of the softmax anchors (svla_softmax_attention through the C ABI)
against the numpy fp64 oracle.

Tolerance (normwise per (b,h) slice): the logits, weights and sums are fp32
and the inputs bf16-exact, but the weights enter the matrix cores rounded to
bf16 (at most 2^-9 of each) while the sum that divides them is taken
unrounded, and O is rounded to bf16; each output element is a convex
combination of V values, so its error is at most about 2^-8 of max|V| over its
visible keys, which is a few times max|O|; measured 2.3e-3 to 3.8e-3 on the
cases below; tested at 1e-2.
"""
import numpy as np
import pytest
import torch

from oracle import normwise_error as nerr
from oracle.softmax import softmax_attention
from workloads import bf16_round

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-2


@pytest.fixture(scope="module")
def svla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_causal_linear_relu_amd as m
    m.library()
    return m


def _inputs(seed, B, H, Nq, Nk, d):
    rng = np.random.default_rng(seed)
    Q = bf16_round(rng.standard_normal((B, H, Nq, d), dtype=np.float32))
    K = bf16_round(rng.standard_normal((B, H, Nk, d), dtype=np.float32))
    V = bf16_round(rng.standard_normal((B, H, Nk, d), dtype=np.float32))
    return Q, K, V


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(torch.bfloat16)


CASES = [
    # name, B, H, nb, n, extra cached keys, d
    ("three_blocks_ragged", 1, 2, 3, 50, 0, 128),
    ("one_block_bidirectional", 1, 3, 1, 200, 0, 64),
    ("batch_and_odd_blocks", 2, 2, 4, 33, 0, 128),
    ("step_with_cache", 1, 2, 1, 70, 210, 128),
    ("token_causal", 1, 1, 9, 1, 0, 128),
    ("long_blocks_d64", 1, 2, 2, 300, 0, 64),
    ("query_tile_spans_blocks", 1, 2, 5, 100, 37, 128),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_matches_oracle(svla, case):
    name, B, H, nb, n, extra, d = case
    print("softmax case %s" % name, flush=True)
    Nq = nb * n
    Q, K, V = _inputs(80 + len(name), B, H, Nq, Nq + extra, d)
    O = svla.softmax_attention(_t(Q), _t(K), _t(V), nb)
    torch.cuda.synchronize()
    ref = softmax_attention(Q, K, V, nb)
    got = O.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    assert nerr(got, ref) <= TOL, nerr(got, ref)


def test_sharp_logits_and_explicit_scale(svla):
    """Large logits (scale 1): the running max must carry the sum."""
    Q, K, V = _inputs(90, 1, 2, 3 * 64, 3 * 64, 64)
    O = svla.softmax_attention(_t(Q), _t(K), _t(V), 3, scale=1.0)
    torch.cuda.synchronize()
    ref = softmax_attention(Q, K, V, 3, scale=1.0)
    assert nerr(O.float().cpu().numpy(), ref) <= TOL


def test_steps_equal_one_call_bit_for_bit(svla):
    """Each block as a streaming step (nb = 1 against the cache of the blocks
    so far) gives the one-shot call's rows bit for bit: every query row sees
    the same keys in the same tile order."""
    B, H, nb, n, d = 1, 3, 4, 90, 128
    Q, K, V = _inputs(91, B, H, nb * n, nb * n, d)
    Qt, Kt, Vt = _t(Q), _t(K), _t(V)
    one = svla.softmax_attention(Qt, Kt, Vt, nb)
    for c in range(nb):
        step = svla.softmax_attention(Qt[:, :, c * n:(c + 1) * n].contiguous(),
                                      Kt[:, :, :(c + 1) * n].contiguous(),
                                      Vt[:, :, :(c + 1) * n].contiguous(), 1)
        assert torch.equal(step, one[:, :, c * n:(c + 1) * n])


def test_full_size_anchor_every_head(svla):
    """The 2.0-style 720p anchor: B1 H20 d128, 8 blocks of 1760 tokens, every
    head against the oracle."""
    B, H, nb, n, d = 1, 20, 8, 1760, 128
    print("softmax full size", flush=True)
    Q, K, V = _inputs(95, B, H, nb * n, nb * n, d)
    O = svla.softmax_attention(_t(Q), _t(K), _t(V), nb)
    torch.cuda.synchronize()
    got = O.float().cpu().numpy()
    for h0 in range(0, H, 5):
        sl = slice(h0, h0 + 5)
        ref = softmax_attention(Q[:, sl], K[:, sl], V[:, sl], nb)
        assert nerr(got[:, sl], ref) <= TOL
