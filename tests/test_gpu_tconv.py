"""GPU parity of the temporal convolution (svla_temporal_conv through the C
ABI) against the numpy fp64 oracle.

Tolerance (normwise per (b, frame) slice, the oracle's measure): the kernel
sums three products in fp32 from exact inputs and fp32 taps, so its only
sizeable error is the final rounding to the output type: at most 2^-9 of an
element for bf16 (tested at 2^-8), about 1e-7 for fp32 (tested at 1e-6).
"""
import numpy as np
import pytest
import torch

from oracle import normwise_error as nerr
from oracle.tconv import temporal_conv, temporal_conv_training_form
from workloads import CONV_CONFIGS, make_conv_inputs, scaled_config

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {"bf16": 2.0 ** -8, "f32": 1e-6}


@pytest.fixture(scope="module")
def svla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_causal_linear_relu_amd as m
    m.library()
    return m


def _t(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dtype)


def _dt(x):
    return torch.bfloat16 if x["dtype"] == "bf16" else torch.float32


def _run(svla, x, with_cache=True, bias=True):
    dt = _dt(x)
    X = _t(x["X"], dt)
    cin = _t(x["cache"], dt) if with_cache else None
    cout = torch.empty((x["B"], x["P"], x["C"]), dtype=dt, device=DEV)
    Y, c = svla.temporal_conv(X, _t(x["w"], torch.float32), x["F"],
                              bias=_t(x["bias"], torch.float32) if bias else None,
                              cache_in=cin, cache_out=cout)
    torch.cuda.synchronize()
    return Y.float().cpu().numpy(), c.float().cpu().numpy()


def test_tiny_workload_on_its_own_inputs(svla):
    x = make_conv_inputs(CONV_CONFIGS["t1"])
    Y, c = _run(svla, x)
    ref, last = temporal_conv(x["X"], x["w"], x["F"], bias=x["bias"], cache_in=x["cache"])
    assert nerr(Y, ref) <= TOL["f32"]
    assert np.array_equal(c, last)
    tf = temporal_conv_training_form(x["X"], x["w"], x["F"], bias=x["bias"], cache_in=x["cache"])
    assert nerr(Y, tf) <= TOL["f32"]


SHAPES = [
    # name, dtype, B, nb, F, P, C, cache, bias
    ("one_frame_blocks", "bf16", 2, 9, 1, 7, 16, True, True),
    ("block_longer_than_a_chunk", "bf16", 1, 2, 13, 5, 24, True, True),
    ("chunks_end_at_block_ends", "bf16", 1, 6, 4, 3, 8, False, True),
    ("chunks_end_inside_blocks", "bf16", 3, 4, 5, 11, 40, True, False),
    ("one_position_one_chunk", "bf16", 1, 3, 3, 1, 8, True, True),
    ("fp32_multi_chunk", "f32", 2, 5, 3, 6, 32, True, True),
    ("many_positions", "bf16", 1, 2, 3, 390, 256, True, True),
]


@pytest.mark.parametrize("case", SHAPES, ids=[c[0] for c in SHAPES])
def test_shapes(svla, case):
    name, dtype, B, nb, F, P, C, cache, bias = case
    x = make_conv_inputs(scaled_config(CONV_CONFIGS["t1"], dtype=dtype, seed=60), B=B, nb=nb, F=F,
                         P=P, C=C)
    Y, c = _run(svla, x, with_cache=cache, bias=bias)
    ref, last = temporal_conv(x["X"], x["w"], F, bias=x["bias"] if bias else None,
                              cache_in=x["cache"] if cache else None)
    assert nerr(Y, ref) <= TOL[dtype], nerr(Y, ref)
    assert np.array_equal(c, last)


def test_stream_equals_one_call_and_in_place_cache(svla):
    """Block steps with the cache committed in place give the one call's bits."""
    x = make_conv_inputs(scaled_config(CONV_CONFIGS["t4"], seed=61), nb=10, P=50, C=64)
    dt = torch.bfloat16
    X = _t(x["X"], dt)
    w, b = _t(x["w"], torch.float32), _t(x["bias"], torch.float32)
    cache0 = _t(x["cache"], dt)
    Y1 = svla.temporal_conv(X, w, 3, bias=b, cache_in=cache0)
    cache = cache0.clone()
    outs = []
    for s in range(10):
        Xs = X[:, 3 * s:3 * (s + 1)].contiguous()
        y, cache = svla.temporal_conv(Xs, w, 3, bias=b, cache_in=cache, cache_out=cache)
        outs.append(y)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=1), Y1)
    assert torch.equal(cache, X[:, -1])


def test_no_frames_passes_the_cache_on(svla):
    x = make_conv_inputs(scaled_config(CONV_CONFIGS["t1"], dtype="bf16"), nb=1, F=2, P=4, C=16)
    X = torch.empty((1, 0, 4, 16), dtype=torch.bfloat16, device=DEV)
    cin = _t(x["cache"], torch.bfloat16)
    cout = torch.full_like(cin, float("nan"))
    Y, c = svla.temporal_conv(X, _t(x["w"], torch.float32), 2, cache_in=cin, cache_out=cout)
    torch.cuda.synchronize()
    assert Y.numel() == 0 and torch.equal(cout, cin)


@pytest.mark.parametrize("name", ["t3", "t4"])
def test_full_size_every_element(svla, name):
    """The 720p clip as one call, and the minute-long stream as 80 block steps
    with the cache carried (and as one call): every element against the oracle."""
    cfg = CONV_CONFIGS[name]
    x = make_conv_inputs(cfg)
    dt = torch.bfloat16
    X = _t(x["X"], dt)
    w, b = _t(x["w"], torch.float32), _t(x["bias"], torch.float32)
    cin = _t(x["cache"], dt)
    Y1 = svla.temporal_conv(X, w, cfg.F, bias=b, cache_in=cin)
    if cfg.streaming:
        bufs = [cin.clone(), torch.empty_like(cin)]
        outs = []
        for s in range(cfg.nb):
            Xs = X[:, s * cfg.F:(s + 1) * cfg.F].contiguous()
            y, _ = svla.temporal_conv(Xs, w, cfg.F, bias=b, cache_in=bufs[s % 2],
                                      cache_out=bufs[(s + 1) % 2])
            outs.append(y)
        Ys = torch.cat(outs, dim=1)
        torch.cuda.synchronize()
        assert torch.equal(Ys, Y1)
    torch.cuda.synchronize()
    ref, _ = temporal_conv(x["X"], x["w"], cfg.F, bias=x["bias"], cache_in=x["cache"])
    e = nerr(Y1.float().cpu().numpy(), ref)
    print("%s every element: %.2e" % (name, e))
    assert e <= TOL["bf16"]
