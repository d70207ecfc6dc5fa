"""The seeded generator's storage-type rounding (CPU only): bf16 and OCP FP8
E4M3, each against a brute-force nearest-value search."""
import numpy as np

from workloads import CONFIGS, bf16_bits, bf16_from_bits, fp8_bits, fp8_from_bits, make_inputs, scaled_config


def test_fp8_decode_of_every_code():
    """The 256 E4M3 codes against the format's definition written out: the
    largest finite value is 448, the smallest subnormal 2^-9, S.1111.111 NaN,
    and 0x00 / 0x80 are +0 / -0."""
    v = fp8_from_bits(np.arange(256, dtype=np.uint8))
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6
    assert v[0x38] == 1.0 and v[0x39] == 1.125 and v[0x40] == 2.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    finite = v[np.isfinite(v) & (np.arange(256) < 0x80)]
    assert np.all(np.diff(finite) > 0)                     # codes 0..0x7E increase


def test_fp8_rounding_is_nearest_ties_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 3,
                        rng.uniform(-2e-3, 2e-3, 5000).astype(np.float32),
                        np.array([0.0, -0.0, 448.0, 500.0, -1e30, 1.0625, 1.1875, 2.0 ** -10,
                                  3 * 2.0 ** -10], dtype=np.float32)])
    got = fp8_from_bits(fp8_bits(x)).astype(np.float64)
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = fp8_from_bits(codes).astype(np.float64)
    for xi, gi in zip(x.astype(np.float64), got):
        a = min(abs(xi), 448.0)
        d = np.abs(vals - a)
        best = np.flatnonzero(d == d.min())
        c = best[0] if len(best) == 1 else best[best % 2 == 0][0]      # tie: even mantissa
        assert abs(gi) == vals[c] and (gi == 0 or np.sign(gi) == np.sign(xi)), (xi, gi, vals[c])


def test_bf16_rounding_is_nearest_ties_even():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(2000).astype(np.float32)
    got = bf16_from_bits(bf16_bits(x)).astype(np.float64)
    for xi, gi in zip(x.astype(np.float64), got):
        u = np.float32(xi).view(np.uint32)
        lo = np.uint32(u & 0xFFFF0000).view(np.float32).astype(np.float64)
        hi = np.uint32((u & 0xFFFF0000) + 0x10000).view(np.float32).astype(np.float64)
        if abs(xi - lo) < abs(hi - xi):
            want = lo
        elif abs(xi - lo) > abs(hi - xi):
            want = hi
        else:
            want = lo if (int(u) >> 16) % 2 == 0 else hi
        assert gi == want


def test_fp8_workload_inputs_are_fp8_exact():
    x = make_inputs(scaled_config(CONFIGS["c3"], dtype="fp8"), nb=2, n=40, H=3)
    assert x["Q_bits"].dtype == np.uint8
    assert np.array_equal(fp8_from_bits(x["K_bits"]), x["K"])
    assert np.array_equal(fp8_from_bits(fp8_bits(x["V"])), x["V"])
