"""Pins of the oracle's power-of-two FP8 quantizer (CPU only)."""
import numpy as np
import pytest

from oracle import codecs, fp8_quantize_ref
from oracle.quantize import pow2_descale
from workloads import WORKLOADS


@pytest.mark.parametrize("amax,want", [
    (448.0, 1.0), (448.0 * 1.0001, 2.0), (449.0, 2.0), (224.0, 0.5), (224.5, 1.0),
    (0.0, 1.0), (448.0 * 2 ** -20, 2.0 ** -20), (5.5, 2.0 ** -6), (7.0, 2.0 ** -6), (7.01, 2.0 ** -5),
    (1e30, 2.0 ** 91), (448.0 * 2.0 ** -126, 2.0 ** -126), (1e-40, 2.0 ** -126),
])
def test_descale_rule(amax, want):
    assert pow2_descale(amax) == want
    # the defining properties: amax/d <= 448 and amax/(d/2) > 448
    d = pow2_descale(amax)
    assert amax / d <= 448.0
    if amax and d > 2.0 ** -126:
        assert amax / (d / 2) > 448.0


def test_quantize_never_saturates_and_roundtrip_error():
    rng = np.random.default_rng(3)
    for scale in (1e-3, 1.0, 37.0, 1e4):
        x = (rng.standard_normal(100000) * scale).astype(np.float32).astype(np.float64)
        codes, d = fp8_quantize_ref(x)
        vals = codecs.e4m3fn_decode(codes) * float(d)
        assert np.all(np.abs(codecs.e4m3fn_decode(codes)) <= 448.0)
        assert np.all((codes & 0x7F) != 0x7F)
        normal = np.abs(x / float(d)) >= 2.0 ** -6
        rel = np.abs(vals[normal] - x[normal]) / np.abs(x[normal])
        assert rel.max() <= 2.0 ** -4
        # the largest value uses the top binade: its code is at least 1.0 * 2^8
        assert np.abs(codecs.e4m3fn_decode(codes)).max() > 224.0


def test_gaussian_workload_descale_is_2_pow_minus_6():
    # workload 3 q: 16384 x 32 x 128 N(0,1) values; amax ~ 5.5 -> 2^-6
    w = WORKLOADS[3]
    rng = np.random.Generator(np.random.PCG64(w.seed))
    q = rng.standard_normal(w.shape("q"), dtype=np.float32)
    assert pow2_descale(float(np.abs(q).max())) == 2.0 ** -6


def test_quantize_empty_and_zero():
    codes, d = fp8_quantize_ref(np.zeros(10))
    assert d == 1.0 and np.all(codes == 0)
