"""Pins of the rotation oracle (oracle/rotation.py): closed forms,
orthogonality and the invariance the README states."""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("n", [1, 2, 4, 64, 128, 256])
def test_hadamard_closed_form(n):
    # Sylvester's matrix has entry (-1)^popcount(i & j)
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    assert np.array_equal(oracle.hadamard(n), (-1.0) ** pc)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_rotation_is_orthogonal_and_keeps_scores(d):
    rng = np.random.default_rng(d)
    s = rng.choice([-1.0, 1.0], d)
    r = oracle.rotation_matrix(d, s)
    np.testing.assert_allclose(r @ r.T, np.eye(d), atol=1e-14)
    q, k = rng.standard_normal((7, d)), rng.standard_normal((9, d))
    np.testing.assert_allclose(oracle.rotate_ref(q, s) @ oracle.rotate_ref(k, s).T, q @ k.T, atol=1e-12)


def test_d128_spreads_a_channel_evenly():
    rng = np.random.default_rng(1)
    s = rng.choice([-1.0, 1.0], 128)
    for i in (0, 5, 127):
        y = oracle.rotate_ref(np.eye(128)[i], s)
        pc = np.array([bin(i & j).count("1") for j in range(128)])
        np.testing.assert_allclose(y, s[i] * (-1.0) ** pc / np.sqrt(128), atol=1e-15)


def test_signs_must_be_plus_minus_one():
    with pytest.raises(ValueError):
        oracle.rotation_matrix(128, np.zeros(128))
    with pytest.raises(ValueError):
        oracle.rotation_matrix(96, np.ones(96))
    with pytest.raises(ValueError):
        oracle.rotation_matrix(192, np.ones(192))


@pytest.mark.parametrize("d", [128])
def test_rotated_quantize_round_trip(d):
    rng = np.random.default_rng(3 + d)
    s = rng.choice([-1.0, 1.0], d)
    x = rng.standard_normal((50, d))
    codes, ds, y = oracle.quantize_rotated_ref(x, s)
    back = oracle.e4m3fn_decode(codes) * float(ds)
    big = np.abs(y) >= 2.0 ** -6 * float(ds)          # normal e4m3 range
    assert np.all(np.abs(back - y)[big] <= 2.0 ** -4 * np.abs(y)[big])
    # rotating back recovers x up to that rounding
    np.testing.assert_allclose(back @ oracle.rotation_matrix(d, s).T, x, atol=0.2)


@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_key_mean_closed_forms(layout):
    rng = np.random.default_rng(9)
    B, S, Hk, d = 2, 37, 3, 8
    shp = (B, S, Hk, d) if layout == "bshd" else (B, Hk, S, d)
    c = rng.standard_normal((B, Hk, d))
    const = np.broadcast_to(c[:, None] if layout == "bshd" else c[:, :, None], shp)
    np.testing.assert_allclose(oracle.key_mean_ref(const, layout), c, atol=1e-15)
    # one position set apart: the mean moves by its deviation / S
    k = np.array(const)
    if layout == "bshd":
        k[1, 5, 2] += 37.0
    else:
        k[1, 2, 5] += 37.0
    want = c.copy()
    want[1, 2] += 1.0
    np.testing.assert_allclose(oracle.key_mean_ref(k, layout), want, atol=1e-13)


def test_smoothing_keeps_output_and_shifts_lse():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((1, 40, 4, 16))
    k = rng.standard_normal((1, 40, 2, 16)) + 3.0        # keys with a large common part
    v = rng.standard_normal((1, 40, 2, 16))
    c = oracle.key_mean_ref(k)
    o1, l1 = oracle.causal_attention_ref(q, k, v)
    o2, l2 = oracle.causal_attention_ref(q, k - c[:, None], v)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    # LSE moves by scale * q . c of the row's KV head
    hk = np.arange(4) * 2 // 4
    qc = np.einsum("bshd,bhd->bhs", q, c[:, hk]) / 4.0
    np.testing.assert_allclose(l1 - l2, qc, atol=1e-12)


def test_shifted_rotated_quantize_is_rotate_of_difference():
    rng = np.random.default_rng(11)
    s = rng.choice([-1.0, 1.0], 128)
    x = rng.standard_normal((1, 20, 2, 128)) + 5.0
    sh = oracle.key_mean_ref(x)
    codes, d, y = oracle.quantize_shifted_rotated_ref(x, sh, s)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-12)    # mean removed before the (linear) rotation
    back = oracle.e4m3fn_decode(codes) * float(d)
    big = np.abs(y) >= 2.0 ** -6 * float(d)
    assert np.all(np.abs(back - y)[big] <= 2.0 ** -4 * np.abs(y)[big])
