"""Pins of the oracle's e4m3fn and bf16 codecs (CPU only)."""
import os

import numpy as np
import pytest
import torch

from oracle import codecs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _facts():
    rows = []
    with open(os.path.join(GOLD, "e4m3fn_facts.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            v, c = line.split()[:2]
            rows.append((float(v), int(c, 16)))
    return rows


@pytest.mark.parametrize("value,code", _facts())
def test_e4m3fn_page_facts(value, code):
    assert int(codecs.e4m3fn_encode(np.array([value]))[0]) == code
    if code != 0x00 or value == 0.0:
        if value != 2.0 ** -10:
            assert codecs.e4m3fn_decode(np.array([code], np.uint8))[0] == value


def test_e4m3fn_plus8_per_doubling():
    # every normal code c (exponent field 1..14, also 15 below NaN) doubles at c + 8
    for c in range(0x08, 0x7E - 8 + 1):
        a, b = codecs.e4m3fn_decode(np.array([c, c + 8], np.uint8))
        assert b == 2 * a, hex(c)


def test_e4m3fn_subnormals_and_underflow():
    sub = codecs.e4m3fn_decode(np.arange(8, dtype=np.uint8))
    assert np.array_equal(sub, np.arange(8) * 2.0 ** -9)
    assert codecs.e4m3fn_decode(np.array([0x08], np.uint8))[0] == 2.0 ** -6
    tiny = np.array([2.0 ** -11, 2.0 ** -10 * 0.999, 2.0 ** -10])
    assert np.all(codecs.e4m3fn_encode(tiny) == 0)
    assert codecs.e4m3fn_encode(np.array([2.0 ** -10 * 1.001]))[0] == 0x01


def test_e4m3fn_roundtrip_and_ties():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = codecs.e4m3fn_decode(codes)
    back = codecs.e4m3fn_encode(vals)
    # -0.0 keeps its sign bit: 0x80 -> 0x80
    assert np.array_equal(back, codes)
    # midpoints between neighbours go to the even code
    pos = codecs.e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    got = codecs.e4m3fn_encode(mids).astype(int)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, want)
    assert codecs.e4m3fn_decode(np.array([0x7F], np.uint8))[0] != codecs.e4m3fn_decode(np.array([0x7F], np.uint8))[0]


def test_e4m3fn_matches_torch_cast():
    # torch's CPU float8_e4m3fn cast is an independent RNE implementation
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000) * 10,
        rng.uniform(-448, 448, 100000),
        rng.standard_normal(100000) * 2.0 ** -8,
    ]).astype(np.float32)
    pos = codecs.e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))
    x = np.concatenate([x, ((pos[:-1] + pos[1:]) / 2).astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codecs.e4m3fn_encode(x), ref)


def test_bf16_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(300000).astype(np.float32),
                        (rng.standard_normal(100000) * 1e-30).astype(np.float32),
                        (rng.standard_normal(100000) * 1e30).astype(np.float32)])
    # exact ties: low 16 bits == 0x8000
    u = rng.integers(0, 2 ** 32, 50000, dtype=np.uint64).astype(np.uint32)
    u = (u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    u = u[((u >> 23) & 0xFF) < 0xFF]
    x = np.concatenate([x, u.view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(codecs.bf16_encode_bits(x), ref)
    assert np.array_equal(codecs.bf16_decode(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())
