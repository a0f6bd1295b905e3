"""Pins for the oracle's number-format conversions.

Each conversion is checked against an independent library implementation
(NumPy's binary16 cast, torch's float8_e4m3fn cast) and against the format
limits the gsantana.dev page prints ("Number formats: what the bits buy").
"""
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split("=", 1)
            out[k.strip()] = v.strip()
    return out


def test_fp16_encoder_matches_numpy_on_every_fp16_neighbourhood(orc):
    # every binary16 value, the midpoints between neighbours (the RNE ties),
    # and one ulp (binary32) either side of each midpoint
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    v = h.view(np.float16).astype(np.float32)
    nxt = (h + 1).view(np.float16).astype(np.float32)
    mid = ((v.astype(np.float64) + nxt.astype(np.float64)) / 2).astype(np.float32)
    xs = np.concatenate([v, mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(np.inf))])
    xs = np.concatenate([xs, -xs])
    with np.errstate(over="ignore"):
        want = xs.astype(np.float16).view(np.uint16)
    got = orc.f32_to_f16_bits(xs)
    np.testing.assert_array_equal(got, want)


def test_fp16_encoder_matches_numpy_random(orc):
    rng = np.random.default_rng(5)
    xs = (rng.standard_normal(200_000) * np.exp2(rng.uniform(-30, 18, 200_000))).astype(np.float32)
    with np.errstate(over="ignore"):
        want = xs.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(orc.f32_to_f16_bits(xs), want)


def test_fp16_decoder_round_trip(orc):
    h = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    fin = (h & 0x7C00) != 0x7C00
    got = orc.f16_bits_to_f32(h[fin])
    want = h[fin].view(np.float16).astype(np.float32)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


def test_fp16_limits(orc):
    g = _golden("format_limits.txt")
    fmax = float(g["fp16_max"])
    assert orc.f16_bits_to_f32(orc.f32_to_f16_bits([fmax]))[0] == fmax
    assert orc.f32_to_f16_bits([65520.0])[0] == 0x7C00       # rounds to infinity


def test_e4m3_decoder_matches_torch(orc):
    b = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = orc.e4m3_to_f32(b)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], want[~nan])
    g = _golden("format_limits.txt")
    assert np.nanmax(got) == float(g["e4m3_max"])
    assert not np.isinf(got).any()                            # no infinities


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -3, 2.0 ** 5, 0.7071])
def test_e4m3_encoder_matches_torch_on_all_bf16(orc, scale):
    # every finite bf16 value, scaled, is encoded exactly as torch's RNE cast
    # does wherever that cast stays finite (|x| <= 464, the midpoint between
    # 448 and the next binade step); beyond it the oracle saturates to +-448
    # (torch's cast overflows to NaN there).
    u = np.arange(0, 0x10000, dtype=np.uint32)
    x = (u << 16).view(np.float32)
    with np.errstate(over="ignore"):
        x = x[np.isfinite(x)] * np.float32(scale)
    x = x[np.isfinite(x)].astype(np.float32)
    got = orc.f32_to_e4m3(x)
    inr = np.abs(x) <= 464
    want = torch.from_numpy(x[inr]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got[inr], want)
    big = ~inr
    assert np.all((got[big] & 0x7F) == 0x7E)
    assert np.all((got[big] >> 7) == (x[big] < 0))


def test_bf16_decoder(orc):
    u = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    got = orc.bf16_bits_to_f32(u)
    want = torch.from_numpy(u.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    fin = np.isfinite(want)
    np.testing.assert_array_equal(got[fin], want[fin])
