"""Pins for the oracle's NF4 comparator (gsantana.dev "Quantizing LLMs Without
Guesswork", "Weight-only methods: GPTQ, AWQ and the file formats", the NF4
paragraph): the 16 normal-quantile levels against an independent
construction with the standard library's inverse normal CDF, the storage
cost the page prints, nearest-level codes, and the double quantization of
the block scales."""
import os
from statistics import NormalDist

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nf4_bits.txt")


def _golden():
    out = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = (t.strip() for t in line.split("="))
            out[k] = float(v)
    return out


def test_levels_independent_construction():
    # the same quantiles from Python's own NormalDist (float64), rounded once
    L = oracle.nf4_levels()
    nd = NormalDist()
    delta = 0.5 * (1 - 1 / 30) + 0.5 * (1 - 1 / 32)
    pos = [nd.inv_cdf(delta + (0.5 - delta) * i / 8) for i in range(8)]
    neg = [-nd.inv_cdf(delta + (0.5 - delta) * i / 7) for i in range(7)]
    v = np.sort(np.array(pos + [0.0] + neg))
    want = (v / v.max()).astype(np.float32)
    np.testing.assert_array_equal(L.view(np.uint32), want.view(np.uint32))
    # shape of the codebook: 16 ascending levels, exact 0, 7 below, 8 above, ends at -1 and 1
    assert L.dtype == np.float32 and L.shape == (16,)
    assert np.all(np.diff(L) > 0)
    assert L[7] == 0.0 and L[0] == -1.0 and L[15] == 1.0
    assert (L < 0).sum() == 7 and (L > 0).sum() == 8
    # denser near zero, as normal quantiles are
    gaps = np.diff(L)
    assert gaps[7] < gaps[0] and gaps[7] < gaps[-1]


def test_storage_cost_printed_on_the_page():
    g = _golden()
    assert oracle.NF4_BLOCK == g["block"]
    assert 32 / oracle.NF4_BLOCK == g["scale_bits_single"]                      # one fp32 scale per block
    assert round(oracle.nf4_bits_per_weight() - 4, 3) == g["scale_bits_double"]
    assert round(oracle.nf4_bits_per_weight(), 3) == g["bits_per_weight"]


def test_levels_map_to_themselves_and_midpoints_split():
    L = oracle.nf4_levels()
    # a block holding every level exactly (absmax 1): each weight is its own level
    W = np.tile(L, 4)[None, :].astype(np.float32)
    q = oracle.nf4_quantize(W)
    np.testing.assert_array_equal(q["codes"][0], np.tile(np.arange(16), 4))
    # just above / below each midpoint: the upper / lower level
    mids = ((L[:-1].astype(np.float64) + L[1:]) / 2)
    up = np.nextafter(mids.astype(np.float32) + np.float32(1e-6), np.float32(2))
    lo = mids.astype(np.float32) - np.float32(1e-6)
    row = np.concatenate([up, lo, [1.0, -1.0]]).astype(np.float32)
    row = np.concatenate([row, np.zeros(64 - row.size, np.float32)])[None, :]
    c = oracle.nf4_quantize(row)["codes"][0]
    np.testing.assert_array_equal(c[:15], np.arange(1, 16))
    np.testing.assert_array_equal(c[15:30], np.arange(0, 15))


def test_nearest_level_error_bound_and_zero_blocks():
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((32, 256)) * 0.05).astype(np.float32)
    W[5, :64] = 0.0                                        # an all-zero block
    q = oracle.nf4_quantize(W)
    L = oracle.nf4_levels().astype(np.float64)
    amax = q["absmax"].astype(np.float64)
    x = W.reshape(-1, 64).astype(np.float64) / np.where(amax == 0, 1, amax)[:, None]
    err = np.abs(x - L[q["codes"].reshape(-1, 64)])
    assert np.all(err <= np.max(np.diff(L)) / 2 + 1e-7)
    # no level is closer than the chosen one (fp32 distances up to a rounding)
    dist = np.abs(x[:, :, None] - L[None, None, :])
    assert np.all(err <= dist.min(axis=2) + 1e-7)
    assert np.all(q["codes"][5, :64] == 7)                 # the zero level
    assert q["absmax_q"][5 * 4] == 0


def test_double_quantization_of_block_scales():
    rng = np.random.default_rng(4)
    W = (rng.standard_t(4, size=(40, 64 * 20)) * 0.02).astype(np.float32)      # 800 blocks: 3 groups + 32
    q = oracle.nf4_quantize(W)
    a = q["absmax"].astype(np.float64)
    nb = a.size
    assert q["c2"].size == (nb + 255) // 256
    c2 = np.repeat(q["c2"].astype(np.float64), 256)[:nb]
    a2 = q["absmax_q"].astype(np.float64) * c2
    assert np.all(np.abs(a - a2) <= c2 / 2 * (1 + 1e-6))              # half a step of the 8-bit code
    for g in range(q["c2"].size):
        grp = a[g * 256:(g + 1) * 256]
        assert q["absmax_q"][g * 256:(g + 1) * 256].max() == 255       # the group maximum uses the top code
        np.testing.assert_allclose(q["c2"][g], grp.max() / 255, rtol=2 ** -23)


def _normaldist_levels():
    nd = NormalDist()
    delta = 0.5 * (1 - 1 / 30) + 0.5 * (1 - 1 / 32)
    pos = [nd.inv_cdf(delta + (0.5 - delta) * i / 8) for i in range(8)]
    neg = [-nd.inv_cdf(delta + (0.5 - delta) * i / 7) for i in range(7)]
    v = np.sort(np.array(pos + [0.0] + neg))
    return (v / v.max()).astype(np.float32)


def test_constructed_blocks_dequantize_exactly():
    # Blocks built so that every stored quantity is known in advance: block b
    # holds levels L[c] times a chosen absmax a_b = q_b / 256 (q_b an integer
    # code, the largest 255, so the second-level constant is exactly
    # 255/256 / 255 = 1/256), and each block contains a level of magnitude 1
    # so that its absmax is a_b itself.  The quantizer must return the codes
    # c, the scale codes q_b and c2 = 1/256; the dequantized weight must be
    # L[c] * q_b / 256 exactly (levels from NormalDist, not the oracle); and a
    # one-hot activation row must select one dequantized column exactly.
    import synth
    L = _normaldist_levels()
    rng = np.random.default_rng(5)
    qb = np.array([255, 200, 17, 1, 128, 64, 3, 250], dtype=np.int64)
    nblk = qb.size
    codes = rng.integers(0, 16, size=(nblk, 64))
    codes[:, 0] = np.where(np.arange(nblk) % 2 == 0, 15, 0)          # level +1 or -1 in every block
    a = (qb.astype(np.float32) / np.float32(256)).astype(np.float32)
    W = (L[codes] * a[:, None]).astype(np.float32).reshape(2, 4 * 64)
    q = oracle.nf4_quantize(W)
    np.testing.assert_array_equal(q["codes"], codes.reshape(2, 4 * 64))
    np.testing.assert_array_equal(q["absmax"], a)
    np.testing.assert_array_equal(q["absmax_q"], qb.astype(np.uint8))
    assert q["c2"].tolist() == [1.0 / 256]
    want = (L[codes].astype(np.float64) * (qb[:, None] / 256.0)).reshape(2, 4 * 64)
    Wd = oracle.nf4_dequant(q["codes"], q["absmax_q"], q["c2"])
    np.testing.assert_array_equal(Wd, want)
    for k in (0, 77, 255):
        x = np.zeros((1, 4 * 64), np.float32)
        x[0, k] = 1.0
        y = oracle.nf4_gemv_ref(synth.to_bf16_bits(x), q["codes"], q["absmax_q"], q["c2"])
        np.testing.assert_array_equal(y, want[:, k])
    # a 0/1 activation row sums the chosen dequantized columns (each term exact)
    xb = (np.arange(W.shape[1]) % 7 == 0).astype(np.float32)
    y = oracle.nf4_gemv_ref(synth.to_bf16_bits(xb[None, :]), q["codes"], q["absmax_q"], q["c2"])
    np.testing.assert_allclose(y, want[:, xb > 0].sum(axis=1), rtol=1e-15, atol=0)
