"""Pins for the oracle's dequantization, per-row FP8 activation quantization and
float64 reference products."""
import numpy as np
import pytest

import synth


def _quant(orc, wl_name="smollm2_135m_mlp", rows=64, mode="asym", G=32, fr=None):
    wl = synth.WORKLOADS[wl_name]
    w = synth.weight(wl, 0, rows=rows)
    return w, orc.quantize(w, G, mode, fracs=fr)


@pytest.mark.parametrize("mode", ["sym", "asym"])
def test_dequant_matches_codes(orc, mode):
    w, r = _quant(orc, mode=mode)
    Wd = orc.dequant(r["packed"], r["scale"], r["zero"], 32, mode)
    np.testing.assert_array_equal(Wd, orc.fake_quant(w, 32, mode))


def test_one_hot_rows_recover_weights(orc):
    # X = e_k picks column k of W' exactly (float64, no rounding anywhere)
    w, r = _quant(orc, rows=48)
    N, K = w.shape
    Wd = orc.dequant(r["packed"], r["scale"], r["zero"], 32, "asym")
    ks = np.array([0, 1, 31, 32, 287, K - 1])
    X = np.zeros((len(ks), K))
    X[np.arange(len(ks)), ks] = 1.0
    Y = orc.gemm_ref(X, r["packed"], r["scale"], r["zero"], 32, "asym")
    np.testing.assert_array_equal(Y, Wd[:, ks].T)


def test_gemm_ref_matches_library_matmul(orc):
    # the float64 product agrees with NumPy's matmul on the dequantized weights
    w, r = _quant(orc, rows=96)
    Wd = orc.dequant(r["packed"], r["scale"], r["zero"], 32, "asym")
    X = synth.normal_matrix(6, 5, w.shape[1]).astype(np.float64)
    Y = orc.gemm_ref(X, r["packed"], r["scale"], r["zero"], 32, "asym")
    np.testing.assert_allclose(Y, X @ Wd.T, rtol=1e-12, atol=1e-12)
    # row / column subsets and the per-row scale
    a = np.array([0.5, 2.0, 1.0, 4.0, 0.25], dtype=np.float32)
    Ys = orc.gemm_ref(X, r["packed"], r["scale"], r["zero"], 32, "asym", a_scale=a,
                      rows=[4, 1], cols=[95, 0, 7])
    full = (X @ Wd.T) * a[:, None]
    np.testing.assert_allclose(Ys, full[[4, 1]][:, [95, 0, 7]], rtol=1e-12, atol=1e-12)


def test_row_quant_e4m3_pins(orc):
    """gowda.ai "Achievement 2": per-row scale from the row max over 448 with a
    1e-8 floor; an all-zero row stays exactly zero."""
    wl = synth.WORKLOADS["gemma12b_w4a8"]
    X = synth.activations_bf16_bits(wl, 16, 3840)
    X[3] = 0                                      # all-zero row
    xq, s = orc.row_quant_e4m3(X)
    assert s[3] == np.float32(1e-8)
    assert np.all(xq[3] == 0)
    x = orc.bf16_bits_to_f32(X).astype(np.float64)
    for m in range(16):
        if m == 3:
            continue
        i = np.argmax(np.abs(x[m]))
        assert xq[m, i] in (0x7E, 0xFE)           # the row max maps to +-448
        assert s[m] == np.float32(np.float32(np.abs(x[m]).max()) / np.float32(448.0))
    dec = orc.e4m3_to_f32(xq).astype(np.float64) * s[:, None].astype(np.float64)
    # E4M3 keeps 3 mantissa bits: relative error <= 2^-4 on normal values,
    # absolute error <= s * 2^-10 on subnormal ones
    err = np.abs(dec - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, s[:, None] * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)
    # the four outlier features dominate the row scales: every scale is
    # set by a value far above the N(0,1) bulk
    assert np.all(s[np.arange(16) != 3] * 448 > 30)


def test_row_quant_tiny_values_floor(orc):
    # rows whose max is below 448e-8 use the 1e-8 floor
    X = synth.to_bf16_bits(np.array([[1e-7, -2e-7, 0.0, 3e-7]], dtype=np.float32))
    xq, s = orc.row_quant_e4m3(X)
    assert s[0] == np.float32(1e-8)
    dec = orc.e4m3_to_f32(xq)[0] * np.float64(s[0])
    x = orc.bf16_bits_to_f32(X)[0]
    np.testing.assert_allclose(dec, x, rtol=2.0 ** -4)


def test_w4a8_reference_is_scaled_product(orc):
    w, r = _quant(orc, wl_name="gemma12b_w4a8", rows=32, G=128, fr=synth.FRACS_11)
    wl = synth.WORKLOADS["gemma12b_w4a8"]
    X = synth.activations_bf16_bits(wl, 4, w.shape[1])
    Y, xq, s = orc.w4a8_ref(X, r["packed"], r["scale"], r["zero"], 128, "asym")
    Wd = orc.dequant(r["packed"], r["scale"], r["zero"], 128, "asym")
    want = (orc.e4m3_to_f32(xq).astype(np.float64) @ Wd.T) * s[:, None]
    np.testing.assert_allclose(Y, want, rtol=1e-12, atol=1e-12)
    # and it is close to the unquantized-activation product (FP8 error only)
    Y16 = orc.gemm_ref(orc.bf16_bits_to_f64(X), r["packed"], r["scale"], r["zero"], 128, "asym")
    assert orc.frobenius_gap(Y16, Y) < 0.05


def test_gate_activations_against_library_routines(orc):
    # the oracle's gate activations pinned to torch's own (float64, CPU):
    # SiLU and the tanh form of GELU, on a wide range and near zero; the tanh
    # form stays within 1e-3 of the exact erf GELU
    import torch
    from scipy.special import erf
    x = np.concatenate([np.linspace(-30, 30, 2001), np.geomspace(1e-8, 1e-1, 50), -np.geomspace(1e-8, 1e-1, 50)])
    t = torch.from_numpy(x)
    np.testing.assert_allclose(orc.activation("silu", x), torch.nn.functional.silu(t).numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(orc.activation("gelu_tanh", x),
                               torch.nn.functional.gelu(t, approximate="tanh").numpy(), rtol=1e-13, atol=1e-14)
    exact = 0.5 * x * (1 + erf(x / np.sqrt(2)))
    assert np.max(np.abs(orc.activation("gelu_tanh", x) - exact)) < 1e-3
    with pytest.raises(ValueError):
        orc.activation("relu", x)


def test_gate_up_reference_composes_the_products(orc):
    # act(X Wg'^T) * (X Wu'^T): with the up weights equal to the gate weights
    # the result is act(y) * y for the plain product y
    W = synth.normal_matrix(60, 48, 128, 0.05)
    q = orc.quantize(W, 32, "asym")
    Xb = synth.to_bf16_bits(synth.normal_matrix(61, 3, 128))
    y = orc.gemm_ref(orc.bf16_bits_to_f64(Xb), q["packed"], q["scale"], q["zero"], 32, "asym")
    h = orc.gate_up_ref(Xb, q, q, 32, "asym", "silu")
    np.testing.assert_array_equal(h, orc.activation("silu", y) * y)
    h8, xq, s = orc.gate_up_ref(Xb, q, q, 32, "asym", "gelu_tanh", kind="w4a8")
    y8, _, _ = orc.w4a8_ref(Xb, q["packed"], q["scale"], q["zero"], 32, "asym")
    np.testing.assert_array_equal(h8, orc.activation("gelu_tanh", y8) * y8)
