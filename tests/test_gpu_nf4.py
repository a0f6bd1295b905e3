"""NF4 comparator on the GPU against the oracle: the quantizer bit-exact
(codes, 8-bit block scales, second-level constants) and the decode GEMV
within the product tolerance, on the 8B-class shapes and ragged ones
(gsantana.dev "Quantizing LLMs Without Guesswork", "Weight-only methods:
GPTQ, AWQ and the file formats", the NF4 paragraph)."""
import numpy as np
import pytest

import oracle
import synth
from helpers import REL_TOL, assert_bits_equal, assert_outputs_close, bf16_dev, host, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _check_gemv(want, got, xb, ref, what, rows=slice(None)):
    """Frobenius check and the per-output bound 2^-8 (|y| + sum |x W'|)."""
    err = oracle.frobenius_gap(want, got)
    assert err <= REL_TOL, f"{what}: relative error {err:.3e}"
    Wd = oracle.nf4_dequant(ref["codes"], ref["absmax_q"], ref["c2"])[rows]
    x = oracle.bf16_bits_to_f64(np.asarray(xb).reshape(1, -1))[0]
    assert_outputs_close(want, got, np.abs(Wd) @ np.abs(x), what)


@pytest.mark.parametrize("name,idx,rows", [("llama8b_decode", 0, 2048), ("llama8b_decode", 1, 512),
                                           ("smollm2_135m_mlp", 0, None), ("tiny", 0, None)])
def test_nf4_quantize_and_gemv(name, idx, rows):
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    wl = synth.WORKLOADS[name]
    W = synth.weight(wl, idx, rows=rows)
    N, K = W.shape
    print(f"[nf4] {name}[{idx}] N={N} K={K}", flush=True)
    ref = oracle.nf4_quantize(W)
    out = w4.w4_nf4_quantize(to_dev(W))
    torch.cuda.synchronize()
    assert_bits_equal(host(out["packed"]), ref["packed"], "NF4 codes")
    assert_bits_equal(host(out["absmax_q"]), ref["absmax_q"], "8-bit block scales")
    assert_bits_equal(host(out["absmax_c2"]).view(np.uint32), ref["c2"].view(np.uint32), "second-level constants")
    xb = synth.activations_bf16_bits(wl, 1, K)[0]
    y = w4.w4_nf4_gemv(bf16_dev(xb), out)
    torch.cuda.synchronize()
    want = oracle.nf4_gemv_ref(xb, ref["codes"], ref["absmax_q"], ref["c2"])
    _check_gemv(want, y.float().cpu().numpy(), xb, ref, f"NF4 GEMV {name}[{idx}]")


def test_nf4_ragged_and_zero_blocks():
    # blocks not a multiple of 256 (a partial last group), a zero row, an
    # outlier, and K not a multiple of 2048 (lanes past the row's chunks)
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    rng = np.random.default_rng(12)
    for N, K in ((37, 576), (301, 1600), (5, 64)):
        W = (rng.standard_normal((N, K)) * 0.03).astype(np.float32)
        W[0] = 0.0
        W[-1, K // 2] = 2.5
        ref = oracle.nf4_quantize(W)
        out = w4.w4_nf4_quantize(to_dev(W))
        torch.cuda.synchronize()
        assert_bits_equal(host(out["packed"]), ref["packed"], f"codes N={N} K={K}")
        assert_bits_equal(host(out["absmax_q"]), ref["absmax_q"], f"block scales N={N} K={K}")
        assert_bits_equal(host(out["absmax_c2"]).view(np.uint32), ref["c2"].view(np.uint32), f"c2 N={N} K={K}")
        xb = synth.to_bf16_bits(rng.standard_normal((1, K)).astype(np.float32))[0]
        y = w4.w4_nf4_gemv(bf16_dev(xb), out)
        torch.cuda.synchronize()
        want = oracle.nf4_gemv_ref(xb, ref["codes"], ref["absmax_q"], ref["c2"])
        got = y.float().cpu().numpy()
        assert got[0] == 0.0
        _check_gemv(want[1:], got[1:], xb, ref, f"NF4 GEMV N={N} K={K}", rows=slice(1, None))


def test_nf4_full_8b_shapes_sampled():
    # the full 8B up and down weights, quantized and multiplied in the launch
    # configuration the bench times; checked on row chunks that start and end
    # on second-level group boundaries (4 rows of K = 4096 or 8 rows of
    # K = 14336 hold whole groups of 256 blocks), so the oracle quantizes each
    # chunk as a matrix of its own with the same groups
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    wl = synth.WORKLOADS["llama8b_decode"]
    for idx in (0, 1):
        W = synth.weight(wl, idx)
        N, K = W.shape
        nb = K // 64
        span = 4 if K == 4096 else 8
        assert (span * nb) % 256 == 0
        print(f"[nf4 full] idx={idx} N={N} K={K}", flush=True)
        out = w4.w4_nf4_quantize(to_dev(W))
        xb = synth.activations_bf16_bits(wl, 1, K)[0]
        y = w4.w4_nf4_gemv(bf16_dev(xb), out)
        torch.cuda.synchronize()
        packed, aq, c2 = host(out["packed"]), host(out["absmax_q"]), host(out["absmax_c2"])
        yg = y.float().cpu().numpy()
        for r0 in (0, (N // 2 // span) * span, N - span):
            ref = oracle.nf4_quantize(W[r0:r0 + span])
            b0 = r0 * nb
            assert_bits_equal(packed[r0:r0 + span], ref["packed"], f"codes rows {r0}..")
            assert_bits_equal(aq[b0:b0 + span * nb], ref["absmax_q"], f"block scales rows {r0}..")
            g0 = b0 // 256
            assert_bits_equal(c2[g0:g0 + ref["c2"].size].view(np.uint32), ref["c2"].view(np.uint32), f"c2 rows {r0}..")
            want = oracle.nf4_gemv_ref(xb, ref["codes"], ref["absmax_q"], ref["c2"])
            _check_gemv(want, yg[r0:r0 + span], xb, ref, f"NF4 GEMV full rows {r0}..")
