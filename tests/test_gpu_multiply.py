"""Parity of the HIP row quantizer (bit-exact) and of the W4A16 / W4A8
GEMV and GEMM (relative Frobenius error <= 5e-3 against the float64 oracle
over the oracle's own quantized weights)."""
import numpy as np
import pytest

import oracle
import synth
from helpers import (REL_TOL, assert_bits_equal, bf16_dev, bits16, host, oracle_quant, prepack_dev,
                     require_gpu, to_dev)

pytestmark = pytest.mark.gpu


def _rows_cols(M, N, max_rows, max_cols, seed=0):
    rng = np.random.default_rng(seed)
    rows = np.arange(M) if M <= max_rows else np.sort(rng.choice(M, max_rows, replace=False))
    cols = np.arange(N) if N <= max_cols else np.sort(rng.choice(N, max_cols, replace=False))
    return rows.astype(np.int64), cols.astype(np.int64)


# ------------------------------------------------------------ row quantizer

def test_rowquant_bit_exact_workloads():
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    for name, K, Ms in (("gemma12b_w4a8", 3840, (1, 16, 64, 256)), ("gemma12b_w4a8", 15360, (16,)),
                        ("llama70b_prefill", 8192, (2048,))):
        wl = synth.WORKLOADS[name]
        for M in Ms:
            Xb = synth.activations_bf16_bits(wl, M, K)
            Xb[M // 2] = 0                                    # an all-zero row
            xq, xs = w4.w4_quantize_rows_e4m3(bf16_dev(Xb))
            torch.cuda.synchronize()
            rq, rs = oracle.row_quant_e4m3(Xb)
            assert_bits_equal(host(xq), rq, f"E4M3 codes {name} M={M} K={K}")
            assert_bits_equal(host(xs).view(np.uint32), rs.view(np.uint32), f"row scales {name} M={M}")
            assert np.all(host(xq)[M // 2] == 0)


def test_rowquant_every_bf16_value():
    # every finite bf16 magnitude pattern, in rows whose max fixes the scale at a
    # power of two (x / s is then exact), plus rows with arbitrary scales
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    u = np.arange(0, 0x10000, dtype=np.uint32)
    x = (u << 16).view(np.float32)
    rows = []
    for e in (-10, 0, 6):
        lim = np.float32(448.0 * 2.0 ** e)
        v = x[np.isfinite(x) & (np.abs(x) <= lim)]
        v = np.concatenate([v, [lim]])
        pad = (-len(v)) % 8
        v = np.concatenate([v, np.zeros(pad, np.float32)])
        rows.append(v)
    rng = np.random.default_rng(4)
    for _ in range(4):
        v = (rng.standard_normal(4096) * np.exp2(rng.uniform(-12, 12, 4096))).astype(np.float32)
        rows.append(v)
    K = max(len(r) for r in rows)
    K += (-K) % 8
    X = np.zeros((len(rows), K), np.float32)
    for i, r in enumerate(rows):
        X[i, :len(r)] = r
    Xb = synth.to_bf16_bits(X)
    xq, xs = w4.w4_quantize_rows_e4m3(bf16_dev(Xb))
    torch.cuda.synchronize()
    rq, rs = oracle.row_quant_e4m3(Xb)
    assert_bits_equal(host(xs).view(np.uint32), rs.view(np.uint32), "row scales")
    assert_bits_equal(host(xq), rq, "E4M3 codes")


# ------------------------------------------------------------------ products

MUL_CASES = [
    # (workload, matrix, rows of W or None, mode, G, n_fracs, M values)
    ("tiny", 0, None, "asym", 32, 20, (1, 2, 3, 16, 17, 40)),
    ("tiny", 0, None, "sym", 32, 20, (1, 5, 33)),
    ("smollm2_135m_mlp", 0, None, "asym", 32, 1, (1, 4, 16)),
    ("smollm2_135m_mlp", 1, None, "asym", 32, 1, (1, 4, 16, 64)),
    ("llama8b_decode", 0, None, "asym", 128, 1, (1, 4, 16)),
    ("llama8b_decode", 1, None, "asym", 128, 1, (1, 4, 16)),
    ("gemma12b_w4a8", 0, None, "asym", 128, 11, (1, 16, 64, 256)),
    ("gemma12b_w4a8", 1, None, "asym", 128, 11, (1, 16, 64, 256)),
]


def _x(name, M, K):
    return synth.activations_bf16_bits(synth.WORKLOADS[name], M, K)


@pytest.mark.parametrize("case", MUL_CASES, ids=lambda c: f"{c[0]}-{c[1]}-{c[3]}-g{c[4]}")
@pytest.mark.parametrize("kind", ["w4a16", "w4a8"])
def test_products_match_oracle(case, kind):
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    name, idx, rows, mode, G, nf, Ms = case
    q = oracle_quant(name, idx, rows, mode, G, nf)
    pk, G = prepack_dev(q)
    N, K = q["q"].shape
    for M in Ms:
        print(f"[{kind}] {name}[{idx}] {mode} G={G} M={M} N={N} K={K}", flush=True)
        Xb = _x(name, M, K)
        r, c = _rows_cols(M, N, 64, 1024, seed=M)
        if kind == "w4a16":
            Y = w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G)
            torch.cuda.synchronize()
            want = oracle.gemm_ref(oracle.bf16_bits_to_f64(Xb), q["packed"], q["scale"], q["zero"], G, mode,
                                   rows=r, cols=c)
        else:
            Y, xq, xs = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G)
            torch.cuda.synchronize()
            want, rq, rs = oracle.w4a8_ref(Xb, q["packed"], q["scale"], q["zero"], G, mode, rows=r, cols=c)
            assert_bits_equal(host(xq), rq, "E4M3 activations")
            assert_bits_equal(host(xs).view(np.uint32), rs.view(np.uint32), "row scales")
        got = Y.float().cpu().numpy()[np.ix_(r, c)]
        err = oracle.rel_error(want, got)
        print(f"    rel err {err:.3e}", flush=True)
        assert err <= REL_TOL, f"{kind} {name} M={M}: relative error {err:.3e} > {REL_TOL}"


@pytest.mark.parametrize("kind", ["w4a16", "w4a8"])
def test_70b_prefill_gemm_sampled(kind):
    # full 2048 x 28672 x 8192 launch; outputs checked on sampled rows and columns
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    from helpers import weight
    W = weight("llama70b_prefill", 0, None)
    fr = synth.FRACS_11
    print(f"[{kind}] 70B prefill: quantizing on the GPU", flush=True)
    quant = w4.w4_quantize_blockwise(to_dev(W), 128, "asym", fr)
    # the oracle's codes for the sampled weight rows must agree bit for bit
    rng = np.random.default_rng(11)
    cols = np.sort(rng.choice(W.shape[0], 192, replace=False)).astype(np.int64)
    qs = oracle.quantize(np.ascontiguousarray(W[cols]), 128, "asym", fracs=fr)
    torch.cuda.synchronize()
    assert_bits_equal(host(quant["packed"])[cols], qs["packed"], "packed codes (sampled rows)")
    pk = w4.w4_prepack(quant["packed"], quant["scale"], quant["zero"], 128, "asym")
    M = 2048
    Xb = _x("llama70b_prefill", M, W.shape[1])
    rows = np.sort(rng.choice(M, 48, replace=False)).astype(np.int64)
    if kind == "w4a16":
        Y = w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], 128)
        torch.cuda.synchronize()
        want = oracle.gemm_ref(oracle.bf16_bits_to_f64(Xb[rows]), qs["packed"], qs["scale"], qs["zero"], 128, "asym")
    else:
        Y, xq, xs = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], 128)
        torch.cuda.synchronize()
        want, rq, rs = oracle.w4a8_ref(Xb[rows], qs["packed"], qs["scale"], qs["zero"], 128, "asym")
        assert_bits_equal(host(xq)[rows], rq, "E4M3 activations (sampled rows)")
    got = Y.float().cpu().numpy()[np.ix_(rows, cols)]
    err = oracle.rel_error(want, got)
    print(f"    rel err {err:.3e}", flush=True)
    assert err <= REL_TOL


@pytest.mark.parametrize("kind", ["w4a16", "w4a8"])
def test_one_hot_rows_recover_dequantized_weights(kind):
    # X = e_k: W4A16 output column k is bf16(W'[n, k]) exactly, since a single
    # product of exact values is accumulated; W4A8 equals it after removing the
    # row scale (one-hot rows quantize to a single 448 code)
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    q = oracle_quant("smollm2_135m_mlp", 1, None, "asym", 32, 1)
    pk, G = prepack_dev(q)
    N, K = q["q"].shape
    Wd = oracle.dequant(q["packed"], q["scale"], q["zero"], G, "asym")
    for M in (1, 8, 16, 48):
        ks = np.linspace(0, K - 1, M).astype(np.int64)
        X = np.zeros((M, K), np.float32)
        X[np.arange(M), ks] = 1.0
        Xb = synth.to_bf16_bits(X)
        want = synth.to_bf16_bits(Wd[:, ks].T.astype(np.float32))   # exact W' rounded once to bf16
        if kind == "w4a16":
            Y = w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G)
            torch.cuda.synchronize()
            assert_bits_equal(bits16(Y), want, f"one-hot W4A16 M={M}")
        else:
            Y, xq, xs = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G)
            torch.cuda.synchronize()
            # xscale = 1/448, code 448: the product is W' * 448 * (1/448) in fp32
            got = Y.float().cpu().numpy()
            np.testing.assert_allclose(got, Wd[:, ks].T, rtol=2 ** -8, atol=0)


def test_zero_rows_and_ragged_shapes():
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    # K = 96 (3 groups of 32, less than one lane chunk), N = 200 (ragged tile)
    W = synth.normal_matrix(31, 200, 96, 0.05)
    for mode, G in (("asym", 32), ("sym", 32)):
        q = oracle.quantize(W, G, mode, fracs=synth.FRACS_11)
        pk, G2 = prepack_dev(q)
        for M in (1, 3, 7, 17, 130):
            Xb = synth.to_bf16_bits(synth.normal_matrix(M, M, 96))
            Xb[0] = 0
            Y = w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G2)
            Y8, _, _ = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G2)
            torch.cuda.synchronize()
            want = oracle.gemm_ref(oracle.bf16_bits_to_f64(Xb), q["packed"], q["scale"], q["zero"], G2, mode)
            want8, _, _ = oracle.w4a8_ref(Xb, q["packed"], q["scale"], q["zero"], G2, mode)
            assert np.all(bits16(Y)[0] & 0x7FFF == 0)           # a zero row gives zeros
            assert np.all(bits16(Y8)[0] & 0x7FFF == 0)
            if M > 1:
                assert oracle.rel_error(want[1:], Y.float().cpu().numpy()[1:]) <= REL_TOL
                assert oracle.rel_error(want8[1:], Y8.float().cpu().numpy()[1:]) <= REL_TOL


def test_w4a8_decode_row_quant_in_product():
    # one or two rows: the product kernel quantizes the bf16 rows itself; its
    # codes and scales must still be the row quantizer's, bit for bit, over
    # wide dynamic ranges, bf16 values at the clamp, and an all-zero row.
    # K = 32768 does not fit the in-kernel staging and takes the separate path.
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    rng = np.random.default_rng(11)
    for K, N in ((8192, 96), (3840, 40), (32768, 48)):
        W = synth.normal_matrix(41, N, K, 0.05)
        q = oracle.quantize(W, 128, "asym")
        pk, G = prepack_dev(q)
        allv = (np.arange(0, 0x10000, dtype=np.uint32) << 16).view(np.float32)
        lim = np.float32(448.0 * 2.0 ** -3)
        pool = allv[np.isfinite(allv) & (np.abs(allv) <= lim)]
        rows = [
            (rng.standard_normal(K) * np.exp2(rng.uniform(-14, 14, K))).astype(np.float32),
            np.concatenate([[lim], rng.choice(pool, K - 1)]).astype(np.float32),
            np.zeros(K, np.float32),
        ]
        for M, pick in ((1, (0,)), (1, (1,)), (2, (0, 1)), (2, (2, 0)), (1, (2,))):
            print(f"[w4a8 decode] K={K} N={N} M={M} rows={pick}", flush=True)
            Xb = synth.to_bf16_bits(np.stack([rows[i] for i in pick]))
            Y, xq, xs = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G)
            torch.cuda.synchronize()
            want, rq, rs = oracle.w4a8_ref(Xb, q["packed"], q["scale"], q["zero"], G, "asym")
            assert_bits_equal(host(xq), rq, f"E4M3 activations K={K} M={M}")
            assert_bits_equal(host(xs).view(np.uint32), rs.view(np.uint32), f"row scales K={K} M={M}")
            got = Y.float().cpu().numpy()
            for i, r in enumerate(pick):
                if r == 2:
                    assert np.all(bits16(Y)[i] & 0x7FFF == 0)
                else:
                    err = oracle.rel_error(want[i], got[i])
                    assert err <= REL_TOL, f"K={K} M={M} row {i}: relative error {err:.3e}"


def test_split_k_products():
    # few output tiles: the K split (fp32 partials in the workspace, summed in
    # a second kernel) on a ragged shape, with a caller workspace that holds
    # NaNs on entry, and on the 12B down shape at M = 256 (16 splits)
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    W = synth.normal_matrix(52, 200, 4096, 0.02)
    q = oracle.quantize(W, 128, "asym")
    pk, G = prepack_dev(q)
    M, K, N = 300, 4096, 200
    need = w4.w4_gemm_workspace_bytes(M, K, N)
    assert need == 2 * 8 * 256 * 256 * 4             # 2 tiles, each in 8 K ranges
    Xb = synth.to_bf16_bits(synth.normal_matrix(53, M, K))
    ws = torch.full((need // 4 + 16,), float("nan"), dtype=torch.float32, device="cuda")
    for kind in ("w4a16", "w4a8"):
        print(f"[split-K] {kind} M={M} K={K} N={N}", flush=True)
        if kind == "w4a16":
            Y = w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G, workspace=ws)
            want = oracle.gemm_ref(oracle.bf16_bits_to_f64(Xb), q["packed"], q["scale"], q["zero"], G, "asym")
        else:
            Y, xq, xs = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G, workspace=ws)
            want, rq, rs = oracle.w4a8_ref(Xb, q["packed"], q["scale"], q["zero"], G, "asym")
            torch.cuda.synchronize()
            assert_bits_equal(host(xq), rq, "E4M3 activations")
        torch.cuda.synchronize()
        err = oracle.rel_error(want, Y.float().cpu().numpy())
        assert err <= REL_TOL, f"{kind}: relative error {err:.3e}"
        # the same call again gives the same bits (fixed summation order)
        Y2 = (w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G, workspace=ws) if kind == "w4a16" else
              w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G, workspace=ws)[0])
        torch.cuda.synchronize()
        assert np.array_equal(bits16(Y), bits16(Y2))
    # too small a workspace is an error, not a slower path
    with pytest.raises(w4.W4Error):
        w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G, workspace=ws[:16])


def test_w4a8_widened_activations():
    # above 128 rows, with at least 256 output tiles, a workspace of
    # w4a8_gemm_workspace_bytes lets the row quantizer also write the E4M3
    # codes widened to bf16, and the bf16 tiled kernel runs on them (row
    # scales in its epilogue or split sum); with the required minimum the
    # E4M3 kernel runs.  Both match the oracle on sampled outputs, with the
    # same codes and scales: 258 tiles of a ragged N with the last two split
    # (workspace full of NaNs on entry), 256 whole tiles with G = 64, and the
    # 12B down shape at M = 256, whose 15 tiles take no widened copy
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    cases = [("258 tiles", synth.normal_matrix(54, 33000, 1024, 0.02), 300, 128, True),
             ("256 tiles, G = 64", synth.normal_matrix(55, 16384, 512, 0.02), 1024, 64, True),
             ("12B down", synth.weight(synth.WORKLOADS["gemma12b_w4a8"], 1), 256, 128, False)]
    for name, W, M, G, widened in cases:
        q = oracle.quantize(np.ascontiguousarray(W), G, "asym")
        pk, G = prepack_dev(q)
        N, K = W.shape
        fast, least = w4.w4a8_gemm_workspace_bytes(M, K, N), w4.w4_gemm_workspace_bytes(M, K, N)
        assert fast >= least + M * K * 2 if widened else fast == least, (name, fast, least)
        Xb = synth.to_bf16_bits(synth.normal_matrix(56, M, K))
        r, c = _rows_cols(M, N, 64, 1024, seed=M)
        r = np.unique(np.concatenate([r, np.arange(M - 4, M)]))      # the last (partial) row tile
        c = np.unique(np.concatenate([c, np.arange(N - 8, N)]))      # the ragged last column tile
        want, rq, rs = oracle.w4a8_ref(Xb, q["packed"], q["scale"], q["zero"], G, "asym", rows=r, cols=c)
        outs = []
        for label, nbytes in (("fastest", fast), ("required", least)):
            print(f"[w4a8 {label} workspace] {name} M={M} K={K} N={N} bytes={nbytes}", flush=True)
            ws = torch.full((max(nbytes, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
            Y, xq, xs = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G, workspace=ws)
            torch.cuda.synchronize()
            assert_bits_equal(host(xq), rq, "E4M3 activations")
            assert_bits_equal(host(xs).view(np.uint32), rs.view(np.uint32), "row scales")
            got = Y.float().cpu().numpy()[np.ix_(r, c)]
            err = oracle.rel_error(want, got)
            assert err <= REL_TOL, f"{label} {name}: relative error {err:.3e}"
            outs.append(got)
        # the same activations and weights: the two kernels differ only in
        # the fp32 summation order
        assert oracle.rel_error(outs[1].astype(np.float64), outs[0]) <= 1e-3


def test_split_last_round_products():
    # 258 output tiles over 256 compute units: the first 256 tiles whole, the
    # last two (rows 256..299, columns 32512..32999, ragged in both) in eight
    # K ranges each; sampled outputs cover both kinds of tile
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    M, K, N = 300, 4096, 33000
    W = synth.normal_matrix(54, N, K, 0.02)
    q = oracle.quantize(W, 128, "asym")
    del W
    pk, G = prepack_dev(q)
    Xb = synth.to_bf16_bits(synth.normal_matrix(55, M, K))
    rng = np.random.default_rng(56)
    rows = np.concatenate([np.arange(0, 8), np.arange(250, 300)]).astype(np.int64)
    cols = np.unique(np.concatenate([rng.choice(32512, 256, replace=False), np.arange(32512, N, 2)])).astype(np.int64)
    for kind in ("w4a16", "w4a8"):
        print(f"[split last round] {kind} M={M} K={K} N={N}", flush=True)
        if kind == "w4a16":
            Y = w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G)
            want = oracle.gemm_ref(oracle.bf16_bits_to_f64(Xb), q["packed"], q["scale"], q["zero"], G, "asym",
                                   rows=rows, cols=cols)
        else:
            Y, _, _ = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G)
            want, _, _ = oracle.w4a8_ref(Xb, q["packed"], q["scale"], q["zero"], G, "asym", rows=rows, cols=cols)
        torch.cuda.synchronize()
        got = Y.float().cpu().numpy()[np.ix_(rows, cols)]
        err = oracle.rel_error(want, got)
        assert err <= REL_TOL, f"{kind}: relative error {err:.3e}"
        tail = np.ix_(rows >= 256, cols >= 32512)
        err_t = oracle.rel_error(want[tail], got[tail])
        assert err_t <= REL_TOL, f"{kind} split tiles: relative error {err_t:.3e}"


def test_group_size_64():
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    q = oracle_quant("smollm2_135m_mlp", 1, None, "sym", 64, 11)
    pk, G = prepack_dev(q)
    N, K = q["q"].shape
    for M in (1, 16, 64):
        Xb = _x("smollm2_135m_mlp", M, K)
        Y = w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G)
        torch.cuda.synchronize()
        want = oracle.gemm_ref(oracle.bf16_bits_to_f64(Xb), q["packed"], q["scale"], q["zero"], G, "sym")
        assert oracle.rel_error(want, Y.float().cpu().numpy()) <= REL_TOL


def test_invalid_arguments_raise():
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    W = torch.zeros((4, 96), device="cuda:0")
    with pytest.raises(w4.W4Error):
        w4.w4_quantize_blockwise(W, 48, "asym")            # unsupported group size
    with pytest.raises(w4.W4Error):
        w4.w4_quantize_blockwise(W, 32, "asym", (0.9, 0.8))  # fracs[0] must be 1
    with pytest.raises(w4.W4Error):
        w4.w4_quantize_blockwise(torch.zeros((4, 100), device="cuda:0"), 32, "asym")  # K % G


def test_per_channel_products():
    # per-channel weights (G = K) through every product kernel: one and two
    # rows (dot form), 16 and 64 rows (MFMA with the exact correction), 256
    # rows (tiled GEMM with a K split) and K = 14336, not a power of two
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    for name, idx, rows in (("llama8b_decode", 0, 512), ("llama8b_decode", 1, 384)):
        W = synth.weight(synth.WORKLOADS[name], idx, rows=rows)
        N, K = W.shape
        q = oracle.quantize(W, K, "asym", fracs=synth.FRACS_11)
        pk, G = prepack_dev(q)
        assert G == K
        for M in (1, 2, 16, 64, 256):
            print(f"[per-channel] {name}[{idx}] N={N} K={K} M={M}", flush=True)
            Xb = _x(name, M, K)
            Y = w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G)
            Y8, xq, xs = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G)
            torch.cuda.synchronize()
            want = oracle.gemm_ref(oracle.bf16_bits_to_f64(Xb), q["packed"], q["scale"], q["zero"], G, "asym")
            want8, rq, rs = oracle.w4a8_ref(Xb, q["packed"], q["scale"], q["zero"], G, "asym")
            assert_bits_equal(host(xq), rq, "E4M3 activations")
            e16 = oracle.rel_error(want, Y.float().cpu().numpy())
            e8 = oracle.rel_error(want8, Y8.float().cpu().numpy())
            assert e16 <= REL_TOL and e8 <= REL_TOL, (M, e16, e8)


@pytest.mark.parametrize("kind", ["w4a16", "w4a8"])
def test_gate_up_products(kind):
    # gate and up projections in one pass with the activation-and-multiply
    # epilogue, against act(X Wg'^T) * (X Wu'^T) in float64: 8B-class rows
    # (gate and up are disjoint row ranges of the 8B up weight), one to 32
    # activation rows in the streaming kernel and 48 to 300 in the tiled pair
    # GEMM (64-row tiles, 128-row tiles on both sides of M = 128 and at 256,
    # and W4A16 at 300 the 256-row direct-to-LDS tiles), both activations;
    # and a ragged
    # N with symmetric G = 32 weights (the dequantizing form for more than
    # two rows, and the tiled form at 70 rows)
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    wl = synth.WORKLOADS["llama8b_decode"]
    W = synth.weight(wl, 0, rows=2048)
    cases = [(W[:1024], W[1024:], 128, "asym", (1, 2, 3, 16, 32, 48, 100, 200, 256, 300)),
             (W[:1000, :1536], W[1000:2000, :1536], 32, "sym", (1, 2, 5, 70))]
    for Wg, Wu, G, mode, Ms in cases:
        qg = oracle.quantize(np.ascontiguousarray(Wg), G, mode)
        qu = oracle.quantize(np.ascontiguousarray(Wu), G, mode)
        pg, _ = prepack_dev(qg)
        pu, _ = prepack_dev(qu)
        N, K = Wg.shape
        for act in ("silu", "gelu_tanh"):
            for M in Ms:
                print(f"[gate_up] {kind} N={N} K={K} G={G} {mode} {act} M={M}", flush=True)
                Xb = _x("llama8b_decode", M, K)
                if kind == "w4a16":
                    H = w4.w4a16_gate_up(bf16_dev(Xb), pg, pu, G, act)
                    want = oracle.gate_up_ref(Xb, qg, qu, G, mode, act)
                else:
                    H, xq, xs = w4.w4a8_gate_up(bf16_dev(Xb), pg, pu, G, act)
                    want, rq, rs = oracle.gate_up_ref(Xb, qg, qu, G, mode, act, kind="w4a8")
                    torch.cuda.synchronize()
                    assert_bits_equal(host(xq), rq, "E4M3 activations")
                    assert_bits_equal(host(xs).view(np.uint32), rs.view(np.uint32), "row scales")
                torch.cuda.synchronize()
                err = oracle.rel_error(want, H.float().cpu().numpy())
                assert err <= REL_TOL, f"{kind} {act} M={M}: relative error {err:.3e}"
    # above 32 rows the tiled form needs K to be a multiple of 64
    Wr = synth.normal_matrix(62, 64, 1568, 0.05)
    qr = oracle.quantize(Wr, 32, "asym")
    pr_, _ = prepack_dev(qr)
    with pytest.raises(w4.W4Error):
        w4.w4a16_gate_up(bf16_dev(_x("llama8b_decode", 33, 1568)), pr_, pr_, 32, "silu")
    w4.w4a16_gate_up(bf16_dev(_x("llama8b_decode", 32, 1568)), pr_, pr_, 32, "silu")


def test_mid_size_products():
    # 64 < M <= 128 with K a multiple of 64: 64 x 128 output tiles, split
    # along K into fp32 partials (a caller workspace holding NaNs on entry)
    # when the tiles are few; both kinds, every group size, per-channel
    # groups, ragged M and N, a zero row, and the 12B shapes at M = 128 on
    # sampled outputs
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    cases = [(200, 1024, 32, "asym", (65, 100)), (333, 2048, 64, "sym", (128,)),
             (130, 576, 576, "asym", (97,)), (256, 4096, 128, "asym", (128, 70))]
    for N, K, G, mode, Ms in cases:
        W = synth.normal_matrix(60 + N, N, K, 0.03)
        q = oracle.quantize(W, G, mode)
        pk, G2 = prepack_dev(q)
        for M in Ms:
            Xb = synth.to_bf16_bits(synth.normal_matrix(M + K, M, K))
            Xb[M // 2] = 0
            need = w4.w4_gemm_workspace_bytes(M, K, N)
            ws = torch.full((need // 4 + 16,), float("nan"), dtype=torch.float32, device="cuda")
            print(f"[mid] N={N} K={K} G={G} {mode} M={M} workspace={need}", flush=True)
            Y = w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G2, workspace=ws)
            Y8, xq, xs = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G2, workspace=ws)
            torch.cuda.synchronize()
            want = oracle.gemm_ref(oracle.bf16_bits_to_f64(Xb), q["packed"], q["scale"], q["zero"], G2, mode)
            want8, rq, rs = oracle.w4a8_ref(Xb, q["packed"], q["scale"], q["zero"], G2, mode)
            assert_bits_equal(host(xq), rq, "E4M3 activations")
            assert np.all(bits16(Y)[M // 2] & 0x7FFF == 0) and np.all(bits16(Y8)[M // 2] & 0x7FFF == 0)
            e16 = oracle.rel_error(want, Y.float().cpu().numpy())
            e8 = oracle.rel_error(want8, Y8.float().cpu().numpy())
            assert e16 <= REL_TOL and e8 <= REL_TOL, (N, K, G, M, e16, e8)
    # the 12B shapes at M = 128 (sampled rows and columns; K split 2 and 16 ways)
    wl = synth.WORKLOADS["gemma12b_w4a8"]
    rng = np.random.default_rng(61)
    for idx in (0, 1):
        q = oracle_quant("gemma12b_w4a8", idx, None, "asym", 128, 1)
        pk, G = prepack_dev(q)
        N, K = q["q"].shape
        M = 128
        Xb = synth.activations_bf16_bits(wl, M, K)
        rows = np.sort(rng.choice(M, 24, replace=False))
        cols = np.sort(rng.choice(N, 192, replace=False))
        print(f"[mid] 12B[{idx}] N={N} K={K} M={M}", flush=True)
        Y = w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G)
        Y8, _, _ = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G)
        torch.cuda.synchronize()
        want = oracle.gemm_ref(oracle.bf16_bits_to_f64(Xb), q["packed"], q["scale"], q["zero"], G, "asym",
                               rows=rows, cols=cols)
        want8, _, _ = oracle.w4a8_ref(Xb, q["packed"], q["scale"], q["zero"], G, "asym", rows=rows, cols=cols)
        got = Y.float().cpu().numpy()[np.ix_(rows, cols)]
        got8 = Y8.float().cpu().numpy()[np.ix_(rows, cols)]
        assert oracle.rel_error(want, got) <= REL_TOL
        assert oracle.rel_error(want8, got8) <= REL_TOL


def test_gate_up_full_8b_shapes_sampled():
    # the fused gate and up product at the 8B shapes (two 14336 x 4096
    # weights) in the launch configurations the bench times: M = 1 and 16
    # (streaming kernel) and M = 2048 (tiled pair GEMM), on sampled outputs
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    wl = synth.WORKLOADS["llama8b_decode"]
    Wg = synth.weight(wl, 0)
    Wu = synth.normal_matrix(63, *Wg.shape, 0.015)
    qg = oracle.quantize(Wg, 128, "asym")
    qu = oracle.quantize(Wu, 128, "asym")
    pg, G = prepack_dev(qg)
    pu, _ = prepack_dev(qu)
    N, K = Wg.shape
    rng = np.random.default_rng(64)
    cols = np.sort(rng.choice(N, 256, replace=False))
    for M in (1, 16, 2048):
        rows = np.arange(M) if M <= 16 else np.sort(rng.choice(M, 24, replace=False))
        Xb = synth.activations_bf16_bits(wl, M, K)
        print(f"[gate_up full] M={M}", flush=True)
        H = w4.w4a16_gate_up(bf16_dev(Xb), pg, pu, G, "silu")
        H8, xq, xs = w4.w4a8_gate_up(bf16_dev(Xb), pg, pu, G, "silu")
        torch.cuda.synchronize()
        want = oracle.gate_up_ref(Xb, qg, qu, G, "asym", "silu", rows=rows, cols=cols)
        want8, rq, rs = oracle.gate_up_ref(Xb, qg, qu, G, "asym", "silu", kind="w4a8", rows=rows, cols=cols)
        assert_bits_equal(host(xq), rq, "E4M3 activations")
        assert oracle.rel_error(want, H.float().cpu().numpy()[np.ix_(rows, cols)]) <= REL_TOL
        assert oracle.rel_error(want8, H8.float().cpu().numpy()[np.ix_(rows, cols)]) <= REL_TOL


def test_streaming_k_split_products():
    # 3..64 rows whose widest column blocks are fewer than the compute units:
    # with a workspace the streaming kernel splits K into ranges (fp32
    # partials, summed by a second kernel), without one it runs unsplit; both
    # against the oracle and against each other, on a ragged N (16 blocks of
    # 64 columns and 15 K ranges, or 32 of 32 and 8 for four row blocks),
    # W4A16 and W4A8, NaNs in the workspace on entry
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    N, K = 1000, 8192
    W = synth.normal_matrix(65, N, K, 0.02)
    q = oracle.quantize(W, 128, "asym")
    pk, G = prepack_dev(q)
    none = torch.empty((0,), dtype=torch.uint8, device="cuda")
    for M in (16, 40, 64):
        Xb = synth.to_bf16_bits(synth.normal_matrix(66 + M, M, K))
        need = w4.w4_gemm_workspace_bytes(M, K, N)
        assert need == (15 if M <= 16 else 8) * M * N * 4      # 16 blocks of 64 columns, or 32 of 32
        ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
        print(f"[k-split] M={M} N={N} K={K} workspace={need}", flush=True)
        Ys = w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G, workspace=ws)
        Yu = w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G, workspace=none)
        Y8s, xq, xs = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G, workspace=ws)
        Y8u, _, _ = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G, workspace=none)
        torch.cuda.synchronize()
        want = oracle.gemm_ref(oracle.bf16_bits_to_f64(Xb), q["packed"], q["scale"], q["zero"], G, "asym")
        want8, rq, _ = oracle.w4a8_ref(Xb, q["packed"], q["scale"], q["zero"], G, "asym")
        assert_bits_equal(host(xq), rq, "E4M3 activations")
        for got, ref, what in ((Ys, want, "w4a16 split"), (Yu, want, "w4a16 unsplit"),
                               (Y8s, want8, "w4a8 split"), (Y8u, want8, "w4a8 unsplit")):
            err = oracle.rel_error(ref, got.float().cpu().numpy())
            assert err <= REL_TOL, f"{what} M={M}: relative error {err:.3e}"
        # the two schedules differ only in the order of fp32 additions
        d = (Ys.float() - Yu.float()).abs().max().item()
        assert d <= 2 ** -6 * Yu.float().abs().max().item()
