"""Parity of the HIP row quantizer (bit-exact) and of the W4A16 / W4A8
GEMV and GEMM (relative Frobenius error <= 5e-3 against the float64 oracle
over the oracle's own quantized weights)."""
import numpy as np
import pytest

import oracle
import synth
from helpers import (REL_TOL, abs_products, assert_bits_equal, assert_gate_up_close, assert_outputs_close,
                     bf16_dev, bits16, check_products, host, oracle_quant, prepack_dev, require_gpu, to_dev,
                     w4a8_x64)

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
            X64 = oracle.bf16_bits_to_f64(Xb)
            want = oracle.gemm_ref(X64, q["packed"], q["scale"], q["zero"], G, mode, rows=r, cols=c)
        else:
            Y, xq, xs = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G)
            torch.cuda.synchronize()
            want, rq, rs = oracle.w4a8_ref(Xb, q["packed"], q["scale"], q["zero"], G, mode, rows=r, cols=c)
            assert_bits_equal(host(xq), rq, "E4M3 activations")
            assert_bits_equal(host(xs).view(np.uint32), rs.view(np.uint32), "row scales")
            X64 = w4a8_x64(rq, rs)
        got = Y.float().cpu().numpy()[np.ix_(r, c)]
        err = check_products(want, got, X64, q, G, mode, f"{kind} {name} M={M}", rows=r, cols=c)
        print(f"    rel err {err:.3e}", flush=True)


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
        X64 = oracle.bf16_bits_to_f64(Xb[rows])
        want = oracle.gemm_ref(X64, qs["packed"], qs["scale"], qs["zero"], 128, "asym")
    else:
        Y, xq, xs = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], 128)
        torch.cuda.synchronize()
        want, rq, rs = oracle.w4a8_ref(Xb[rows], qs["packed"], qs["scale"], qs["zero"], 128, "asym")
        assert_bits_equal(host(xq)[rows], rq, "E4M3 activations (sampled rows)")
        X64 = w4a8_x64(rq, rs)
    got = Y.float().cpu().numpy()[np.ix_(rows, cols)]
    err = check_products(want, got, X64, qs, 128, "asym", f"70B {kind}")
    print(f"    rel err {err:.3e}", flush=True)


# One-hot activation rows (x = e_k) through every product kernel.  A W4A16
# output is then bf16(W'[n, k]) exactly: the kernels round W' at most once to
# bf16 (or keep it exact) and add a single nonzero product to zeros, also
# across K splits.  W4A8 quantizes such a row to one code 448 with row scale
# fl(1/448), so its outputs are W'[n, k] up to two bf16-sized roundings.  The
# cases pick shapes whose schedule (checked through the workspace sizes)
# reaches each kernel: the streaming kernel (dot and MFMA forms, its K split),
# the 64 x 128 tiles with and without a K split (W4A16 from 33 rows; with
# groups of 128 or per-channel rows on the fp8 kernel's bf16-activation form,
# whose split rounds the ranges down), the 128 x 128 tiles (K not a
# multiple of 64), the 256 x 256 tiles whole, all split, and with only the
# last partial round split, for W4A8 also on widened activations.
ONE_HOT_CASES = [
    # label, N, K, G, mode, M, expected schedule
    ("streaming", 576, 1536, 32, "asym", (1, 8, 16, 24), "stream"),
    ("streaming G128", 1000, 8192, 128, "asym", (2, 16), "stream"),
    ("streaming one row, 8B up width", 14336, 512, 128, "asym", (1,), "stream"),
    ("streaming K split", 1000, 8192, 128, "asym", (24,), "stream-split"),
    ("64x128 split", 1536, 1024, 128, "asym", (40, 65, 100), "split"),
    ("64x128 per-channel", 700, 1024, 1024, "asym", (48, 128), "split"),
    ("64x128 whole", 32768, 256, 32, "sym", (128,), "whole"),
    ("128x128", 300, 1568, 32, "asym", (130,), "whole"),
    ("256x256 all split", 1000, 1024, 128, "asym", (300,), "split"),
    ("256x256 whole", 1000, 256, 64, "asym", (257,), "whole"),
    ("256x256 last round split", 8448, 1024, 128, "asym", (2048,), "split"),
]


@pytest.mark.parametrize("case", ONE_HOT_CASES, ids=lambda c: c[0].replace(" ", "_"))
@pytest.mark.parametrize("kind", ["w4a16", "w4a8"])
def test_one_hot_rows_recover_dequantized_weights(case, kind):
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    label, N, K, G, mode, Ms, sched = case
    W = synth.normal_matrix(70 + N, N, K, 0.02)
    q = oracle.quantize(W, G, mode)
    pk, G2 = prepack_dev(q)
    Wd = oracle.dequant(q["packed"], q["scale"], q["zero"], G2, mode)
    for M in Ms:
        need = w4.w4_gemm_workspace_bytes(M, K, N)
        if sched == "whole":
            assert need == 0, (label, M, need)
        elif sched in ("split", "stream-split"):
            assert need > 0, (label, M)
        ks = (np.arange(M, dtype=np.int64) * 7919 + 3) % K          # every group position, tails included
        X = np.zeros((M, K), np.float32)
        X[np.arange(M), ks] = 1.0
        Xb = synth.to_bf16_bits(X)
        want = Wd[:, ks].T                                           # exact float64 W'[n, k_m]
        print(f"[one-hot {kind}] {label} M={M} N={N} K={K} G={G} workspace={need}", flush=True)
        if kind == "w4a16":
            Y = w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G2)
            torch.cuda.synchronize()
            assert_bits_equal(bits16(Y), synth.to_bf16_bits(want.astype(np.float32)), f"one-hot W4A16 {label} M={M}")
        else:
            outs = []
            ws_sizes = [None]
            if M > 128 and G2 % 128 != 0 and w4.w4a8_gemm_workspace_bytes(M, K, N) > need:
                ws_sizes.append(max(need, 16))      # the E4M3 kernel instead of the widened copy
            for nb in ws_sizes:
                ws = None if nb is None else torch.empty((nb,), dtype=torch.uint8, device="cuda")
                Y, xq, xs = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G2, workspace=ws)
                torch.cuda.synchronize()
                assert np.all(host(xq)[np.arange(M), ks] == 0x7E)    # the E4M3 code of 448
                got = Y.float().cpu().numpy()
                assert_outputs_close(want, got, np.zeros_like(want), f"one-hot W4A8 {label} M={M} ws={nb}",
                                     tol=2.0 ** -8 * 1.01)
                outs.append(got)


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
                rq, rs = oracle.row_quant_e4m3(Xb)
                check_products(want[1:], Y.float().cpu().numpy()[1:], oracle.bf16_bits_to_f64(Xb)[1:], q, G2, mode,
                               f"w4a16 {mode} M={M}")
                check_products(want8[1:], Y8.float().cpu().numpy()[1:], w4a8_x64(rq, rs)[1:], q, G2, mode,
                               f"w4a8 {mode} M={M}")


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
            X64 = w4a8_x64(rq, rs)
            for i, r in enumerate(pick):
                if r == 2:
                    assert np.all(bits16(Y)[i] & 0x7FFF == 0)
                else:
                    check_products(want[i:i + 1], got[i:i + 1], X64[i:i + 1], q, G, "asym", f"K={K} M={M} row {i}")


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
            X64 = oracle.bf16_bits_to_f64(Xb)
            want = oracle.gemm_ref(X64, q["packed"], q["scale"], q["zero"], G, "asym")
        else:
            Y, xq, xs = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G, workspace=ws)
            want, rq, rs = oracle.w4a8_ref(Xb, q["packed"], q["scale"], q["zero"], G, "asym")
            torch.cuda.synchronize()
            assert_bits_equal(host(xq), rq, "E4M3 activations")
            X64 = w4a8_x64(rq, rs)
        torch.cuda.synchronize()
        check_products(want, Y.float().cpu().numpy(), X64, q, G, "asym", f"split-K {kind}")
        # the same call again gives the same bits (fixed summation order)
        Y2 = (w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G, workspace=ws) if kind == "w4a16" else
              w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G, workspace=ws)[0])
        torch.cuda.synchronize()
        assert np.array_equal(bits16(Y), bits16(Y2))
    # too small a workspace is an error, not a slower path
    with pytest.raises(w4.W4Error):
        w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G, workspace=ws[:16])


def test_w4a8_widened_activations():
    # groups of 32 or 64 (no fp8 kernel): above 128 rows, with at least 256
    # output tiles, a workspace of w4a8_gemm_workspace_bytes lets the row
    # quantizer also write the E4M3 codes widened to bf16, and the bf16 tiled
    # kernel runs on them (row scales in its epilogue or split sum); with the
    # required minimum the E4M3 kernel runs.  Both match the oracle on
    # sampled outputs, with the same codes and scales: 258 tiles of a ragged N
    # with the last two split (workspace full of NaNs on entry) and 256 whole
    # tiles.  The 12B down shape at M = 256 (groups of 128) takes the fp8
    # kernel and no widened copy.
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    cases = [("258 tiles", synth.normal_matrix(54, 33000, 1024, 0.02), 300, 64, True),
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
            check_products(want, got, w4a8_x64(rq, rs), q, G, "asym", f"{label} {name}", rows=r, cols=c)
            outs.append(got)
        # the same activations and weights: the two kernels differ only in
        # the fp32 summation order
        assert oracle.frobenius_gap(outs[1].astype(np.float64), outs[0]) <= 1e-3


# The fp8 W4A8 kernel's tile shapes, each whole and with a K split (the shape
# chooses the tile and schedule; the expected one is pinned through the
# workspace the call requires: its fp32 partial tiles).  Ragged M and N, and
# K down to two 128-k steps.
F8_TILE_CASES = [
    # label, M, K, N, (tile rows, tile columns, tiles, whole tiles, splits)
    ("256x256 whole", 1024, 256, 8200, (256, 256, 132, 132, 1)),
    ("256x256 split", 961, 8192, 2080, (256, 256, 36, 0, 7)),
    ("128x256 whole", 800, 256, 8200, (128, 256, 231, 231, 1)),
    ("128x256 split", 321, 4096, 3000, (128, 256, 36, 0, 7)),
    ("256x128 whole", 800, 256, 5000, (256, 128, 160, 160, 1)),
    ("256x128 split", 641, 8192, 2000, (256, 128, 48, 0, 5)),
    ("256x64 whole", 1024, 256, 2080, (256, 64, 132, 132, 1)),
    ("256x64 split", 129, 4096, 4000, (256, 64, 63, 0, 4)),
    ("256x64 last round split", 449, 2048, 8200, (256, 64, 258, 256, 4)),
    ("64x128 whole", 33, 256, 1000, (64, 128, 8, 8, 1)),
    ("64x128 split", 33, 1024, 1000, (64, 128, 8, 0, 2)),
    ("128x64 whole", 400, 1024, 2080, (128, 64, 132, 132, 1)),
    ("128x64 split", 65, 1024, 1056, (128, 64, 17, 0, 2)),
]


@pytest.mark.parametrize("case", F8_TILE_CASES, ids=lambda c: c[0].replace(" ", "_"))
def test_w4a8_fp8_tiles(case):
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    label, M, K, N, (bm, bn, tiles, t0, splits) = case
    assert tiles == -(-M // bm) * -(-N // bn)
    part = (tiles - t0) * splits * bm * bn * 4 if splits > 1 else 0
    W = synth.normal_matrix(60 + M, N, K, 0.02)
    q = oracle.quantize(W, 128, "asym")
    del W
    pk, G = prepack_dev(q)
    Xb = synth.to_bf16_bits(synth.normal_matrix(61 + M, M, K))
    r, c = _rows_cols(M, N, 48, 768, seed=M)
    r = np.unique(np.concatenate([r, np.arange(max(M - 5, 0), M)]))     # the last (partial) row tile
    c = np.unique(np.concatenate([c, np.arange(N - 9, N)]))              # the ragged last column tile
    want, rq, rs = oracle.w4a8_ref(Xb, q["packed"], q["scale"], q["zero"], G, "asym", rows=r, cols=c)
    X64 = w4a8_x64(rq, rs)
    # exactly the partials' bytes (NaNs on entry) are enough; fewer are refused
    ws = torch.full((max(part, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    print(f"[w4a8 fp8 tiles] {label} M={M} K={K} N={N} partial bytes={part}", flush=True)
    Y, xq, xs = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G, workspace=ws)
    torch.cuda.synchronize()
    assert_bits_equal(host(xq), rq, "E4M3 activations")
    got = Y.float().cpu().numpy()[np.ix_(r, c)]
    check_products(want, got, X64, q, G, "asym", f"fp8 tiles {label}", rows=r, cols=c)
    if part:
        with pytest.raises(w4.W4Error):
            w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G, workspace=ws.view(torch.uint8)[: part - 16])
    # the product on the row-quantized activations directly: the same bits
    Y2 = w4.w4a8_gemm_e4m3(xq, xs, pk["wq"], pk["sz"], G, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits16(Y), bits16(Y2))


def test_split_last_round_products():
    # 258 output tiles over 256 compute units: the first 256 tiles whole, the
    # last two in eight K ranges each.  Tiles are numbered column by column
    # over the two row tiles, so the split ones are the last column tile
    # (columns 32768..32999, ragged, both row tiles, the second ragged);
    # sampled outputs cover both kinds of tile
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
    cols = np.unique(np.concatenate([rng.choice(32768, 256, replace=False), np.arange(32512, N, 2)])).astype(np.int64)
    for kind in ("w4a16", "w4a8"):
        print(f"[split last round] {kind} M={M} K={K} N={N}", flush=True)
        if kind == "w4a16":
            Y = w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G)
            X64 = oracle.bf16_bits_to_f64(Xb)
            want = oracle.gemm_ref(X64, q["packed"], q["scale"], q["zero"], G, "asym", rows=rows, cols=cols)
        else:
            Y, _, _ = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G)
            want, rq, rs = oracle.w4a8_ref(Xb, q["packed"], q["scale"], q["zero"], G, "asym", rows=rows, cols=cols)
            X64 = w4a8_x64(rq, rs)
        torch.cuda.synchronize()
        got = Y.float().cpu().numpy()[np.ix_(rows, cols)]
        check_products(want, got, X64, q, G, "asym", f"split last round {kind}", rows=rows, cols=cols)
        tail = np.ix_(rows >= 0, cols >= 32768)
        err_t = oracle.frobenius_gap(want[tail], got[tail])
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
        X64 = oracle.bf16_bits_to_f64(Xb)
        want = oracle.gemm_ref(X64, q["packed"], q["scale"], q["zero"], G, "sym")
        check_products(want, Y.float().cpu().numpy(), X64, q, G, "sym", f"G=64 M={M}")


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
            X64 = oracle.bf16_bits_to_f64(Xb)
            want = oracle.gemm_ref(X64, q["packed"], q["scale"], q["zero"], G, "asym")
            want8, rq, rs = oracle.w4a8_ref(Xb, q["packed"], q["scale"], q["zero"], G, "asym")
            assert_bits_equal(host(xq), rq, "E4M3 activations")
            check_products(want, Y.float().cpu().numpy(), X64, q, G, "asym", f"per-channel w4a16 M={M}")
            check_products(want8, Y8.float().cpu().numpy(), w4a8_x64(rq, rs), q, G, "asym", f"per-channel w4a8 M={M}")


def _check_gate_up(H64, got, Xb, qg, qu, G, mode, act, kind, what, rows=None, cols=None):
    """Frobenius check and per-output bound of a fused gate and up result."""
    err = oracle.frobenius_gap(H64, got)
    assert err <= REL_TOL, f"{what}: relative error {err:.3e} > {REL_TOL}"
    if kind == "w4a16":
        X64 = oracle.bf16_bits_to_f64(Xb)
    else:
        rq, rs = oracle.row_quant_e4m3(Xb)
        X64 = w4a8_x64(rq, rs)
    r = np.arange(Xb.shape[0]) if rows is None else np.asarray(rows)
    g64 = oracle.gemm_ref(X64, qg["packed"], qg["scale"], qg["zero"], G, mode, rows=r, cols=cols)
    u64 = oracle.gemm_ref(X64, qu["packed"], qu["scale"], qu["zero"], G, mode, rows=r, cols=cols)
    ag = abs_products(X64[r], qg, G, mode, cols)
    au = abs_products(X64[r], qu, G, mode, cols)
    assert_gate_up_close(H64, got, g64, u64, ag, au, act, what)


@pytest.mark.parametrize("kind", ["w4a16", "w4a8"])
def test_gate_up_products(kind):
    # gate and up projections in one pass with the activation-and-multiply
    # epilogue, against act(X Wg'^T) * (X Wu'^T) in float64: 8B-class rows
    # (gate and up are disjoint row ranges of the 8B up weight), one to 32
    # activation rows in the streaming kernel and 48 to 300 in the tiled pair
    # GEMM (W4A16 with G = 128 up to 256 rows: the fp8 kernel's
    # bf16-activation pair form on 64-row tiles; W4A8: its fp8 pair form;
    # W4A16 at 300 the 256-row direct-to-LDS tiles), both activations;
    # and a ragged
    # N with symmetric G = 32 weights (the dequantizing form for more than
    # two rows, and the tiled form at 70 rows) and with G = 128 (the pair
    # form's 64- and 128-row tiles)
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    wl = synth.WORKLOADS["llama8b_decode"]
    W = synth.weight(wl, 0, rows=2048)
    cases = [(W[:1024], W[1024:], 128, "asym", (1, 2, 3, 16, 32, 48, 100, 200, 256, 300)),
             (W[:1000, :1536], W[1000:2000, :1536], 32, "sym", (1, 2, 5, 70)),
             (W[:1000, :1536], W[1000:2000, :1536], 128, "asym", (40, 130, 200))]
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
                _check_gate_up(want, H.float().cpu().numpy(), Xb, qg, qu, G, mode, act, kind,
                               f"{kind} {act} M={M}")
    # above 32 rows the tiled form needs K to be a multiple of 64
    Wr = synth.normal_matrix(62, 64, 1568, 0.05)
    qr = oracle.quantize(Wr, 32, "asym")
    pr_, _ = prepack_dev(qr)
    with pytest.raises(w4.W4Error):
        w4.w4a16_gate_up(bf16_dev(_x("llama8b_decode", 33, 1568)), pr_, pr_, 32, "silu")
    w4.w4a16_gate_up(bf16_dev(_x("llama8b_decode", 32, 1568)), pr_, pr_, 32, "silu")


def test_mid_size_products():
    # 64 < M <= 128 (and 33 with a workspace) with K a multiple of 64:
    # 64 x 128 output tiles (W4A16 with groups of 128 or per-channel rows on
    # the fp8 kernel's bf16-activation form), split along K into fp32
    # partials (a caller workspace holding NaNs on entry) when the tiles are
    # few; both kinds, every group size, per-channel groups, ragged M and N,
    # a zero row, and the 12B shapes at M = 128 on
    # sampled outputs
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    cases = [(200, 1024, 32, "asym", (65, 100)), (333, 2048, 64, "sym", (128,)),
             (130, 576, 576, "asym", (97,)), (256, 4096, 128, "asym", (128, 70)),
             (700, 1024, 1024, "sym", (33, 128))]
    for N, K, G, mode, Ms in cases:
        W = synth.normal_matrix(60 + N, N, K, 0.03)
        q = oracle.quantize(W, G, mode)
        pk, G2 = prepack_dev(q)
        for M in Ms:
            Xb = synth.to_bf16_bits(synth.normal_matrix(M + K, M, K))
            Xb[M // 2] = 0
            need = max(w4.w4_gemm_workspace_bytes(M, K, N), w4.w4a8_gemm_workspace_bytes(M, K, N))
            ws = torch.full((need // 4 + 16,), float("nan"), dtype=torch.float32, device="cuda")
            print(f"[mid] N={N} K={K} G={G} {mode} M={M} workspace={need}", flush=True)
            Y = w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G2, workspace=ws)
            Y8, xq, xs = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G2, workspace=ws)
            torch.cuda.synchronize()
            X64 = oracle.bf16_bits_to_f64(Xb)
            want = oracle.gemm_ref(X64, q["packed"], q["scale"], q["zero"], G2, mode)
            want8, rq, rs = oracle.w4a8_ref(Xb, q["packed"], q["scale"], q["zero"], G2, mode)
            assert_bits_equal(host(xq), rq, "E4M3 activations")
            assert np.all(bits16(Y)[M // 2] & 0x7FFF == 0) and np.all(bits16(Y8)[M // 2] & 0x7FFF == 0)
            check_products(want, Y.float().cpu().numpy(), X64, q, G2, mode, f"mid w4a16 N={N} K={K} M={M}")
            check_products(want8, Y8.float().cpu().numpy(), w4a8_x64(rq, rs), q, G2, mode, f"mid w4a8 N={N} K={K} M={M}")
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
        X64 = oracle.bf16_bits_to_f64(Xb)
        want = oracle.gemm_ref(X64, q["packed"], q["scale"], q["zero"], G, "asym", rows=rows, cols=cols)
        want8, rq, rs = oracle.w4a8_ref(Xb, q["packed"], q["scale"], q["zero"], G, "asym", rows=rows, cols=cols)
        got = Y.float().cpu().numpy()[np.ix_(rows, cols)]
        got8 = Y8.float().cpu().numpy()[np.ix_(rows, cols)]
        check_products(want, got, X64, q, G, "asym", f"mid 12B[{idx}] w4a16", rows=rows, cols=cols)
        check_products(want8, got8, w4a8_x64(rq, rs), q, G, "asym", f"mid 12B[{idx}] w4a8", rows=rows, cols=cols)


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
        _check_gate_up(want, H.float().cpu().numpy()[np.ix_(rows, cols)], Xb, qg, qu, G, "asym", "silu", "w4a16",
                       f"full 8B gate_up w4a16 M={M}", rows=rows, cols=cols)
        _check_gate_up(want8, H8.float().cpu().numpy()[np.ix_(rows, cols)], Xb, qg, qu, G, "asym", "silu", "w4a8",
                       f"full 8B gate_up w4a8 M={M}", rows=rows, cols=cols)


def test_gate_up_split_last_round():
    # W4A16 gate and up above 256 rows with the workspace of
    # w4a16_gate_up_workspace_bytes: the pair kernel's 256 x 128 output tiles
    # of the last partial round split along K (all 32 tiles of a 300 x 2000
    # product in 8 ranges; of a 600 x 14336 product, 336 tiles, the last 80 in
    # 3), NaNs in the workspace on entry; against the oracle on sampled
    # outputs (split tiles included), and against the unsplit call (an empty
    # workspace), which differs only in the fp32 order of additions
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    for (M, N, K, parts) in ((300, 2000, 4096, (32, 0, 8)), (600, 14336, 4096, (336, 256, 3))):
        Wg = synth.normal_matrix(70 + N, N, K, 0.02)
        Wu = synth.normal_matrix(71 + N, N, K, 0.015)
        qg = oracle.quantize(Wg, 128, "asym")
        qu = oracle.quantize(Wu, 128, "asym")
        del Wg, Wu
        pg, G = prepack_dev(qg)
        pu, _ = prepack_dev(qu)
        tiles, t0, splits = parts
        need = w4.w4a16_gate_up_workspace_bytes(M, K, N)
        assert need == (tiles - t0) * splits * 256 * 256 * 4, (M, N, need)
        Xb = synth.to_bf16_bits(synth.normal_matrix(72 + M, M, K))
        rng = np.random.default_rng(73)
        rows = np.unique(np.concatenate([rng.choice(M, 24, replace=False), np.arange(M - 4, M)]))
        cols = np.unique(np.concatenate([rng.choice(N, 192, replace=False), np.arange(N - 8, N)]))
        ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
        print(f"[gate_up split] M={M} N={N} K={K} workspace={need}", flush=True)
        Hs = w4.w4a16_gate_up(bf16_dev(Xb), pg, pu, G, "silu", workspace=ws)
        Hu = w4.w4a16_gate_up(bf16_dev(Xb), pg, pu, G, "silu", workspace=torch.empty((0,), dtype=torch.uint8,
                                                                                     device="cuda"))
        torch.cuda.synchronize()
        want = oracle.gate_up_ref(Xb, qg, qu, G, "asym", "silu", rows=rows, cols=cols)
        for H, what in ((Hs, "split"), (Hu, "unsplit")):
            _check_gate_up(want, H.float().cpu().numpy()[np.ix_(rows, cols)], Xb, qg, qu, G, "asym", "silu", "w4a16",
                           f"gate_up {what} M={M} N={N}", rows=rows, cols=cols)
        d = (Hs.float() - Hu.float()).abs().max().item()
        assert d <= 2 ** -6 * Hu.float().abs().max().item()


def test_streaming_k_split_products():
    # 3..64 rows whose widest column blocks are fewer than the compute units:
    # with a workspace the streaming kernel splits K into ranges (fp32
    # partials, summed by a second kernel), without one it runs unsplit; both
    # against the oracle and against each other, on a ragged N (16 blocks of
    # 64 columns and 15 K ranges), W4A16 and W4A8, NaNs in the workspace on
    # entry.  Above 32 rows W4A16 with a workspace runs on the 64 x 128 tiles
    # (their own K split) and W4A8 with groups of 128 on the fp8 kernel; the
    # streaming kernel's four-row-block split (32 blocks of 32 columns, 8 K
    # ranges) is then reached by W4A8 with groups of 64.
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    N, K = 1000, 8192
    W = synth.normal_matrix(65, N, K, 0.02)
    q = oracle.quantize(W, 128, "asym")
    pk, G = prepack_dev(q)
    none = torch.empty((0,), dtype=torch.uint8, device="cuda")
    for M in (16, 32, 40, 64):
        Xb = synth.to_bf16_bits(synth.normal_matrix(66 + M, M, K))
        need = w4.w4_gemm_workspace_bytes(M, K, N)
        if M <= 32:
            assert need == 15 * M * N * 4                       # 16 blocks of 64 columns
        else:
            assert need > 0                                     # the 64 x 128 tiles' split of K
        ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
        print(f"[k-split] M={M} N={N} K={K} workspace={need}", flush=True)
        Ys = w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G, workspace=ws)
        Yu = w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G, workspace=none)
        ws8 = torch.full((max(w4.w4a8_gemm_workspace_bytes(M, K, N), need) // 4,), float("nan"),
                         dtype=torch.float32, device="cuda")
        Y8s, xq, xs = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G, workspace=ws8)
        if M <= 32:
            Y8u, _, _ = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G, workspace=none)
        else:
            with pytest.raises(w4.W4Error):       # the fp8 kernel's split needs its partials
                w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G, workspace=none)
            Y8u = Y8s
        torch.cuda.synchronize()
        X64 = oracle.bf16_bits_to_f64(Xb)
        want = oracle.gemm_ref(X64, q["packed"], q["scale"], q["zero"], G, "asym")
        want8, rq, rs = oracle.w4a8_ref(Xb, q["packed"], q["scale"], q["zero"], G, "asym")
        assert_bits_equal(host(xq), rq, "E4M3 activations")
        X8 = w4a8_x64(rq, rs)
        for got, ref, xx, what in ((Ys, want, X64, "w4a16 split"), (Yu, want, X64, "w4a16 unsplit"),
                                   (Y8s, want8, X8, "w4a8 split"), (Y8u, want8, X8, "w4a8 unsplit")):
            check_products(ref, got.float().cpu().numpy(), xx, q, G, "asym", f"{what} M={M}")
        # the two schedules differ only in the order of fp32 additions
        d = (Ys.float() - Yu.float()).abs().max().item()
        assert d <= 2 ** -6 * Yu.float().abs().max().item()
        if M > 32:
            # W4A8, groups of 64: the streaming kernel's four row blocks, K
            # split 8 ways with the workspace (32 blocks of 32 columns)
            q64 = oracle.quantize(W, 64, "asym")
            pk64, _ = prepack_dev(q64)
            need64 = w4.w4a8_gemm_workspace_bytes(M, K, N)
            assert need64 >= 8 * M * N * 4                      # (and the fp8 schedule's for groups of 128)
            ws64 = torch.full((need64 // 4,), float("nan"), dtype=torch.float32, device="cuda")
            Y64s, _, _ = w4.w4a8_gemm(bf16_dev(Xb), pk64["wq"], pk64["sz"], 64, workspace=ws64)
            Y64u, _, _ = w4.w4a8_gemm(bf16_dev(Xb), pk64["wq"], pk64["sz"], 64, workspace=none)
            torch.cuda.synchronize()
            want64, _, _ = oracle.w4a8_ref(Xb, q64["packed"], q64["scale"], q64["zero"], 64, "asym")
            for got, what in ((Y64s, "w4a8 G=64 split"), (Y64u, "w4a8 G=64 unsplit")):
                check_products(want64, got.float().cpu().numpy(), X8, q64, 64, "asym", f"{what} M={M}")


def test_zero_points_outside_the_code_range():
    # Groups whose values are all of one sign have a zero point outside
    # 0..15 (the range [lo, hi] excludes 0): all-positive groups get z < 0,
    # all-negative ones z > 15.  Every product path must still use the exact
    # W' = (u - z) s; the fp8 W4A8 kernel restores the part of z beyond its
    # clamped operand separately.  Rows at 300 take the 256 x 256 tiles
    # (W4A8: the fp8 kernel), 24 the streaming kernel, 40 and 100 the 64 x 128
    # tiles (W4A8: the fp8 kernel).
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    N, K = 600, 2048
    W = synth.normal_matrix(80, N, K, 0.02)
    W[:, 128:256] += 1.0                     # group 1 of every row: all positive
    W[::7, 1024:1152] -= 0.5                 # group 8 of every 7th row: all negative
    q = oracle.quantize(W, 128, "asym")
    z = oracle.f16_bits_to_f32(q["zero"])
    assert (z < 0).sum() >= N and (z > 15).sum() >= N // 7
    pk, G = prepack_dev(q)
    for M in (300, 24, 40, 100):
        print(f"[zero outside 0..15] M={M}", flush=True)
        Xb = synth.to_bf16_bits(synth.normal_matrix(81 + M, M, K))
        Y = w4.w4a16_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G)
        Y8, xq, xs = w4.w4a8_gemm(bf16_dev(Xb), pk["wq"], pk["sz"], G)
        torch.cuda.synchronize()
        X64 = oracle.bf16_bits_to_f64(Xb)
        want = oracle.gemm_ref(X64, q["packed"], q["scale"], q["zero"], G, "asym")
        want8, rq, rs = oracle.w4a8_ref(Xb, q["packed"], q["scale"], q["zero"], G, "asym")
        assert_bits_equal(host(xq), rq, "E4M3 activations")
        check_products(want, Y.float().cpu().numpy(), X64, q, G, "asym", f"w4a16 M={M}")
        check_products(want8, Y8.float().cpu().numpy(), w4a8_x64(rq, rs), q, G, "asym", f"w4a8 M={M}")


def test_gate_up_emits_the_down_projection_input():
    # w4a8_gate_up with hq: the E4M3 rows of H and their scales, formed from
    # the row maxima the pass leaves behind, must be bit for bit the oracle's
    # row quantization of the bf16 H the same call returns; the down
    # projection on them (w4a8_gemm_e4m3) must equal w4a8_gemm on H bit for
    # bit and the oracle within the product bounds.  Streaming pass (1, 2,
    # 16, 32 rows: 16-column tiles) and tiled pass (48, 300 rows: 128-column
    # tiles), a zero activation row (H row 0: scale 1e-8, codes 0), a ragged N.
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    wl = synth.WORKLOADS["llama8b_decode"]
    W = synth.weight(wl, 0, rows=2 * 1056)
    for N in (1024, 1056, 12416):
        # N = 1056 leaves a partial last 128-column tile (the tiled pass) and
        # gives the down weight [640, N] groups of 32; rows of H of 12416
        # values take the row quantizer's 1024-thread blocks
        if N > 1056:
            qg = oracle.quantize(synth.weight(wl, 0, rows=N), 128, "asym")
            qu = oracle.quantize(synth.normal_matrix(86, N, W.shape[1], 0.02), 128, "asym")
        else:
            qg = oracle.quantize(np.ascontiguousarray(W[:N]), 128, "asym")
            qu = oracle.quantize(np.ascontiguousarray(W[N:2 * N]), 128, "asym")
        Gd = 128 if N % 128 == 0 else 32
        qd = oracle.quantize(synth.normal_matrix(85, 640, N, 0.03), Gd, "asym")
        pg, _ = prepack_dev(qg)
        pu, _ = prepack_dev(qu)
        pd, _ = prepack_dev(qd)
        K = W.shape[1]
        for M in ((1, 2, 16, 32, 48, 300) if N <= 1056 else (1, 48)):
            print(f"[gate_up e4m3] N={N} M={M}", flush=True)
            Xb = _x("llama8b_decode", M, K)
            Xb[0] = 0
            H, xq, xs, hq, hs = w4.w4a8_gate_up(bf16_dev(Xb), pg, pu, 128, "silu", emit_e4m3=True)
            torch.cuda.synchronize()
            Hb = bits16(H)
            rq, rs = oracle.row_quant_e4m3(Hb)
            assert_bits_equal(host(hs).view(np.uint32), rs.view(np.uint32), f"H row scales M={M}")
            assert_bits_equal(host(hq), rq, f"H E4M3 codes M={M}")
            assert host(hs)[0] == np.float32(1e-8) and np.all(host(hq)[0] == 0)
            # the down projection on the emitted codes
            Yd = w4.w4a8_gemm_e4m3(hq, hs, pd["wq"], pd["sz"], Gd)
            Yr, _, _ = w4.w4a8_gemm(H, pd["wq"], pd["sz"], Gd)
            torch.cuda.synchronize()
            assert np.array_equal(bits16(Yd), bits16(Yr)), f"w4a8_gemm_e4m3 differs from w4a8_gemm M={M}"
            want, _, _ = oracle.w4a8_ref(Hb, qd["packed"], qd["scale"], qd["zero"], Gd, "asym")
            if M > 1:
                check_products(want[1:], Yd.float().cpu().numpy()[1:], w4a8_x64(rq, rs)[1:], qd, Gd, "asym",
                               f"down on emitted codes M={M}")
