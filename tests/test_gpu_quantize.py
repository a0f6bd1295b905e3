"""Bit-exact parity of the HIP quantizer, clip search and prepack against the
CPU oracle, on every workload shape (row prefixes where the oracle's search
would take long; groups are independent, so a prefix is a full-width check)."""
import numpy as np
import pytest

import oracle
import synth
from helpers import (assert_bits_equal, bits16, dev, fracs_for, host, oracle_quant, require_gpu, to_dev,
                     weight)

pytestmark = pytest.mark.gpu

CASES = [
    # (workload, matrix index, rows or None, mode, G, n_fracs)
    ("tiny", 0, None, "sym", 32, 20),
    ("tiny", 0, None, "asym", 32, 20),
    ("tiny", 0, None, "asym", 32, 1),
    ("smollm2_135m_mlp", 0, None, "asym", 32, 1),
    ("smollm2_135m_mlp", 1, None, "asym", 32, 1),
    ("smollm2_135m_mlp", 1, None, "sym", 64, 11),
    ("llama8b_decode", 0, None, "asym", 128, 1),
    ("llama8b_decode", 1, None, "asym", 128, 1),
    ("gemma12b_w4a8", 0, 3072, "asym", 128, 11),
    ("gemma12b_w4a8", 1, 768, "asym", 128, 11),
    ("gemma12b_w4a8", 1, 512, "sym", 128, 11),
    ("llama70b_prefill", 0, 1024, "asym", 128, 11),
]


def _run_gpu_quant(W, mode, G, fr):
    import torch
    import w4_dequant_gemm_amd as w4
    out = w4.w4_quantize_blockwise(to_dev(W), G, mode, fr)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}-{c[3]}-g{c[4]}-n{c[5]}")
def test_quantize_bit_exact(case):
    require_gpu()
    name, idx, rows, mode, G, nf = case
    print(f"[quantize] {case}", flush=True)
    W = weight(name, idx, rows)
    ref = oracle_quant(name, idx, rows, mode, G, nf)
    out = _run_gpu_quant(W, mode, G, fracs_for(nf))
    assert_bits_equal(host(out["packed"]), ref["packed"], "packed codes")
    assert_bits_equal(bits16(out["scale"]), ref["scale"], "fp16 scales")
    if mode == "asym":
        assert_bits_equal(bits16(out["zero"]), ref["zero"], "fp16 zero points")
    assert_bits_equal(host(out["clip_idx"]), ref["clip"], "clip indices")


@pytest.mark.parametrize("mode", ["asym", "sym"])
def test_clip_search_sse_table_bit_exact(mode):
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    W = weight("gemma12b_w4a8", 0, 256)
    fr = fracs_for(11)
    ref = oracle.quantize(W, 128, mode, fracs=fr, want_sse=True)
    out = w4.w4_mse_clip_search(to_dev(W), 128, mode, fr, want_sse=True)
    torch.cuda.synchronize()
    assert_bits_equal(host(out["clip_idx"]), ref["clip"], "clip indices")
    assert_bits_equal(host(out["sse"]).view(np.uint32), ref["sse"].view(np.uint32), "candidate errors")


def test_quantize_full_70b_row_sample():
    # the full 28672 x 8192 matrix on the GPU; bit-exact on a spread of rows
    require_gpu()
    W = weight("llama70b_prefill", 0, None)
    fr = fracs_for(11)
    out = _run_gpu_quant(W, "asym", 128, fr)
    rows = np.random.default_rng(7).choice(W.shape[0], size=96, replace=False)
    rows.sort()
    ref = oracle.quantize(np.ascontiguousarray(W[rows]), 128, "asym", fracs=fr)
    assert_bits_equal(host(out["packed"])[rows], ref["packed"], "packed codes")
    assert_bits_equal(bits16(out["scale"])[rows], ref["scale"], "fp16 scales")
    assert_bits_equal(bits16(out["zero"])[rows], ref["zero"], "fp16 zero points")
    assert_bits_equal(host(out["clip_idx"])[rows], ref["clip"], "clip indices")


def test_quantize_edge_blocks():
    # degenerate and extreme groups: zeros, constants, one-signed, a single
    # outlier, tiny values with subnormal fp16 scales, ragged group counts
    require_gpu()
    rng = np.random.default_rng(3)
    rows = []
    rows.append(np.zeros(96, np.float32))
    rows.append(np.full(96, 0.3, np.float32))
    rows.append(np.full(96, -2.7, np.float32))
    rows.append(np.abs(rng.standard_normal(96)).astype(np.float32) + 1.0)       # one-signed
    r = rng.standard_normal(96).astype(np.float32) * 0.01
    r[5] = 3.0
    rows.append(r)
    rows.append((rng.standard_normal(96) * 1e-6).astype(np.float32))              # subnormal fp16 scales
    rows.append((rng.standard_normal(96) * 1e4).astype(np.float32))               # large
    rows.append(np.array([(-1.0) ** i * (i % 7) * 0.25 for i in range(96)], np.float32))  # ties
    W = np.stack(rows)
    for mode in ("asym", "sym"):
        for nf in (1, 11, 20):
            fr = fracs_for(nf)
            ref = oracle.quantize(W, 32, mode, fracs=fr)
            out = _run_gpu_quant(W, mode, 32, fr)
            assert_bits_equal(host(out["packed"]), ref["packed"], f"packed {mode} n={nf}")
            assert_bits_equal(bits16(out["scale"]), ref["scale"], f"scales {mode} n={nf}")
            if mode == "asym":
                assert_bits_equal(bits16(out["zero"]), ref["zero"], f"zeros {mode} n={nf}")
            assert_bits_equal(host(out["clip_idx"]), ref["clip"], f"clip {mode} n={nf}")


def test_quantize_empty_and_ragged():
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    W = np.zeros((0, 128), np.float32)
    out = w4.w4_quantize_blockwise(torch.zeros((0, 128), device=dev()), 32, "asym")
    torch.cuda.synchronize()
    assert out["packed"].shape == (0, 64)
    # 3 rows x 5 groups = 15 groups: far from a multiple of the 256-lane block
    W = synth.normal_matrix(12, 3, 5 * 64, 0.05)
    for mode in ("asym", "sym"):
        ref = oracle.quantize(W, 64, mode, fracs=fracs_for(11))
        out = _run_gpu_quant(W, mode, 64, fracs_for(11))
        assert_bits_equal(host(out["packed"]), ref["packed"], "packed")
        assert_bits_equal(bits16(out["scale"]), ref["scale"], "scales")


def _blocked(a: np.ndarray, per_tile: int) -> np.ndarray:
    """Host model of the header's blocked order: rows in blocks of 16 (the
    last may be shorter), items of a row in tiles of `per_tile`, each tile
    holding that many items of every row of the block in turn."""
    N, per_row = a.shape
    out = np.empty(N * per_row, a.dtype)
    for r0 in range(0, N, 16):
        nr = min(16, N - r0)
        blk = a[r0:r0 + nr].reshape(nr, per_row // per_tile, per_tile)      # [row, tile, item]
        out[r0 * per_row:(r0 + nr) * per_row] = blk.transpose(1, 0, 2).reshape(-1)
    return out


def test_prepack_layout():
    # the GPU layout is a permutation of the canonical nibbles (plus the sym
    # offset), with scale and zero interleaved, in 16-row blocks of 32-k tiles
    # -- checked against the layout the header defines, from the oracle's
    # codes; 37 rows leave a last block of 5
    require_gpu()
    import torch
    from helpers import prepack_dev
    for mode, rows in (("asym", None), ("sym", None), ("asym", 37)):
        q = oracle_quant("smollm2_135m_mlp", 0, rows, mode, 32, 1)
        pk, G = prepack_dev(q)
        torch.cuda.synchronize()
        codes = q["q"].astype(np.int64)
        u = codes if mode == "asym" else codes + 8
        N, K = u.shape
        u8 = u.reshape(N, K // 8, 8)
        want = np.zeros((N, K // 8), np.uint64)
        for i in range(4):
            want |= (u8[:, :, 2 * i].astype(np.uint64) << np.uint64(4 * i))
            want |= (u8[:, :, 2 * i + 1].astype(np.uint64) << np.uint64(16 + 4 * i))
        assert_bits_equal(host(pk["wq"]).view(np.uint32).reshape(-1), _blocked(want.astype(np.uint32), 4),
                          f"GPU-layout words ({mode}, N={N})")
        zero = q["zero"] if mode == "asym" else np.full_like(q["scale"], 0x4800)
        want_sz = q["scale"].astype(np.uint32) | (zero.astype(np.uint32) << np.uint32(16))
        assert_bits_equal(host(pk["sz"]).view(np.uint32).reshape(-1), _blocked(want_sz, 1),
                          f"scale|zero words ({mode}, N={N})")


# ------------------------------------------------------------ per-channel

PER_CHANNEL = [
    # (workload, matrix index, rows, mode, n_fracs): G = K, one group per row
    ("smollm2_135m_mlp", 0, None, "asym", 11),     # K = 576: tree padded to 1024
    ("smollm2_135m_mlp", 1, None, "sym", 11),      # K = 1536: padded to 2048
    ("llama8b_decode", 0, 512, "asym", 11),        # K = 4096
    ("llama8b_decode", 1, 256, "asym", 11),        # K = 14336: padded to 16384
    ("llama8b_decode", 1, 128, "sym", 1),
    ("llama70b_prefill", 0, 64, "asym", 11),       # K = 8192
]


@pytest.mark.parametrize("case", PER_CHANNEL, ids=lambda c: f"{c[0]}-{c[1]}-{c[3]}-n{c[4]}")
def test_per_channel_quantize_bit_exact(case):
    # gsantana.dev "Granularity: who shares a scale": per-channel is the group
    # G = K; codes, scales, zeros, clip indices and every candidate's error
    # equal the oracle's bit for bit
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    name, idx, rows, mode, nf = case
    W = weight(name, idx, rows)
    K = W.shape[1]
    print(f"[per-channel quantize] {case} K={K}", flush=True)
    fr = fracs_for(nf)
    ref = oracle.quantize(W, K, mode, fracs=fr, want_sse=True)
    out = _run_gpu_quant(W, mode, K, fr)
    assert_bits_equal(host(out["packed"]), ref["packed"], "packed codes")
    assert_bits_equal(bits16(out["scale"]), ref["scale"], "fp16 scales")
    if mode == "asym":
        assert_bits_equal(bits16(out["zero"]), ref["zero"], "fp16 zero points")
    assert_bits_equal(host(out["clip_idx"]), ref["clip"], "clip indices")
    srch = w4.w4_mse_clip_search(to_dev(W), K, mode, fr, want_sse=True)
    torch.cuda.synchronize()
    assert_bits_equal(host(srch["sse"]).view(np.uint32), ref["sse"].view(np.uint32), "candidate errors")


def test_per_channel_largest_and_smallest_rows():
    # K = 32768 (32 values per thread) and K = 96 (the tree mostly padding),
    # heavy-tailed rows with an outlier, both modes
    require_gpu()
    rng = np.random.default_rng(31)
    for K in (32768, 96, 32 * 37):
        W = (rng.standard_t(3, size=(6, K)) * 0.02).astype(np.float32)
        W[1, K // 3] = 0.9
        for mode in ("asym", "sym"):
            print(f"[per-channel quantize] K={K} {mode}", flush=True)
            fr = fracs_for(11)
            ref = oracle.quantize(W, K, mode, fracs=fr)
            out = _run_gpu_quant(W, mode, K, fr)
            assert_bits_equal(host(out["packed"]), ref["packed"], f"packed codes K={K}")
            assert_bits_equal(bits16(out["scale"]), ref["scale"], f"fp16 scales K={K}")
            assert_bits_equal(host(out["clip_idx"]), ref["clip"], f"clip indices K={K}")
