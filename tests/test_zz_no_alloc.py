"""w4a16_gemm_noalloc, the product form for callers that cannot allocate
device memory: its K-split partial sums live in an array the library holds
on each GPU.  Called through the C ABI, it must give the same bits as
w4a16_gemm with a caller workspace (same kernels, same split schedule), on
two calls in a row whose second is smaller, and match the oracle on sampled
outputs."""
import numpy as np
import pytest

import oracle
import synth
from helpers import bf16_dev, bits16, check_products, require_gpu, to_dev

pytestmark = pytest.mark.gpu

# (label, N, K, M): a 16-way K split of 15 output tiles of 256 x 256 (60 MiB
# of partial tiles), then a smaller 64 x 128-tile split, then the same tiles
# at 40 rows (below 65 rows they take the product only when the scratch
# holds their split), then the streaming kernel's optional split, then a
# shape with no split at all
CASES = [("12B down M=256", 3840, 15360, 256), ("mid split", 1536, 1024, 100),
         ("mid split at 40 rows", 1000, 8192, 40), ("streaming split", 1000, 8192, 24),
         ("one row", 1000, 8192, 1)]


def test_noalloc_matches_the_workspace_entry_point():
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    assert w4.lib().w4a16_gemm_noalloc is not None
    prev = None
    for label, N, K, M in CASES:
        W = synth.normal_matrix(90 + M, N, K, 0.02)
        qd = w4.w4_quantize_blockwise(to_dev(W), 128, "asym")
        pk = w4.w4_prepack(qd["packed"], qd["scale"], qd["zero"], 128, "asym")
        Xb = synth.to_bf16_bits(synth.normal_matrix(91 + M, M, K))
        X = bf16_dev(Xb)
        need = w4.w4_gemm_workspace_bytes(M, K, N)
        print(f"[noalloc] {label} M={M} N={N} K={K} split workspace={need}", flush=True)
        assert need <= 64 << 20
        if prev is not None:
            assert M * N < prev                 # each call smaller than the one before
        prev = M * N
        ws = torch.full((max(need, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
        Yw = w4.w4a16_gemm(X, pk["wq"], pk["sz"], 128, workspace=ws)
        Yn = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        w4.w4a16_gemm_noalloc(X, pk["wq"], pk["sz"], 128, Yn)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        assert np.array_equal(bits16(Yn), bits16(Yw)), f"{label}: noalloc differs from w4a16_gemm"
        # and the oracle on sampled outputs (codes from the GPU quantizer,
        # checked against the oracle's on the sampled weight rows)
        rng = np.random.default_rng(M)
        rows = np.sort(rng.choice(M, min(M, 32), replace=False))
        cols = np.sort(rng.choice(N, 128, replace=False))
        qs = oracle.quantize(np.ascontiguousarray(W[cols]), 128, "asym")
        assert np.array_equal(qd["packed"].cpu().numpy()[cols], qs["packed"])
        X64 = oracle.bf16_bits_to_f64(Xb)[rows]
        want = oracle.gemm_ref(X64, qs["packed"], qs["scale"], qs["zero"], 128, "asym")
        check_products(want, Yn.float().cpu().numpy()[np.ix_(rows, cols)], X64, qs, 128, "asym",
                       f"noalloc {label}")
