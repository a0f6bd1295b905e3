"""HIP graph capture of the library's launches.  A serving loop captures its
decode step once and replays it; the library records nothing but kernel
launches into a capture (no allocation, no memset, no copy), so a replay must
reproduce, bit for bit, what the same calls give when issued eagerly.  Each
case is captured once and replayed three times on new inputs written eagerly
before each replay, with the eager calls run (and the stream synchronised)
between the replays."""
import numpy as np
import pytest

import synth
from helpers import bf16_dev, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _weights(w4, seed, N, K, G=128):
    W = synth.normal_matrix(seed, N, K, 0.02)
    q = w4.w4_quantize_blockwise(to_dev(W), G, "asym")
    return w4.w4_prepack(q["packed"], q["scale"], q["zero"], G, "asym")


def _replays_match_eager(torch, label, fn, inputs, outputs, seed):
    """Capture fn, then three times: new inputs (eager), replay, compare with fn run eagerly."""
    print(f"[graph] {label}", flush=True)
    fn()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda:0").manual_seed(seed)
    for rep in range(3):
        for x in inputs:
            x.copy_(torch.randn(x.shape, generator=gen, device="cuda:0").to(x.dtype))
        for o in outputs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outputs]
        fn()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, outputs)):
            assert torch.equal(a, b), f"{label}: replay {rep} output {i} differs from the eager call"


@pytest.mark.parametrize("M", [1, 2, 16, 64, 300])
def test_products_replay_from_a_graph(M):
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    N, K = 3072, 4096
    pk = _weights(w4, 700 + M, N, K)
    pk2 = _weights(w4, 800 + M, N, K)
    X = bf16_dev(synth.to_bf16_bits(synth.normal_matrix(900 + M, M, K)))
    Y16 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    Y8 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    xq = torch.empty((M, K), dtype=torch.uint8, device="cuda:0")
    xs = torch.empty((M,), dtype=torch.float32, device="cuda:0")
    ws16 = torch.empty((max(w4.w4_gemm_workspace_bytes(M, K, N), 16),), dtype=torch.uint8, device="cuda:0")
    ws8 = torch.empty((max(w4.w4a8_gemm_workspace_bytes(M, K, N), 16),), dtype=torch.uint8, device="cuda:0")
    H = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    wsg = torch.empty((max(w4.w4a16_gate_up_workspace_bytes(M, K, N), 16),), dtype=torch.uint8, device="cuda:0")

    def fn():
        # two W4A16 calls with and without the split workspace, W4A8 with its
        # row quantization, the fused gate + up
        w4.w4a16_gemm(X, pk["wq"], pk["sz"], 128, Y=Y16, workspace=ws16)
        w4.w4a8_gemm(X, pk2["wq"], pk2["sz"], 128, Y=Y8, xq=xq, xscale=xs, workspace=ws8)
        w4.w4a16_gate_up(X, pk, pk2, 128, "silu", H=H, workspace=wsg)
    _replays_match_eager(torch, f"products M={M}", fn, [X], [Y16, Y8, xq, xs, H], 31 + M)


def test_decode_step_and_nf4_replay_from_a_graph():
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    # a short decode step: two layers of up + down at M = 1, then the NF4 GEMV
    Nu, Ku = 2048, 1024
    ups = [_weights(w4, 40 + i, Nu, Ku) for i in range(2)]
    downs = [_weights(w4, 50 + i, Ku, Nu) for i in range(2)]
    xu = bf16_dev(synth.to_bf16_bits(synth.normal_matrix(60, 1, Ku)))
    xd = bf16_dev(synth.to_bf16_bits(synth.normal_matrix(61, 1, Nu)))
    yu = torch.empty((1, Nu), dtype=torch.bfloat16, device="cuda:0")
    yd = torch.empty((1, Ku), dtype=torch.bfloat16, device="cuda:0")
    nf = w4.w4_nf4_quantize(to_dev(synth.normal_matrix(62, Nu, Ku, 0.02)))
    yn = torch.empty((Nu,), dtype=torch.bfloat16, device="cuda:0")

    def fn():
        for i in range(2):
            w4.w4a16_gemm(xu, ups[i]["wq"], ups[i]["sz"], 128, Y=yu)
            w4.w4a16_gemm(xd, downs[i]["wq"], downs[i]["sz"], 128, Y=yd)
        w4.w4_nf4_gemv(xu.view(-1), nf, y=yn)
    _replays_match_eager(torch, "decode step + NF4", fn, [xu, xd], [yu, yd, yn], 7)
    assert np.isfinite(yu.float().cpu().numpy()).all()
