"""Load-time prepack from the portable file form (gowda.ai "LLM fast
inference", "MSE clipping", last paragraph; "What the WMT26 paper finds"):
weights quantized on the GPU, saved, loaded and rearranged into the GPU
layout give the same layout words and the same products, bit for bit, as
the weights that never left the GPU."""
import numpy as np
import pytest

import synth
from helpers import bf16_dev, bits16, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,idx,mode,G,n", [("smollm2_135m_mlp", 1, "asym", 32, 11),
                                               ("llama8b_decode", 0, "asym", 128, 1),
                                               ("tiny", 0, "sym", 64, 20)])
def test_load_time_prepack_matches(tmp_path, name, idx, mode, G, n):
    require_gpu()
    import torch
    import w4_dequant_gemm_amd as w4
    wl = synth.WORKLOADS[name]
    W = torch.from_numpy(synth.weight(wl, idx)).cuda()
    fr = tuple(float(f) for f in (synth.FRACS_11 if n == 11 else (synth.fracs_linspace(n) if n > 1 else (1.0,))))
    q = w4.w4_quantize_blockwise(W, G, mode, fr, want_clip=True)
    direct = w4.w4_prepack(q["packed"], q["scale"], q["zero"], G, mode)
    path = str(tmp_path / f"{name}.w4q")
    w4.w4_portable_save(path, q["packed"], q["scale"], q["zero"], G, mode, fr, clip_idx=q["clip_idx"])
    loaded = w4.w4_portable_load(path, device="cuda")
    torch.cuda.synchronize()
    print(f"[portable] {name}[{idx}] {mode} G={G}: {loaded['payload_bytes']} payload bytes", flush=True)
    for key in ("wq", "sz"):
        assert torch.equal(loaded[key], direct[key]), key
    assert torch.equal(loaded["clip_idx"], q["clip_idx"])
    N, K = W.shape
    for M in (1, 16):
        X = bf16_dev(synth.activations_bf16_bits(wl, M, K))
        Y0 = w4.w4a16_gemm(X, direct["wq"], direct["sz"], G)
        Y1 = w4.w4a16_gemm(X, loaded["wq"], loaded["sz"], G)
        torch.cuda.synchronize()
        assert np.array_equal(bits16(Y0), bits16(Y1))
