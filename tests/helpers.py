"""Shared helpers of the GPU parity tests: seeded inputs, cached oracle results,
host <-> device transfers, and the comparisons the parity bar asks for."""
from __future__ import annotations

import functools

import numpy as np
import pytest

import oracle
import synth

REL_TOL = 5e-3        # relative Frobenius error of products vs the float64 oracle


def have_gpu() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def require_gpu():
    if not have_gpu():
        pytest.skip("needs a GPU")


def dev():
    import torch
    return torch.device("cuda:0")


def to_dev(a: np.ndarray):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev())
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bf16_dev(bits: np.ndarray):
    import torch
    return to_dev(bits).view(torch.bfloat16)


def fp16_dev(bits: np.ndarray):
    import torch
    return to_dev(bits).view(torch.float16)


def bits16(t) -> np.ndarray:
    """A 16-bit device tensor (fp16 / bf16 / int16) -> uint16 bit patterns on the host."""
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


@functools.lru_cache(maxsize=16)
def weight(name: str, index: int = 0, rows: int | None = None) -> np.ndarray:
    return synth.weight(synth.WORKLOADS[name], index, rows=rows)


@functools.lru_cache(maxsize=16)
def oracle_quant(name: str, index: int, rows: int | None, mode: str, G: int, n_fracs: int):
    W = weight(name, index, rows)
    fr = fracs_for(n_fracs)
    return oracle.quantize(W, G, mode, fracs=fr)


def fracs_for(n: int) -> np.ndarray:
    if n == 1:
        return np.array([1.0], dtype=np.float32)
    if n == 11:
        return synth.FRACS_11.copy()
    return synth.fracs_linspace(n)


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    if bad.size:
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} of {got.size} differ; first at flat index {i}: "
                             f"got {got.reshape(-1)[i]!r}, want {want.reshape(-1)[i]!r}")


def prepack_dev(q):
    """Upload an oracle quantization and rearrange it with w4_prepack."""
    import w4_dequant_gemm_amd as w4
    mode = "asym" if q["zero"] is not None else "sym"
    G = q["q"].shape[1] // q["scale"].shape[1]
    packed = to_dev(q["packed"])
    scale = fp16_dev(q["scale"])
    zero = fp16_dev(q["zero"]) if q["zero"] is not None else None
    return w4.w4_prepack(packed, scale, zero, G, mode), G
