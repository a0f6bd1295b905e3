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


# ------------------------------------------------ per-output error bounds
#
# Every product output is also checked on its own, not only through the
# Frobenius norm of all of them.  With fp32 accumulation of K terms, weights
# rounded at most once to bf16 (relative 2^-9) and one bf16 rounding of the
# result (relative 2^-9), an output differs from the float64 product y64 by
# at most
#     2^-9 |y64| + (2^-9 + K 2^-24 + small) sum_k |x_k W'_nk|,
# which for K <= 16384 is below  2^-8 (|y64| + sum_k |x_k W'_nk|).  The sum of
# magnitudes is taken in float64 from the oracle's dequantized weights.

ELEM_TOL = 2.0 ** -8


def abs_products(X64: np.ndarray, q: dict, G: int, mode: str, cols=None) -> np.ndarray:
    """float64 sum_k |x[m, k]| |W'[n, k]| for the rows of ``X64`` and the weight
    rows ``cols`` (all when None) of an oracle quantization ``q``."""
    sel = slice(None) if cols is None else np.asarray(cols)
    zero = q["zero"][sel] if q["zero"] is not None else None
    Wd = oracle.dequant(q["packed"][sel], q["scale"][sel], zero, G, mode)
    return np.abs(np.asarray(X64, dtype=np.float64)) @ np.abs(Wd).T


def w4a8_x64(xq: np.ndarray, xs: np.ndarray) -> np.ndarray:
    """The W4A8 operand as float64: decoded E4M3 codes times the row scale."""
    return oracle.e4m3_to_f32(xq).astype(np.float64) * xs.astype(np.float64)[:, None]


def assert_outputs_close(want: np.ndarray, got: np.ndarray, absdot: np.ndarray, what: str,
                         tol: float = ELEM_TOL):
    """|got - want| <= tol (|want| + absdot) for every output (float64 want)."""
    want = np.asarray(want, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == want.shape == absdot.shape, (what, got.shape, want.shape, absdot.shape)
    bound = tol * (np.abs(want) + absdot)
    bad = ~(np.abs(got - want) <= bound)
    if bad.any():
        idx = np.argwhere(bad)[0]
        i = tuple(int(v) for v in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outputs outside the per-output bound; "
                             f"first at {i}: got {got[i]!r}, want {want[i]!r}, bound {bound[i]!r}")


def check_products(want, got, X64, q, G, mode, what, rows=None, cols=None):
    """The two parity checks of a product: relative Frobenius error <= REL_TOL
    over the compared outputs, and the per-output bound on each of them."""
    err = oracle.frobenius_gap(want, got)
    assert err <= REL_TOL, f"{what}: relative error {err:.3e} > {REL_TOL}"
    Xr = X64 if rows is None else np.asarray(X64)[np.asarray(rows)]
    assert_outputs_close(want, got, abs_products(Xr, q, G, mode, cols), what)
    return err


def assert_gate_up_close(H64, got, g64, u64, ag, au, act: str, what: str):
    """Per-output bound of the fused gate and up product H = act(g) * u.

    g and u each obey the product bound (|dg| <= 2^-8 (|g| + sum |x Wg'|)); the
    activation's slope is at most 1.2 in magnitude for SiLU and the tanh form
    of GELU; the fp32 activation itself and the final bf16 rounding add at
    most 2^-8 |H| + 1e-6 |act(g) u|."""
    g64 = np.asarray(g64, np.float64)
    u64 = np.asarray(u64, np.float64)
    dg = ELEM_TOL * (np.abs(g64) + ag)
    du = ELEM_TOL * (np.abs(u64) + au)
    a = np.abs(oracle.activation(act, g64))
    bound = ELEM_TOL * np.abs(H64) + 1.2 * dg * (np.abs(u64) + du) + a * du + 1e-6 * a * np.abs(u64)
    got = np.asarray(got, np.float64)
    bad = ~(np.abs(got - H64) <= bound)
    if bad.any():
        i = tuple(int(v) for v in np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outputs outside the per-output bound; "
                             f"first at {i}: got {got[i]!r}, want {H64[i]!r}, bound {bound[i]!r}")
