"""Seeded synthetic inputs for the W4 quantize / dequant-multiply path.

This module only draws random numbers and lays them out.  It holds none of the
method's arithmetic (no scales, no codes, no rounding to a grid), so both the CPU
oracle and the HIP path can take their inputs from it without sharing any of
the computation being checked.

The pages measure on trained layers (SmolLM2-135M, an 8B Llama-class model,
Gemma-3-12B, a 70B MLP) and public text.  Neither is available here, so the
weights and activations below are drawn to stand in for them: the same shapes,
the same kind of heavy input-channel outliers the pages describe ("Emergent
Outliers at 6.7B Parameters", nebelwolfi.xyz; "Why activations are the hard
part", gsantana.dev), and the distributions listed per workload.

Recipe (every draw is float64 from NumPy's PCG64 ``default_rng``):

* weight matrix ``i`` of a workload (``i = 0`` for the first, ``1`` for the
  second): ``rng = default_rng(i)``; draw ``W[N, K]`` from the stated
  distribution; then pick ``max(1, round(frac * K))`` input columns without
  replacement and multiply each whole column by the outlier factor; cast to
  float32.
* activation block with ``M`` rows: ``rng = default_rng(1000 + M)``; draw
  ``X[M, K]``; then (12B-class only) pick 4 feature columns without replacement
  and multiply them by 100; cast float64 -> float32 -> bfloat16 (round to
  nearest even, done by torch's dtype cast).
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np

__all__ = ["Workload", "WORKLOADS", "weight", "activations", "activations_bf16_bits",
           "fracs_linspace", "FRACS_11"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shapes: Tuple[Tuple[int, int], ...]       # weight matrices [N, K]
    dist: str                                 # "normal" or "t"
    w_scale: float
    w_df: Optional[float]                     # Student-t degrees of freedom
    outlier_frac: float                       # fraction of input channels (0 = none)
    outlier_mult: float
    group: int
    modes: Tuple[str, ...]                    # "sym" / "asym"
    n_fracs: int                              # clip candidates (1 = plain min/max)
    ms: Tuple[int, ...]                       # activation rows
    x_dist: str                               # "normal" or "t"
    x_df: Optional[float]
    x_outlier_features: int
    x_outlier_mult: float


# The five workloads, smallest first.
WORKLOADS = {
    "tiny": Workload("tiny", ((256, 512),), "normal", 0.02, None, 0.001, 50.0,
                     32, ("sym", "asym"), 20, (1,), "normal", None, 0, 1.0),
    "smollm2_135m_mlp": Workload("smollm2_135m_mlp", ((1536, 576), (576, 1536)), "normal", 0.02,
                                 None, 0.001, 30.0, 32, ("asym",), 1, (1, 4, 16), "normal", None,
                                 0, 1.0),
    "llama8b_decode": Workload("llama8b_decode", ((14336, 4096), (4096, 14336)), "normal", 0.015,
                               None, 0.0005, 50.0, 128, ("asym",), 1, (1, 4, 16), "normal", None,
                               0, 1.0),
    "gemma12b_w4a8": Workload("gemma12b_w4a8", ((15360, 3840), (3840, 15360)), "t", 0.01, 5.0,
                              0.0, 1.0, 128, ("asym",), 11, (1, 16, 64, 256), "normal", None,
                              4, 100.0),
    "llama70b_prefill": Workload("llama70b_prefill", ((28672, 8192),), "normal", 0.01, None,
                                 0.001, 100.0, 128, ("asym",), 11, (2048,), "t", 3.0, 0, 1.0),
}

# The clip fractions the MSE search walks: 1.00 down to 0.50 in steps of 0.05.
FRACS_11 = np.array([1.00, 0.95, 0.90, 0.85, 0.80, 0.75, 0.70, 0.65, 0.60, 0.55, 0.50],
                    dtype=np.float32)


def fracs_linspace(n: int, lo: float = 0.5) -> np.ndarray:
    """``n`` fractions from 1.0 down to ``lo`` (float64 linspace cast to float32)."""
    if n == 1:
        return np.array([1.0], dtype=np.float32)
    return np.linspace(1.0, lo, n, dtype=np.float64).astype(np.float32)


def workload_fracs(wl: Workload) -> np.ndarray:
    if wl.n_fracs == 1:
        return np.array([1.0], dtype=np.float32)
    if wl.n_fracs == 11:
        return FRACS_11.copy()
    return fracs_linspace(wl.n_fracs)


def weight(wl: Workload, index: int = 0, rows: Optional[int] = None) -> np.ndarray:
    """fp32 weight ``W[N, K]`` of matrix ``index`` of workload ``wl``.

    ``rows`` keeps only the first ``rows`` output rows (the draw is the same, so
    a row prefix of the full matrix is returned); used to bound test sizes.
    """
    n, k = wl.shapes[index]
    rng = np.random.default_rng(index)
    if wl.dist == "normal":
        w = rng.standard_normal((n, k)) * wl.w_scale
    elif wl.dist == "t":
        w = rng.standard_t(wl.w_df, size=(n, k)) * wl.w_scale
    else:
        raise ValueError(wl.dist)
    if wl.outlier_frac > 0:
        n_out = max(1, int(round(wl.outlier_frac * k)))
        cols = rng.choice(k, size=n_out, replace=False)
        w[:, cols] *= wl.outlier_mult
    w = w.astype(np.float32)
    if rows is not None:
        w = np.ascontiguousarray(w[:rows])
    return w


def activations(wl: Workload, m: int, k: int) -> np.ndarray:
    """float32 activations ``X[m, k]`` before the bf16 cast."""
    rng = np.random.default_rng(1000 + m)
    if wl.x_dist == "normal":
        x = rng.standard_normal((m, k))
    elif wl.x_dist == "t":
        x = rng.standard_t(wl.x_df, size=(m, k))
    else:
        raise ValueError(wl.x_dist)
    if wl.x_outlier_features:
        cols = rng.choice(k, size=wl.x_outlier_features, replace=False)
        x[:, cols] *= wl.x_outlier_mult
    return x.astype(np.float32)


def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 (round to nearest even via torch's cast), as uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def activations_bf16_bits(wl: Workload, m: int, k: int) -> np.ndarray:
    """bf16 activations ``X[m, k]`` as uint16 bit patterns."""
    return to_bf16_bits(activations(wl, m, k))


def uniform_block(seed: int, n: int, lo: float, hi: float) -> np.ndarray:
    """A float32 vector of ``n`` uniform draws in ``[lo, hi)`` (worked examples)."""
    rng = np.random.default_rng(seed)
    return rng.uniform(lo, hi, size=n).astype(np.float32)


def normal_matrix(seed: int, n: int, k: int, scale: float = 1.0) -> np.ndarray:
    """A float32 ``[n, k]`` matrix of N(0, scale^2) draws (generic test input)."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, k)) * scale).astype(np.float32)
