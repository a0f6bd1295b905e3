"""CPU oracle: the plain, slow definition of the W4 quantize / multiply path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  The HIP library never loads it and shares no code with it; the two
meet only through the seeded inputs of ``synth``.

The arithmetic lives in ``w4_oracle.c`` (plain C, IEEE fp32 without
contraction for the quantizer, float64 for the products).  This module only
marshals NumPy arrays into it, plus two host-side formulas from the pages that
need no compiled code:

* ``frobenius_gap`` -- the error measure of gsantana.dev, "Quantizing LLMs
  Without Guesswork", section "Quantize, then dequantize" (Frobenius norm of
  the difference over that of the reference);
* ``bits_per_weight`` -- the storage accounting of the same section, and of
  gowda.ai "LLM fast inference", "Achievement 1" (16-bit scale and 16-bit zero
  per group).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libw4oracle.so")

SYM = 0
ASYM = 1
_MODES = {"sym": SYM, "asym": ASYM, SYM: SYM, ASYM: ASYM}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.w4o_f32_to_f16.argtypes = [ctypes.c_float]
    lib.w4o_f32_to_f16.restype = ctypes.c_uint16
    lib.w4o_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.w4o_f16_to_f32.restype = ctypes.c_float
    lib.w4o_f32_to_e4m3.argtypes = [ctypes.c_float]
    lib.w4o_f32_to_e4m3.restype = ctypes.c_uint8
    lib.w4o_e4m3_to_f32.argtypes = [ctypes.c_uint8]
    lib.w4o_e4m3_to_f32.restype = ctypes.c_float
    lib.w4o_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.w4o_bf16_to_f32.restype = ctypes.c_float
    lib.w4o_quantize.argtypes = [P, i64, i64, i64, ctypes.c_int, ctypes.c_int, P, ctypes.c_int,
                                 P, P, P, P, P]
    lib.w4o_quantize.restype = ctypes.c_int
    lib.w4o_pack.argtypes = [P, i64, i64, P]
    lib.w4o_pack.restype = ctypes.c_int
    lib.w4o_dequant.argtypes = [P, P, P, i64, i64, i64, ctypes.c_int, P]
    lib.w4o_dequant.restype = ctypes.c_int
    lib.w4o_row_quant_e4m3.argtypes = [P, i64, i64, P, P]
    lib.w4o_row_quant_e4m3.restype = ctypes.c_int
    lib.w4o_gemm_ref.argtypes = [P, i64, P, P, P, i64, i64, i64, ctypes.c_int, P, P, i64, P, i64, P]
    lib.w4o_gemm_ref.restype = ctypes.c_int
    for name in ("w4o_f32_to_f16_n", "w4o_f16_to_f32_n", "w4o_f32_to_e4m3_n", "w4o_bf16_to_f32_n"):
        getattr(lib, name).argtypes = [P, i64, P]
        getattr(lib, name).restype = None
    lib.w4o_num_threads.argtypes = []
    lib.w4o_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().w4o_num_threads())


# ----------------------------------------------------------------- formats

def _map(fn, x, in_dtype, out_dtype):
    x = np.ascontiguousarray(np.asarray(x, dtype=in_dtype))
    out = np.empty(x.shape, dtype=out_dtype)
    fn(_ptr(x), x.size, _ptr(out))
    return out


def f32_to_f16_bits(x) -> np.ndarray:
    return _map(_load().w4o_f32_to_f16_n, x, np.float32, np.uint16)


def f16_bits_to_f32(h) -> np.ndarray:
    return _map(_load().w4o_f16_to_f32_n, h, np.uint16, np.float32)


def f32_to_e4m3(x) -> np.ndarray:
    return _map(_load().w4o_f32_to_e4m3_n, x, np.float32, np.uint8)


def e4m3_to_f32(b) -> np.ndarray:
    lib = _load()
    b = np.asarray(b, dtype=np.uint8)
    table = np.array([lib.w4o_e4m3_to_f32(i) for i in range(256)], dtype=np.float32)
    return table[b]


def bf16_bits_to_f32(b) -> np.ndarray:
    return _map(_load().w4o_bf16_to_f32_n, b, np.uint16, np.float32)


def bf16_bits_to_f64(b) -> np.ndarray:
    """bf16 bits -> float64 (exact): the bits are the top half of a binary32."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# --------------------------------------------------------------- quantizer

def quantize(W: np.ndarray, G: int, mode, fracs=None, bits: int = 4, want_sse: bool = False):
    """Blockwise quantization of ``W[N, K]`` (fp32) in groups of ``G`` along K.

    Returns a dict with ``q`` (int16 codes [N, K]), ``scale`` and ``zero``
    (fp16 bits [N, K/G]; zero is None for symmetric), ``clip`` (uint8 index of
    the winning fraction), ``sse`` ([N, K/G, n] float32, if asked) and, for
    4-bit, ``packed`` (canonical nibbles [N, K/2]).
    """
    lib = _load()
    W = np.ascontiguousarray(W, dtype=np.float32)
    assert W.ndim == 2
    N, K = W.shape
    m = _MODES[mode]
    fr = np.ascontiguousarray(np.array([1.0] if fracs is None else fracs, dtype=np.float32))
    ng = K // G
    q = np.empty((N, K), dtype=np.int16)
    scale = np.empty((N, ng), dtype=np.uint16)
    zero = np.empty((N, ng), dtype=np.uint16) if m == ASYM else None
    clip = np.empty((N, ng), dtype=np.uint8)
    sse = np.empty((N, ng, len(fr)), dtype=np.float32) if want_sse else None
    rc = lib.w4o_quantize(_ptr(W), N, K, G, bits, m, _ptr(fr), len(fr), _ptr(q), _ptr(scale),
                          _ptr(zero), _ptr(clip), _ptr(sse))
    if rc != 0:
        raise ValueError(f"oracle quantize rejected its arguments (code {rc})")
    out = {"q": q, "scale": scale, "zero": zero, "clip": clip, "sse": sse}
    if bits == 4:
        out["packed"] = pack(q)
    return out


def pack(q: np.ndarray) -> np.ndarray:
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.int16)
    N, K = q.shape
    packed = np.empty((N, K // 2), dtype=np.uint8)
    if lib.w4o_pack(_ptr(q), N, K, _ptr(packed)) != 0:
        raise ValueError("K must be even")
    return packed


def dequant(packed, scale, zero, G: int, mode) -> np.ndarray:
    """W'[n, k] = (q - zero) * scale as float64 [N, K]."""
    lib = _load()
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scale = np.ascontiguousarray(scale, dtype=np.uint16)
    m = _MODES[mode]
    zero = None if m == SYM else np.ascontiguousarray(zero, dtype=np.uint16)
    N, K2 = packed.shape
    K = 2 * K2
    Wd = np.empty((N, K), dtype=np.float64)
    if lib.w4o_dequant(_ptr(packed), _ptr(scale), _ptr(zero), N, K, G, m, _ptr(Wd)) != 0:
        raise ValueError("bad shapes")
    return Wd


def fake_quant(W: np.ndarray, G: int, mode, fracs=None, bits: int = 4) -> np.ndarray:
    """Quantize then dequantize (float64 result), as the pages' fake-quant does."""
    r = quantize(W, G, mode, fracs, bits)
    ng = W.shape[1] // G
    s = f16_bits_to_f32(r["scale"]).astype(np.float64)
    z = f16_bits_to_f32(r["zero"]).astype(np.float64) if r["zero"] is not None else np.zeros_like(s)
    q = r["q"].astype(np.float64).reshape(W.shape[0], ng, G)
    return ((q - z[:, :, None]) * s[:, :, None]).reshape(W.shape)


# ------------------------------------------------------------- activations

def row_quant_e4m3(X_bits: np.ndarray):
    """Per-row dynamic E4M3 of bf16 activations: returns (xq uint8 [M, K], s float32 [M])."""
    lib = _load()
    X_bits = np.ascontiguousarray(X_bits, dtype=np.uint16)
    M, K = X_bits.shape
    xq = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M,), dtype=np.float32)
    lib.w4o_row_quant_e4m3(_ptr(X_bits), M, K, _ptr(xq), _ptr(s))
    return xq, s


# ---------------------------------------------------------------- products

def gemm_ref(X64: np.ndarray, packed, scale, zero, G: int, mode, a_scale=None, rows=None,
             cols=None) -> np.ndarray:
    """float64 ``Y = diag(a_scale) . X . W'^T`` restricted to ``rows`` x ``cols``."""
    lib = _load()
    X64 = np.ascontiguousarray(X64, dtype=np.float64)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scale = np.ascontiguousarray(scale, dtype=np.uint16)
    m = _MODES[mode]
    zero = None if m == SYM else np.ascontiguousarray(zero, dtype=np.uint16)
    M, K = X64.shape
    N = packed.shape[0]
    assert packed.shape[1] * 2 == K
    rows = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.arange(N, dtype=np.int64) if cols is None else np.ascontiguousarray(cols, dtype=np.int64)
    a = None if a_scale is None else np.ascontiguousarray(a_scale, dtype=np.float32)
    Y = np.empty((len(rows), len(cols)), dtype=np.float64)
    rc = lib.w4o_gemm_ref(_ptr(X64), M, _ptr(packed), _ptr(scale), _ptr(zero), N, K, G, m, _ptr(a),
                          _ptr(rows), len(rows), _ptr(cols), len(cols), _ptr(Y))
    if rc != 0:
        raise ValueError(f"oracle gemm_ref rejected its arguments (code {rc})")
    return Y


def w4a8_ref(X_bits, packed, scale, zero, G: int, mode, rows=None, cols=None):
    """W4A8 reference: per-row E4M3 of X, then s_m * Xq . W'^T in float64."""
    xq, s = row_quant_e4m3(X_bits)
    X64 = e4m3_to_f32(xq).astype(np.float64)
    return gemm_ref(X64, packed, scale, zero, G, mode, a_scale=s, rows=rows, cols=cols), xq, s


def activation(act: str, x: np.ndarray) -> np.ndarray:
    """Gate activation of a gated MLP block in float64: ``silu`` x / (1 + e^-x)
    (SwiGLU) or ``gelu_tanh`` 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))
    (GeGLU), written from their definitions."""
    x = np.asarray(x, dtype=np.float64)
    if act == "silu":
        return x / (1.0 + np.exp(-x))
    if act == "gelu_tanh":
        return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))
    raise ValueError(act)


def gate_up_ref(X_bits, gate, up, G: int, mode, act: str, kind: str = "w4a16", rows=None, cols=None):
    """Gated MLP front half, ``act(X . Wg'^T) * (X . Wu'^T)`` in float64, with
    bf16 activations (``w4a16``) or their per-row E4M3 quantization
    (``w4a8``).  ``gate`` and ``up`` are oracle quantizations (packed, scale,
    zero).  Returns the products' float64 result (and for ``w4a8`` the codes
    and row scales)."""
    if kind == "w4a16":
        X64 = bf16_bits_to_f64(X_bits)
        g = gemm_ref(X64, gate["packed"], gate["scale"], gate["zero"], G, mode, rows=rows, cols=cols)
        u = gemm_ref(X64, up["packed"], up["scale"], up["zero"], G, mode, rows=rows, cols=cols)
        return activation(act, g) * u
    g, xq, s = w4a8_ref(X_bits, gate["packed"], gate["scale"], gate["zero"], G, mode, rows=rows, cols=cols)
    u, _, _ = w4a8_ref(X_bits, up["packed"], up["scale"], up["zero"], G, mode, rows=rows, cols=cols)
    return activation(act, g) * u, xq, s


# --------------------------------------------------------- NF4 comparator
#
# gsantana.dev "Quantizing LLMs Without Guesswork", "Weight-only methods" (the
# NF4 paragraph): 16 levels that are quantiles of a normal distribution, in
# blocks of 64 weights, with double quantization of the block scales
# bringing their cost from 0.5 to 0.127 bits per weight.  The page names
# QLoRA as the source; the steps below are QLoRA's construction and the
# plainest reading of the rest (each listed with the other readings).

NF4_BLOCK = 64          # weights per block (one absmax scale)
NF4_DQ_GROUP = 256      # block scales per second-level fp32 constant


def nf4_levels() -> np.ndarray:
    """The 16 NF4 levels, ascending, as float32: the normal quantiles at 8
    evenly spaced probabilities from delta down to 1/2 (exclusive) for the
    positive side and 7 for the negative side, delta = (1 - 1/30 + 1 - 1/32) / 2,
    plus an exact zero, scaled so that the largest is 1.  Computed in float64
    with scipy's inverse normal CDF, then rounded once to float32."""
    from scipy.special import ndtri
    delta = 0.5 * (1 - 1 / (2 * 15)) + 0.5 * (1 - 1 / (2 * 16))
    pos = ndtri(np.linspace(delta, 0.5, 9)[:-1])
    neg = -ndtri(np.linspace(delta, 0.5, 8)[:-1])
    v = np.sort(np.concatenate([pos, [0.0], neg]))
    return (v / v.max()).astype(np.float32)


def nf4_quantize(W: np.ndarray):
    """NF4 of ``W[N, K]`` (fp32, K a multiple of 64): per block of 64 weights
    along K, absmax = max |w|; every weight becomes the index of the level
    nearest to fp32(w / absmax) (fp32 distances, the lower index on ties; a
    zero block maps to the zero level).  The block absmax values, flattened
    row-major, are quantized in groups of 256: c2 = fp32(max / 255) (1 if
    the group is all zero), q = round_half_even(absmax / c2) as uint8.
    Returns codes [N, K] (uint8 0..15), packed [N, K/2] (even k in the low
    nibble), absmax_q [N*K/64] uint8, c2 [ceil(N*K/64/256)] float32 and the
    unquantized absmax."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    assert K % NF4_BLOCK == 0
    L = nf4_levels()
    blocks = W.reshape(-1, NF4_BLOCK)
    amax = np.abs(blocks).max(axis=1).astype(np.float32)
    safe = np.where(amax == 0, np.float32(1), amax).astype(np.float32)
    x = (blocks / safe[:, None]).astype(np.float32)
    d = np.abs(x[:, :, None] - L[None, None, :]).astype(np.float32)
    codes = np.argmin(d, axis=2).astype(np.uint8).reshape(N, K)
    nb = amax.size
    ng = (nb + NF4_DQ_GROUP - 1) // NF4_DQ_GROUP
    c2 = np.empty(ng, np.float32)
    aq = np.empty(nb, np.uint8)
    for g in range(ng):
        a = amax[g * NF4_DQ_GROUP:(g + 1) * NF4_DQ_GROUP]
        c = np.float32(a.max()) / np.float32(255)
        c = np.float32(1) if c == 0 else np.float32(c)
        c2[g] = c
        aq[g * NF4_DQ_GROUP:(g + 1) * NF4_DQ_GROUP] = np.clip(np.rint(a / c), 0, 255).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return {"codes": codes, "packed": packed, "absmax_q": aq, "c2": c2, "absmax": amax}


def nf4_dequant(codes: np.ndarray, absmax_q: np.ndarray, c2: np.ndarray) -> np.ndarray:
    """W'[n, k] = level[code] * (q * c2) of its block, in float64 from the fp32 values."""
    N, K = codes.shape
    L = nf4_levels().astype(np.float64)
    nb = absmax_q.size
    scale = (absmax_q.astype(np.float32) * np.repeat(c2, NF4_DQ_GROUP)[:nb]).astype(np.float32)
    return L[codes] * np.repeat(scale.astype(np.float64), NF4_BLOCK).reshape(N, K)


def nf4_gemv_ref(x_bits: np.ndarray, codes, absmax_q, c2) -> np.ndarray:
    """float64 ``y = W' . x`` for one bf16 activation row."""
    x = bf16_bits_to_f64(np.asarray(x_bits).reshape(1, -1))[0]
    return nf4_dequant(codes, absmax_q, c2) @ x


def nf4_bits_per_weight() -> float:
    """4-bit codes + an 8-bit scale per 64 weights + an fp32 per 256 blocks."""
    return 4 + 8 / NF4_BLOCK + 32 / (NF4_BLOCK * NF4_DQ_GROUP)


# ----------------------------------------------------------- host formulas

def frobenius_gap(want: np.ndarray, got: np.ndarray) -> float:
    """Distance of ``got`` from ``want`` in the Frobenius norm, relative to the
    norm of ``want`` (both taken as float64)."""
    d = np.asarray(want, dtype=np.float64) - np.asarray(got, dtype=np.float64)
    return float(np.sqrt(np.sum(d * d)) / np.sqrt(np.sum(np.asarray(want, dtype=np.float64) ** 2)))


def bits_per_weight(bits: int, symmetric: bool, block: int, zero_bits: Optional[int] = None) -> float:
    """Storage per weight: code bits + (16-bit scale + zero bits) per block.

    The gsantana.dev page counts a ``bits``-wide zero point (its default); the
    Tahoma page stores a 16-bit zero term (pass ``zero_bits=16``).
    """
    zb = 0 if symmetric else (bits if zero_bits is None else zero_bits)
    return bits + (16 + zb) / block
