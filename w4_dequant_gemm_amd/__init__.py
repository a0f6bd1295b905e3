"""Python binding of the W4 C ABI (``include/w4.h``) for MI355X (gfx950).

Each function has the name of the C entry point it calls and only marshals
arguments: torch tensors supply device memory and the current HIP stream,
every step of the computation runs in the HIP library ``libw4.so``.  There is
no CPU or PyTorch fallback: if the library is not built, or a call returns a
non-zero status, the function raises.
"""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional, Sequence

import torch

__all__ = [
    "W4Error", "SYM", "ASYM", "MAX_FRACS", "lib", "library_path",
    "w4_quantize_blockwise", "w4_mse_clip_search", "w4_prepack", "w4_quantize_rows_e4m3",
    "w4a16_gemm", "w4a16_gemm_noalloc", "w4a8_gemm", "w4_gemm_workspace_bytes", "w4a8_gemm_workspace_bytes", "w4_status_string",
    "w4_last_error",
    "w4_abi_version", "w4_portable_save", "w4_portable_info_read", "w4_portable_load",
    "w4a16_gate_up", "w4a16_gate_up_workspace_bytes", "w4a8_gate_up", "w4a8_gate_up_workspace_bytes", "w4a8_gemm_e4m3", "ACT_SILU", "ACT_GELU_TANH",
    "w4_nf4_levels", "w4_nf4_quantize", "w4_nf4_gemv",
    "FRACS_PLAIN", "FRACS_11",
]

HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(HERE, "libw4.so")

SYM = 0
ASYM = 1
MAX_FRACS = 32
FRACS_PLAIN = (1.0,)
# 1.00 down to 0.50 in steps of 0.05 (gowda.ai "LLM fast inference", "MSE clipping")
FRACS_11 = (1.00, 0.95, 0.90, 0.85, 0.80, 0.75, 0.70, 0.65, 0.60, 0.55, 0.50)

_MODES = {"sym": SYM, "asym": ASYM, SYM: SYM, ASYM: ASYM}
ACT_SILU = 1
ACT_GELU_TANH = 2
_ACTS = {"silu": ACT_SILU, "gelu_tanh": ACT_GELU_TANH, ACT_SILU: ACT_SILU, ACT_GELU_TANH: ACT_GELU_TANH}


class W4Error(RuntimeError):
    """A W4 call returned a non-zero status."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


class _PortableInfo(ctypes.Structure):
    """``w4_portable_info`` of ``include/w4.h``."""
    _fields_ = [("N", ctypes.c_int64), ("K", ctypes.c_int64), ("G", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("n_fracs", ctypes.c_int32), ("has_clip", ctypes.c_int32), ("payload_bytes", ctypes.c_uint64),
                ("fracs", ctypes.c_float * MAX_FRACS)]


_lib = None


def lib():
    """The loaded ``libw4.so`` (raises if it was never built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(f"W4 HIP library not built: {library_path} is missing "
                           "(run __graft_entry__.build() or python w4_dequant_gemm_amd/build.py)")
    L = ctypes.CDLL(library_path)
    P, i64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.w4_quantize_blockwise.argtypes = [P, i64, i64, I, I, P, I, P, P, P, P, P]
    L.w4_mse_clip_search.argtypes = [P, i64, i64, I, I, P, I, P, P, P]
    L.w4_prepack.argtypes = [P, P, P, i64, i64, I, I, P, P, P]
    L.w4_quantize_rows_e4m3.argtypes = [P, i64, i64, P, P, P]
    sz_t = ctypes.c_size_t
    L.w4a16_gemm.argtypes = [P, i64, i64, P, P, i64, I, P, P, sz_t, P]
    L.w4a16_gemm_noalloc.argtypes = [P, i64, i64, P, P, i64, I, P, P]
    L.w4a16_gemm_noalloc.restype = I
    L.w4a8_gemm.argtypes = [P, i64, i64, P, P, i64, I, P, P, P, P, sz_t, P]
    L.w4_gemm_workspace_bytes.argtypes = [i64, i64, i64]
    L.w4_gemm_workspace_bytes.restype = sz_t
    L.w4a8_gemm_workspace_bytes.argtypes = [i64, i64, i64]
    L.w4a8_gemm_workspace_bytes.restype = sz_t
    L.w4a16_gate_up.argtypes = [P, i64, i64, P, P, P, P, i64, I, I, P, P, sz_t, P]
    L.w4a16_gate_up_workspace_bytes.argtypes = [i64, i64, i64]
    L.w4a16_gate_up_workspace_bytes.restype = sz_t
    L.w4a8_gate_up.argtypes = [P, i64, i64, P, P, P, P, i64, I, I, P, P, P, P, P, P, sz_t, P]
    L.w4a8_gate_up_workspace_bytes.argtypes = [i64, i64, i64]
    L.w4a8_gate_up_workspace_bytes.restype = sz_t
    L.w4a8_gemm_e4m3.argtypes = [P, P, i64, i64, P, P, i64, I, P, P, sz_t, P]
    L.w4a8_gemm_e4m3.restype = I
    L.w4a16_gate_up.restype = I
    L.w4_nf4_levels.argtypes = [P]
    L.w4_nf4_quantize.argtypes = [P, i64, i64, P, P, P, P]
    L.w4_nf4_gemv.argtypes = [P, i64, P, P, P, i64, P, P]
    for name in ("w4_nf4_levels", "w4_nf4_quantize", "w4_nf4_gemv"):
        getattr(L, name).restype = I
    L.w4a8_gate_up.restype = I
    cp = ctypes.c_char_p
    L.w4_portable_save.argtypes = [cp, i64, i64, I, I, P, I, P, P, P, P]
    L.w4_portable_info_read.argtypes = [cp, ctypes.POINTER(_PortableInfo)]
    L.w4_portable_load.argtypes = [cp, P, P, P, P]
    for name in ("w4_portable_save", "w4_portable_info_read", "w4_portable_load"):
        getattr(L, name).restype = I
    for name in ("w4_quantize_blockwise", "w4_mse_clip_search", "w4_prepack", "w4_quantize_rows_e4m3",
                 "w4a16_gemm", "w4a8_gemm"):
        getattr(L, name).restype = I
    L.w4_status_string.argtypes = [I]
    L.w4_status_string.restype = ctypes.c_char_p
    L.w4_last_error.argtypes = []
    L.w4_last_error.restype = ctypes.c_char_p
    L.w4_abi_version.argtypes = []
    L.w4_abi_version.restype = I
    _lib = L
    return L


def w4_status_string(status: int) -> str:
    return lib().w4_status_string(status).decode()


def w4_last_error() -> str:
    return lib().w4_last_error().decode()


def w4_abi_version() -> int:
    return int(lib().w4_abi_version())


# ------------------------------------------------------------------ helpers

def _check(fn: str, status: int):
    if status != 0:
        raise W4Error(fn, status, w4_last_error())


def _dev(t: Optional[torch.Tensor], name: str, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


# the current stream's handle as an integer, without building a Stream object
# (about 2 us of host time per call otherwise, as much as a launch)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device, stream=None):
    if stream is None:
        if _raw_stream is not None and device.index is not None:
            return _raw_stream(device.index)
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _fracs(fracs: Sequence[float]):
    arr = (ctypes.c_float * len(fracs))(*[float(f) for f in fracs])
    return arr, len(fracs)


def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check_product_shapes(fn: str, X, wq, sz, G: int, Y=None, xq=None, xscale=None, up=None):
    """Shape checks the C ABI cannot make (it sees only pointers): the GPU
    layout of an [N, K] weight is N*K/2 bytes of codes and 4*N*K/G bytes of
    scale/zero words; outputs and W4A8 buffers must match [M, N] and [M, K].
    Raises ValueError before anything is launched."""
    if X.dim() != 2:
        raise ValueError(f"{fn}: X must be 2-D [M, K], got shape {tuple(X.shape)}")
    M, K = X.shape
    if wq.dim() != 2:
        raise ValueError(f"{fn}: wq must be 2-D [N, K/8], got shape {tuple(wq.shape)}")
    N = wq.shape[0]
    if G <= 0 or K % G != 0 or K % 8 != 0:
        raise ValueError(f"{fn}: K = {K} must be a multiple of 8 and of the group size G = {G}")
    if _nbytes(wq) != N * K // 2:
        raise ValueError(f"{fn}: wq holds {_nbytes(wq)} bytes; an [{N}, {K}] weight needs N*K/2 = {N * K // 2} "
                         f"(K of X does not match the weight?)")
    if _nbytes(sz) != 4 * N * (K // G):
        raise ValueError(f"{fn}: sz holds {_nbytes(sz)} bytes; an [{N}, {K}] weight with G = {G} needs "
                         f"{4 * N * (K // G)}")
    if Y is not None and tuple(Y.shape) != (M, N):
        raise ValueError(f"{fn}: output has shape {tuple(Y.shape)}, expected ({M}, {N})")
    if xq is not None and (tuple(xq.shape) != (M, K) or xq.element_size() != 1):
        raise ValueError(f"{fn}: xq must be one byte per element with shape ({M}, {K}), got "
                         f"{tuple(xq.shape)} of {xq.dtype}")
    if xscale is not None and xscale.numel() != M:
        raise ValueError(f"{fn}: xscale has {xscale.numel()} elements, expected {M}")
    if up is not None:
        if tuple(up["wq"].shape) != tuple(wq.shape) or _nbytes(up["wq"]) != _nbytes(wq):
            raise ValueError(f"{fn}: the up weight's wq {tuple(up['wq'].shape)} differs from the gate's "
                             f"{tuple(wq.shape)}")
        if _nbytes(up["sz"]) != _nbytes(sz):
            raise ValueError(f"{fn}: the up weight's sz differs in size from the gate's")
    return M, K, N


@functools.lru_cache(maxsize=4096)
def _need_bytes(M: int, K: int, N: int, w4a8: bool) -> int:
    # a function of the shape only
    return w4a8_gemm_workspace_bytes(M, K, N) if w4a8 else w4_gemm_workspace_bytes(M, K, N)


def _workspace(M: int, K: int, N: int, device, workspace, stream, w4a8=False):
    """(pointer, bytes) of the product's workspace: the caller's tensor, or a
    new byte tensor of the fastest schedule's size when the shape uses one
    (kept alive on ``stream``)."""
    need = _need_bytes(M, K, N, w4a8)
    if workspace is None:
        if need == 0:
            return None, 0
        workspace = torch.empty((need,), dtype=torch.uint8, device=device)
        if stream is not None:
            workspace.record_stream(stream)
    return _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()


# ---------------------------------------------------------------- quantizer

def w4_quantize_blockwise(W: torch.Tensor, G: int, mode, fracs: Sequence[float] = FRACS_PLAIN, *,
                          packed=None, scale=None, zero=None, clip_idx=None, want_clip: bool = True,
                          stream=None) -> dict:
    """Quantize fp32 ``W[N, K]`` in groups of ``G`` (see ``w4.h``).

    Returns ``packed`` (uint8 [N, K/2], canonical nibbles), ``scale`` and
    ``zero`` (float16 [N, K/G]; zero is None for symmetric) and
    ``clip_idx`` (uint8 [N, K/G] or None).
    """
    m = _MODES[mode]
    N, K = W.shape
    dev = W.device
    ng = K // G if G else 0
    packed = _empty((N, K // 2), torch.uint8, dev) if packed is None else packed
    scale = _empty((N, ng), torch.float16, dev) if scale is None else scale
    if m == ASYM and zero is None:
        zero = _empty((N, ng), torch.float16, dev)
    if m == SYM:
        zero = None
    if want_clip and clip_idx is None:
        clip_idx = _empty((N, ng), torch.uint8, dev)
    fr, nf = _fracs(fracs)
    rc = lib().w4_quantize_blockwise(_dev(W, "W", torch.float32), N, K, G, m, fr, nf,
                                     _dev(packed, "packed"), _dev(scale, "scale"), _dev(zero, "zero"),
                                     _dev(clip_idx, "clip_idx"), _stream(dev, stream))
    _check("w4_quantize_blockwise", rc)
    return {"packed": packed, "scale": scale, "zero": zero, "clip_idx": clip_idx}


def w4_mse_clip_search(W: torch.Tensor, G: int, mode, fracs: Sequence[float], *, clip_idx=None,
                       sse=None, want_sse: bool = False, stream=None) -> dict:
    """Per-group index of the chosen clip fraction (and every candidate's error)."""
    m = _MODES[mode]
    N, K = W.shape
    dev = W.device
    ng = K // G if G else 0
    clip_idx = _empty((N, ng), torch.uint8, dev) if clip_idx is None else clip_idx
    if want_sse and sse is None:
        sse = _empty((N, ng, len(fracs)), torch.float32, dev)
    fr, nf = _fracs(fracs)
    rc = lib().w4_mse_clip_search(_dev(W, "W", torch.float32), N, K, G, m, fr, nf,
                                  _dev(clip_idx, "clip_idx"), _dev(sse, "sse"), _stream(dev, stream))
    _check("w4_mse_clip_search", rc)
    return {"clip_idx": clip_idx, "sse": sse}


def w4_prepack(packed: torch.Tensor, scale: torch.Tensor, zero: Optional[torch.Tensor], G: int, mode, *,
               wq=None, sz=None, stream=None) -> dict:
    """Portable packing -> GPU layout: ``wq`` (int32 [N, K/8]) and ``sz`` (int32 [N, K/G])."""
    m = _MODES[mode]
    N, K2 = packed.shape
    K = 2 * K2
    dev = packed.device
    wq = _empty((N, K // 8), torch.int32, dev) if wq is None else wq
    sz = _empty((N, K // G if G else 0), torch.int32, dev) if sz is None else sz
    rc = lib().w4_prepack(_dev(packed, "packed"), _dev(scale, "scale"), _dev(zero if m == ASYM else None, "zero"),
                          N, K, G, m, _dev(wq, "wq"), _dev(sz, "sz"), _stream(dev, stream))
    _check("w4_prepack", rc)
    return {"wq": wq, "sz": sz}


# ------------------------------------------------------ portable file form

def _host_bytes(t, name, dtype):
    """A C-contiguous host numpy view of tensor/array ``t`` with element type ``dtype``."""
    import numpy as np
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        t = t.detach()
        if t.dtype == torch.float16:
            t = t.view(torch.int16)
        t = t.cpu().numpy()
    a = np.ascontiguousarray(t)
    if a.dtype.itemsize != np.dtype(dtype).itemsize:
        raise ValueError(f"{name} must have {np.dtype(dtype).itemsize}-byte elements, got {a.dtype}")
    return a.view(dtype)


def _ptr_np(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def w4_portable_save(path: str, packed, scale, zero, G: int, mode, fracs: Sequence[float] = FRACS_PLAIN,
                     clip_idx=None) -> None:
    """Writes the canonical arrays (device or host tensors, or numpy arrays) to ``path``."""
    import numpy as np
    m = _MODES[mode]
    pk = _host_bytes(packed, "packed", np.uint8)
    sc = _host_bytes(scale, "scale", np.uint16)
    ze = _host_bytes(zero, "zero", np.uint16) if m == ASYM else None
    ci = _host_bytes(clip_idx, "clip_idx", np.uint8)
    N, K2 = pk.shape
    arr, n = _fracs(fracs)
    rc = lib().w4_portable_save(os.fsencode(path), N, 2 * K2, G, m, arr, n, _ptr_np(pk), _ptr_np(sc), _ptr_np(ze),
                                _ptr_np(ci))
    _check("w4_portable_save", rc)


def w4_portable_info_read(path: str) -> dict:
    """Header of a portable file: N, K, G, mode, fracs, has_clip, payload_bytes."""
    info = _PortableInfo()
    _check("w4_portable_info_read", lib().w4_portable_info_read(os.fsencode(path), ctypes.byref(info)))
    return {"N": info.N, "K": info.K, "G": info.G, "mode": info.mode, "has_clip": bool(info.has_clip),
            "fracs": tuple(info.fracs[i] for i in range(info.n_fracs)), "payload_bytes": info.payload_bytes}


def w4_portable_load(path: str, device=None, *, prepack: bool = True, stream=None) -> dict:
    """Reads a portable file.  With ``device`` (a GPU) the canonical arrays are
    uploaded there and, with ``prepack``, rearranged into the GPU layout
    (``wq``, ``sz``) at once: the load-time prepack.  Without ``device`` the
    arrays stay in host memory (numpy)."""
    import numpy as np
    info = w4_portable_info_read(path)
    N, K, G = info["N"], info["K"], info["G"]
    asym = info["mode"] == ASYM
    packed = np.empty((N, K // 2), np.uint8)
    scale = np.empty((N, K // G), np.uint16)
    zero = np.empty((N, K // G), np.uint16) if asym else None
    clip = np.empty((N, K // G), np.uint8) if info["has_clip"] else None
    rc = lib().w4_portable_load(os.fsencode(path), _ptr_np(packed), _ptr_np(scale), _ptr_np(zero), _ptr_np(clip))
    _check("w4_portable_load", rc)
    out = dict(info)
    if device is None:
        out.update(packed=packed, scale=scale, zero=zero, clip_idx=clip)
        return out
    dev = torch.device(device)
    out["packed"] = torch.from_numpy(packed).to(dev)
    out["scale"] = torch.from_numpy(scale.view(np.float16)).to(dev)
    out["zero"] = torch.from_numpy(zero.view(np.float16)).to(dev) if asym else None
    out["clip_idx"] = torch.from_numpy(clip).to(dev) if clip is not None else None
    if prepack:
        out.update(w4_prepack(out["packed"], out["scale"], out["zero"], G, info["mode"], stream=stream))
    return out


# --------------------------------------------------------------- multiplies

def w4_quantize_rows_e4m3(X: torch.Tensor, *, xq=None, xscale=None, stream=None):
    """Per-row dynamic E4M3 of bf16 ``X[M, K]``: returns (xq uint8 [M, K], xscale fp32 [M])."""
    M, K = X.shape
    dev = X.device
    xq = _empty((M, K), torch.uint8, dev) if xq is None else xq
    xscale = _empty((M,), torch.float32, dev) if xscale is None else xscale
    rc = lib().w4_quantize_rows_e4m3(_dev(X, "X", torch.bfloat16), M, K, _dev(xq, "xq"),
                                     _dev(xscale, "xscale", torch.float32), _stream(dev, stream))
    _check("w4_quantize_rows_e4m3", rc)
    return xq, xscale


def w4_gemm_workspace_bytes(M: int, K: int, N: int) -> int:
    """Device workspace bytes a product of this shape needs (0 for most)."""
    return int(lib().w4_gemm_workspace_bytes(M, K, N))


def w4a8_gemm_workspace_bytes(M: int, K: int, N: int) -> int:
    """Workspace bytes for the fastest ``w4a8_gemm`` schedule (above 128 rows
    also the widened activations); at least ``w4_gemm_workspace_bytes``."""
    return int(lib().w4a8_gemm_workspace_bytes(M, K, N))


def w4a16_gemm(X: torch.Tensor, wq: torch.Tensor, sz: torch.Tensor, G: int, *, Y=None, workspace=None,
               stream=None):
    """``Y[M, N] = bf16(X . W'^T)`` from bf16 ``X[M, K]`` and the GPU-layout weights.

    ``workspace``: a device tensor of at least ``w4_gemm_workspace_bytes(M, K, N)``
    bytes; allocated here when omitted and the shape needs one."""
    M, K, N = _check_product_shapes("w4a16_gemm", X, wq, sz, G, Y=Y)
    dev = X.device
    Y = _empty((M, N), torch.bfloat16, dev) if Y is None else Y
    ws, ws_bytes = _workspace(M, K, N, dev, workspace, stream)
    rc = lib().w4a16_gemm(_dev(X, "X", torch.bfloat16), M, K, _dev(wq, "wq"), _dev(sz, "sz"), N, G,
                          _dev(Y, "Y", torch.bfloat16), ws, ws_bytes, _stream(dev, stream))
    _check("w4a16_gemm", rc)
    return Y


def w4a16_gemm_noalloc(X: torch.Tensor, wq: torch.Tensor, sz: torch.Tensor, G: int, Y: torch.Tensor, *,
                       stream=None):
    """``w4a16_gemm`` into the caller's ``Y`` with the library's own scratch
    memory (no allocation by the library or here); calls that overlap on one
    GPU must not be issued together."""
    M, K, N = _check_product_shapes("w4a16_gemm_noalloc", X, wq, sz, G, Y=Y)
    dev = X.device
    rc = lib().w4a16_gemm_noalloc(_dev(X, "X", torch.bfloat16), M, K, _dev(wq, "wq"), _dev(sz, "sz"), N, G,
                                  _dev(Y, "Y", torch.bfloat16), _stream(dev, stream))
    _check("w4a16_gemm_noalloc", rc)
    return Y


def w4a8_gemm(X: torch.Tensor, wq: torch.Tensor, sz: torch.Tensor, G: int, *, Y=None, xq=None, xscale=None,
              workspace=None, stream=None):
    """W4A8: per-row E4M3 of ``X`` then ``Y = bf16(xscale * Xq . W'^T)``; returns (Y, xq, xscale)."""
    M, K, N = _check_product_shapes("w4a8_gemm", X, wq, sz, G, Y=Y, xq=xq, xscale=xscale)
    dev = X.device
    Y = _empty((M, N), torch.bfloat16, dev) if Y is None else Y
    xq = _empty((M, K), torch.uint8, dev) if xq is None else xq
    xscale = _empty((M,), torch.float32, dev) if xscale is None else xscale
    ws, ws_bytes = _workspace(M, K, N, dev, workspace, stream, w4a8=True)
    rc = lib().w4a8_gemm(_dev(X, "X", torch.bfloat16), M, K, _dev(wq, "wq"), _dev(sz, "sz"), N, G,
                         _dev(Y, "Y", torch.bfloat16), _dev(xq, "xq"), _dev(xscale, "xscale", torch.float32),
                         ws, ws_bytes, _stream(dev, stream))
    _check("w4a8_gemm", rc)
    return Y, xq, xscale


def w4a16_gate_up_workspace_bytes(M: int, K: int, N: int) -> int:
    """Workspace bytes that let ``w4a16_gate_up`` split K in its last round (0: no split)."""
    return int(lib().w4a16_gate_up_workspace_bytes(M, K, N))


def w4a16_gate_up(X: torch.Tensor, gate: dict, up: dict, G: int, act="silu", *, H=None, workspace=None,
                  stream=None):
    """Gate and up projections in one pass: ``H = bf16(act(X . Wg'^T) * (X . Wu'^T))``
    for bf16 ``X[M, K]`` (above 32 rows K must be a multiple of 64); ``gate`` and ``up`` are GPU layouts from
    ``w4_prepack`` (``wq``, ``sz``); ``act`` is ``"silu"`` or ``"gelu_tanh"``.  ``workspace``: a device
    tensor (an empty one for none); by default one of ``w4a16_gate_up_workspace_bytes`` is allocated."""
    M, K, N = _check_product_shapes("w4a16_gate_up", X, gate["wq"], gate["sz"], G, Y=H, up=up)
    dev = X.device
    H = _empty((M, N), torch.bfloat16, dev) if H is None else H
    if workspace is None:
        need = w4a16_gate_up_workspace_bytes(M, K, N)
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev) if need else None
        if workspace is not None and stream is not None:
            workspace.record_stream(stream)
    ws = _dev(workspace, "workspace") if workspace is not None and workspace.numel() else None
    ws_bytes = _nbytes(workspace) if ws is not None else 0
    rc = lib().w4a16_gate_up(_dev(X, "X", torch.bfloat16), M, K, _dev(gate["wq"], "gate wq"), _dev(gate["sz"], "gate sz"),
                             _dev(up["wq"], "up wq"), _dev(up["sz"], "up sz"), N, G, _ACTS[act],
                             _dev(H, "H", torch.bfloat16), ws, ws_bytes, _stream(dev, stream))
    _check("w4a16_gate_up", rc)
    return H


def w4a8_gate_up_workspace_bytes(M: int, K: int, N: int) -> int:
    """Workspace bytes ``w4a8_gate_up`` needs to emit the E4M3 form of H."""
    return int(lib().w4a8_gate_up_workspace_bytes(M, K, N))


def w4a8_gate_up(X: torch.Tensor, gate: dict, up: dict, G: int, act="silu", *, H=None, xq=None, xscale=None,
                 emit_e4m3: bool = False, hq=None, hscale=None, workspace=None, stream=None):
    """W4A8 form of ``w4a16_gate_up``: per-row E4M3 of ``X`` first; returns (H, xq, xscale).

    With ``emit_e4m3`` (or ``hq`` given) the same pass also produces H's rows
    quantized to E4M3 for the down projection (``w4a8_gemm_e4m3``) and
    returns (H, xq, xscale, hq, hscale)."""
    M, K, N = _check_product_shapes("w4a8_gate_up", X, gate["wq"], gate["sz"], G, Y=H, xq=xq, xscale=xscale,
                                    up=up)
    dev = X.device
    emit = emit_e4m3 or hq is not None
    if emit:
        if hq is not None and (tuple(hq.shape) != (M, N) or hq.element_size() != 1):
            raise ValueError(f"w4a8_gate_up: hq must be one byte per element with shape ({M}, {N})")
        if hscale is not None and hscale.numel() != M:
            raise ValueError(f"w4a8_gate_up: hscale has {hscale.numel()} elements, expected {M}")
    H = _empty((M, N), torch.bfloat16, dev) if H is None else H
    xq = _empty((M, K), torch.uint8, dev) if xq is None else xq
    xscale = _empty((M,), torch.float32, dev) if xscale is None else xscale
    ws, ws_bytes = None, 0
    if emit:
        hq = _empty((M, N), torch.uint8, dev) if hq is None else hq
        hscale = _empty((M,), torch.float32, dev) if hscale is None else hscale
        if workspace is None:
            workspace = torch.empty((max(w4a8_gate_up_workspace_bytes(M, K, N), 16),), dtype=torch.uint8, device=dev)
            if stream is not None:
                workspace.record_stream(stream)
        ws, ws_bytes = _dev(workspace, "workspace"), _nbytes(workspace)
    rc = lib().w4a8_gate_up(_dev(X, "X", torch.bfloat16), M, K, _dev(gate["wq"], "gate wq"), _dev(gate["sz"], "gate sz"),
                            _dev(up["wq"], "up wq"), _dev(up["sz"], "up sz"), N, G, _ACTS[act],
                            _dev(H, "H", torch.bfloat16), _dev(xq, "xq"), _dev(xscale, "xscale", torch.float32),
                            _dev(hq, "hq") if emit else None, _dev(hscale, "hscale", torch.float32) if emit else None,
                            ws, ws_bytes, _stream(dev, stream))
    _check("w4a8_gate_up", rc)
    return (H, xq, xscale, hq, hscale) if emit else (H, xq, xscale)


def w4a8_gemm_e4m3(xq: torch.Tensor, xscale: torch.Tensor, wq: torch.Tensor, sz: torch.Tensor, G: int, *, Y=None,
                   workspace=None, stream=None):
    """W4A8 product on activations already quantized per row: ``Y = bf16(xscale * Xq . W'^T)``."""
    if xq.element_size() != 1:
        raise ValueError("w4a8_gemm_e4m3: xq must hold one byte per element")
    M, K, N = _check_product_shapes("w4a8_gemm_e4m3", xq, wq, sz, G, Y=Y, xscale=xscale)
    dev = xq.device
    Y = _empty((M, N), torch.bfloat16, dev) if Y is None else Y
    ws, ws_bytes = _workspace(M, K, N, dev, workspace, stream, w4a8=True)
    rc = lib().w4a8_gemm_e4m3(_dev(xq, "xq"), _dev(xscale, "xscale", torch.float32), M, K, _dev(wq, "wq"),
                              _dev(sz, "sz"), N, G, _dev(Y, "Y", torch.bfloat16), ws, ws_bytes, _stream(dev, stream))
    _check("w4a8_gemm_e4m3", rc)
    return Y


# -------------------------------------------------------- NF4 comparator

def w4_nf4_levels():
    """The 16 NF4 levels (float32, ascending) the library's kernels use."""
    import numpy as np
    out = np.empty(16, np.float32)
    _check("w4_nf4_levels", lib().w4_nf4_levels(_ptr_np(out)))
    return out


def w4_nf4_quantize(W: torch.Tensor, *, stream=None) -> dict:
    """NF4 of fp32 ``W[N, K]`` (K a multiple of 64): ``packed`` (uint8 [N, K/2]),
    ``absmax_q`` (uint8 [N*K/64]) and ``absmax_c2`` (float32 [ceil(N*K/64/256)])."""
    N, K = W.shape
    dev = W.device
    nb = N * (K // 64)
    packed = _empty((N, K // 2), torch.uint8, dev)
    aq = _empty((nb,), torch.uint8, dev)
    c2 = _empty(((nb + 255) // 256,), torch.float32, dev)
    rc = lib().w4_nf4_quantize(_dev(W, "W", torch.float32), N, K, _dev(packed, "packed"), _dev(aq, "absmax_q"),
                               _dev(c2, "absmax_c2", torch.float32), _stream(dev, stream))
    _check("w4_nf4_quantize", rc)
    return {"packed": packed, "absmax_q": aq, "absmax_c2": c2}


def w4_nf4_gemv(x: torch.Tensor, nf4: dict, *, y=None, stream=None):
    """``y[N] = bf16(W' . x)`` for one bf16 row ``x[K]`` and NF4 weights from ``w4_nf4_quantize``."""
    K = x.numel()
    N = nf4["packed"].shape[0]
    dev = x.device
    y = _empty((N,), torch.bfloat16, dev) if y is None else y
    rc = lib().w4_nf4_gemv(_dev(x, "x", torch.bfloat16), K, _dev(nf4["packed"], "packed"), _dev(nf4["absmax_q"], "absmax_q"),
                           _dev(nf4["absmax_c2"], "absmax_c2", torch.float32), N, _dev(y, "y", torch.bfloat16),
                           _stream(dev, stream))
    _check("w4_nf4_gemv", rc)
    return y
