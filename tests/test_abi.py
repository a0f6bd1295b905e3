"""The C ABI without a GPU: the library loads, exports every entry point
``include/w4.h`` declares, and rejects bad arguments on the host before any
launch (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|char\s*\*|size_t|void)\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    import w4_dequant_gemm_amd as w4
    if not os.path.exists(w4.library_path):
        from w4_dequant_gemm_amd import build
        build.build()
    return w4.lib()


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("w4_quantize_blockwise", "w4_mse_clip_search", "w4_prepack", "w4_quantize_rows_e4m3",
              "w4a16_gemm", "w4a8_gemm", "w4_gemm_workspace_bytes", "w4a8_gemm_workspace_bytes",
              "w4_status_string", "w4_last_error",
              "w4_abi_version", "w4_portable_save", "w4_portable_info_read", "w4_portable_load",
              "w4a16_gate_up", "w4a16_gate_up_workspace_bytes", "w4a8_gate_up", "w4_nf4_levels", "w4_nf4_quantize",
              "w4_nf4_gemv",
              "w4a16_gemm_noalloc", "w4a8_gate_up_workspace_bytes", "w4a8_gemm_e4m3"):
        assert n in names


def test_noalloc_validation(lib):
    # the no-alloc product checks its arguments like w4a16_gemm before it
    # looks up its scratch array (no device needed for these)
    fake = ctypes.c_void_p(0x1000)
    f = lib.w4a16_gemm_noalloc
    assert f(fake, 2, 96, fake, fake, 8, 48, fake, None) == 2          # unsupported group size
    assert f(fake, -1, 96, fake, fake, 8, 32, fake, None) == 1         # negative M
    assert f(None, 0, 96, None, None, 8, 32, None, None) == 0          # nothing to do
    assert f(fake, 2, 100, fake, fake, 8, 32, fake, None) == 1         # K not a multiple of G


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), f"{name} declared in w4.h but not exported"


def test_read_probe_library_is_separate(lib):
    # the measurement-only streaming-read kernel lives in its own library;
    # the product library does not export it, and the probe rejects bad
    # arguments before any launch
    path = os.path.join(ROOT, "w4_dequant_gemm_amd", "libw4probe.so")
    assert os.path.exists(path), "libw4probe.so is built beside libw4.so"
    probe = ctypes.CDLL(path)
    fn = probe.w4probe_stream_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                   ctypes.c_void_p]
    assert not hasattr(lib, "w4probe_stream_read")
    fake = (ctypes.c_void_p * 1)(4096)
    assert fn(None, 1, 1024, 1, 64, ctypes.c_void_p(4096), None) == 1       # no buffer list
    assert fn(fake, 1, 1000, 1, 64, ctypes.c_void_p(4096), None) == 1       # not a multiple of 16
    assert fn(fake, 1, 1024, 1, 0, ctypes.c_void_p(4096), None) == 1        # no workgroups
    assert fn(fake, 1, 1024, 1, 64, None, None) == 1                        # no sink
    assert fn(fake, 0, 1024, 1, 64, ctypes.c_void_p(4096), None) == 1       # empty buffer list


def test_status_strings(lib):
    import w4_dequant_gemm_amd as w4
    assert w4.w4_abi_version() == 4
    assert w4.w4_status_string(0) == "ok"
    assert w4.w4_status_string(1) == "invalid argument"
    assert w4.w4_status_string(2) == "unsupported configuration"
    assert w4.w4_status_string(3) == "HIP runtime error"


def _fr(*v):
    return (ctypes.c_float * len(v))(*v)


def test_host_validation(lib):
    import w4_dequant_gemm_amd as w4
    fake = ctypes.c_void_p(0x1000)          # never dereferenced: every call below fails validation
    one = _fr(1.0)
    # unsupported group size
    assert lib.w4_quantize_blockwise(fake, 4, 96, 48, 1, one, 1, fake, fake, fake, None, None) == 2
    assert "group size 48" in w4.w4_last_error()
    # K not a multiple of G
    assert lib.w4_quantize_blockwise(fake, 4, 100, 32, 1, one, 1, fake, fake, fake, None, None) == 1
    # bad mode, bad fracs
    assert lib.w4_quantize_blockwise(fake, 4, 96, 32, 7, one, 1, fake, fake, fake, None, None) == 1
    assert lib.w4_quantize_blockwise(fake, 4, 96, 32, 1, _fr(0.9), 1, fake, fake, fake, None, None) == 1
    assert lib.w4_quantize_blockwise(fake, 4, 96, 32, 1, _fr(1.0, 1.5), 2, fake, fake, fake, None, None) == 1
    assert lib.w4_quantize_blockwise(fake, 4, 96, 32, 1, _fr(1.0), 0, fake, fake, fake, None, None) == 1
    assert lib.w4_quantize_blockwise(fake, 4, 96, 32, 1, _fr(*([1.0] * 33)), 33, fake, fake, fake, None, None) == 1
    # asym needs a zero buffer; sym must not get one
    assert lib.w4_quantize_blockwise(fake, 4, 96, 32, 1, one, 1, fake, fake, None, None, None) == 1
    assert lib.w4_quantize_blockwise(fake, 4, 96, 32, 0, one, 1, fake, fake, fake, None, None) == 1
    # misaligned pointer
    assert lib.w4_quantize_blockwise(ctypes.c_void_p(0x1004), 4, 96, 32, 1, one, 1, fake, fake, fake, None,
                                     None) == 1
    assert "aligned" in w4.w4_last_error()
    # null pointers and negative sizes in the products
    assert lib.w4a16_gemm(None, 2, 96, fake, fake, 8, 32, fake, None, 0, None) == 1
    assert lib.w4a16_gemm(fake, -1, 96, fake, fake, 8, 32, fake, None, 0, None) == 1
    assert lib.w4a8_gemm(fake, 2, 96, fake, fake, 8, 32, fake, None, fake, None, 0, None) == 1
    assert lib.w4a16_gemm(fake, 2, 96, fake, fake, 8, 16, fake, None, 0, None) == 2
    assert lib.w4_quantize_rows_e4m3(fake, 2, 12, fake, fake, None) == 1
    assert lib.w4_prepack(fake, fake, None, 4, 96, 32, 1, fake, fake, None) == 1
    # clip search needs its output
    assert lib.w4_mse_clip_search(fake, 4, 96, 32, 1, one, 1, None, None, None) == 1


def test_gemm_workspace_sizes_and_checks(lib):
    # 256 x 256 output tiles whose K is split across workgroups need one
    # fp32 partial tile (256 KB) per split: every tile when there are few,
    # else the tiles of the last partial round over 256 compute units
    import w4_dequant_gemm_amd as w4
    ws = lib.w4_gemm_workspace_bytes
    tile = 256 * 256 * 4
    assert ws(256, 15360, 3840) == 15 * 16 * tile           # 15 tiles: 16 splits of 15 K steps
    assert ws(256, 3840, 15360) == 60 * 4 * tile            # 60 tiles: 4 splits
    assert ws(2048, 8192, 28672) == 128 * 2 * tile          # 896 tiles: the last 128 in halves
    assert ws(2048, 8192, 32768) == 0                        # 1024 tiles: four full rounds
    assert ws(300, 4096, 33000) == 2 * 8 * tile              # 258 tiles: the last 2 in eighths
    # 33..64 rows, K a multiple of 64: the 64 x 128 tiles' K split (optional:
    # without it the weight-streaming kernel runs the product unsplit)
    mid = 64 * 128 * 4
    assert ws(64, 3840, 15360) == 120 * 5 * mid              # 120 tiles: 5 splits
    assert ws(64, 15360, 3840) == 30 * 16 * mid              # 30 tiles: 16 splits
    assert ws(48, 96, 3840) == 0                             # K not a multiple of 64: streaming, no split
    assert ws(32, 15360, 3840) == 4 * 32 * 3840 * 4          # streaming kernel, optional K split in 4
    assert ws(16, 14336, 4096) == 4 * 16 * 4096 * 4          # 64 blocks of 64 columns: 4 K ranges
    assert ws(2, 14336, 4096) == 0 and ws(1, 14336, 4096) == 0
    assert ws(16, 4096, 14336) == 0                          # 32-column blocks already: no split
    assert ws(8, 14336, 4096) == 0                           # activation re-reads below 4x the weights
    # K = 1536, N = 576 (9 blocks of 64 columns): four-step ranges allow 3
    # splits, 27 workgroups, so the product runs unsplit
    assert ws(16, 1536, 576) == 0 and ws(32, 1536, 576) == 0
    # 64 < M <= 128: 64 x 128 tiles, split along K towards 512 workgroups,
    # at most 16 ways and at least 4 K steps of 64 each
    assert ws(128, 3840, 15360) == 240 * 3 * mid             # 240 tiles: 3 splits
    assert ws(100, 15360, 3840) == 60 * 9 * mid              # 60 tiles: 9 splits
    assert ws(128, 576, 130) == 4 * 2 * mid                  # 9 K steps: 2 splits
    assert ws(65, 256, 128) == 0                             # 4 K steps: no split
    assert ws(256, 96, 3840) == 0                            # K not a multiple of 64: 128 x 128 tiles
    assert ws(256, 512, 256) == 0                            # too few K steps to split
    assert ws(-1, 512, 256) == 0 and ws(256, 0, 256) == 0
    # W4A8: the larger of the fp8 kernel's schedule (groups of 128, K a
    # multiple of 128, above 32 rows) and the bf16 kernels' (w4_gemm_
    # workspace_bytes, plus the widened activations, M * K * 2 bytes at a
    # 256-byte aligned offset after the partials, above 128 rows with at
    # least 256 output tiles of 256 x 256)
    ws8 = lib.w4a8_gemm_workspace_bytes
    assert ws8(2048, 8192, 28672) == 128 * 2 * tile + 2048 * 8192 * 2
    assert ws8(2048, 8192, 32768) == 2048 * 8192 * 2
    assert ws8(300, 4096, 33000) == 2 * 8 * tile + 300 * 4096 * 2       # 258 tiles
    assert ws8(1024, 512, 16384) == 1024 * 512 * 2                       # 256 tiles, none split
    # never less than the W4A16 size (one workspace serves both products):
    # here the bf16 64 x 128 tiles' 16 K ranges of 30 tiles, more than the
    # fp8 kernel's 8 ranges
    assert ws8(64, 15360, 3840) == ws(64, 15360, 3840) == 30 * 16 * mid > 30 * 8 * mid
    # 256 x 256 tiles, 30 of them in 8 K ranges
    assert ws8(1056, 8192, 1500) == 30 * 8 * tile
    for shape in ((128, 3840, 15360), (16, 14336, 4096), (256, 96, 3840), (1, 4096, 14336),
                  (256, 15360, 3840), (256, 3840, 15360), (129, 128, 256)):
        assert ws8(*shape) == ws(*shape), shape
    for shape in ((33, 1024, 1000), (520, 4096, 2000), (700, 2048, 1000), (800, 2048, 5000)):
        assert ws8(*shape) >= ws(*shape), shape
    assert ws8(-1, 512, 256) == 0 and ws8(256, 512, 0) == 0
    # a shape that needs one: NULL or too small is rejected before any launch
    fake = ctypes.c_void_p(0x1000)
    need = ws(256, 15360, 3840)
    assert lib.w4a16_gemm(fake, 256, 15360, fake, fake, 3840, 128, fake, None, 0, None) == 1
    assert "workspace" in w4.w4_last_error()
    assert lib.w4a16_gemm(fake, 256, 15360, fake, fake, 3840, 128, fake, fake, need - 16, None) == 1
    assert lib.w4a8_gemm(fake, 256, 15360, fake, fake, 3840, 128, fake, fake, fake, None, 0, None) == 1
    assert lib.w4a16_gemm(fake, 256, 15360, fake, fake, 3840, 128, fake, ctypes.c_void_p(0x1004), need,
                          None) == 1
    assert "aligned" in w4.w4_last_error()
    # a misaligned workspace is refused even where the shape splits nothing
    # (W4A8 above 128 rows may put the widened activations in it)
    assert ws8(2048, 8192, 32768) > 0 and ws(2048, 8192, 32768) == 0
    assert lib.w4a8_gemm(fake, 2048, 8192, fake, fake, 32768, 128, fake, fake, fake, ctypes.c_void_p(0x1008),
                         ws8(2048, 8192, 32768), None) == 1
    assert "aligned" in w4.w4_last_error()
    assert lib.w4a16_gemm(fake, 2, 4096, fake, fake, 64, 128, fake, ctypes.c_void_p(0x1001), 4096, None) == 1


def test_binding_checks_shapes_before_any_launch(lib):
    # the ABI sees pointers only; the binding compares tensor sizes first and
    # raises ValueError (CPU tensors: nothing here reaches a device)
    import torch
    import w4_dequant_gemm_amd as w4
    N, K, G, M = 64, 4096, 128, 3
    X = torch.zeros((M, K), dtype=torch.bfloat16)
    wq = torch.zeros((N, K // 8), dtype=torch.int32)
    sz = torch.zeros((N, K // G), dtype=torch.int32)
    wq_14336 = torch.zeros((N, 14336 // 8), dtype=torch.int32)
    with pytest.raises(ValueError, match="wq holds"):
        w4.w4a16_gemm(X, wq_14336, sz, G)                       # K of X against a longer weight
    with pytest.raises(ValueError, match="sz holds"):
        w4.w4a16_gemm(X, wq, sz[:, :-1].contiguous(), G)
    with pytest.raises(ValueError, match="sz holds"):
        w4.w4a16_gemm(X, wq, sz, 32)                            # wrong group size for these scales
    with pytest.raises(ValueError, match="output has shape"):
        w4.w4a16_gemm(X, wq, sz, G, Y=torch.zeros((M, N + 1), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="xq must be"):
        w4.w4a8_gemm(X, wq, sz, G, xq=torch.zeros((M, K - 8), dtype=torch.uint8))
    with pytest.raises(ValueError, match="xscale has"):
        w4.w4a8_gemm(X, wq, sz, G, xscale=torch.zeros((M + 1,), dtype=torch.float32))
    gate = {"wq": wq, "sz": sz}
    up = {"wq": torch.zeros((N + 16, K // 8), dtype=torch.int32), "sz": sz}
    with pytest.raises(ValueError, match="up weight"):
        w4.w4a16_gate_up(X, gate, up, G)
    with pytest.raises(ValueError, match="up weight"):
        w4.w4a8_gate_up(X, gate, {"wq": wq, "sz": torch.zeros((N, 2 * K // G), dtype=torch.int32)}, G)
    # well-formed shapes get past the checks, to the device check
    with pytest.raises(ValueError, match="device tensor"):
        w4.w4a16_gemm(X, wq, sz, G)


def test_per_channel_group_sizes(lib):
    # G == K is the per-channel granularity: accepted for K a multiple of 32
    # up to 32768 (checked before the empty-shape early return, so N = 0
    # launches nothing); other sizes are unsupported
    import w4_dequant_gemm_amd as w4
    one = _fr(1.0)
    q = lib.w4_quantize_blockwise
    assert q(None, 0, 4096, 4096, 1, one, 1, None, None, None, None, None) == 0
    assert q(None, 0, 14336, 14336, 1, one, 1, None, None, None, None, None) == 0
    assert q(None, 0, 32768, 32768, 0, one, 1, None, None, None, None, None) == 0
    assert q(None, 0, 4008, 4008, 1, one, 1, None, None, None, None, None) == 2
    assert "per-channel" in w4.w4_last_error()
    assert q(None, 0, 65536, 65536, 1, one, 1, None, None, None, None, None) == 2
    assert q(None, 0, 192, 96, 1, one, 1, None, None, None, None, None) == 2
    assert lib.w4a16_gemm(None, 0, 14336, None, None, 8, 14336, None, None, 0, None) == 0
    assert lib.w4_prepack(None, None, None, 0, 4096, 4096, 1, None, None, None) == 0


def test_gate_up_validation(lib):
    import w4_dequant_gemm_amd as w4
    fake = ctypes.c_void_p(0x1000)
    g = lib.w4a16_gate_up
    assert g(fake, 33, 4000, fake, fake, fake, fake, 64, 32, 1, fake, None, 0, None) == 2   # tiled, K % 64 != 0
    assert "multiple of 64" in w4.w4_last_error()
    assert g(fake, 1, 4096, fake, fake, fake, fake, 64, 128, 3, fake, None, 0, None) == 1   # unknown activation
    assert g(fake, 1, 4096, fake, fake, None, fake, 64, 128, 1, fake, None, 0, None) == 1   # no up weights
    assert g(None, 0, 4096, None, None, None, None, 64, 128, 1, None, None, 0, None) == 0   # nothing to do
    assert g(fake, 300, 4096, fake, fake, fake, fake, 64, 128, 1, fake, ctypes.c_void_p(0x1004), 4096,
             None) == 1                                                                 # misaligned workspace
    # the optional split of the pair kernel's last round: 256 x 128 output
    # tiles, partial tiles of 256 x 256 fp32 (both sums)
    gw16 = lib.w4a16_gate_up_workspace_bytes
    assert gw16(2048, 4096, 14336) == 128 * 2 * 256 * 256 * 4       # 896 tiles: the last 128 in halves
    assert gw16(2048, 4096, 16384) == 0                              # 1024 tiles: four whole rounds
    assert gw16(256, 4096, 14336) == 0 and gw16(32, 4096, 14336) == 0   # other kernels
    assert gw16(300, 4096, 2000) == 32 * 8 * 256 * 256 * 4          # 32 tiles, each in 8 K ranges
    assert lib.w4a8_gate_up(fake, 1, 4096, fake, fake, fake, fake, 64, 128, 2, fake, None, fake, None, None, None,
                            0, None) == 1
    # emitting H's E4M3 form needs hscale and a workspace of the partial row maxima
    gw = lib.w4a8_gate_up_workspace_bytes
    assert gw(16, 4096, 14336) == 16 * (14336 // 16) * 4 and gw(2048, 4096, 14336) == 2048 * 112 * 4
    assert gw(0, 4096, 64) == 0
    assert lib.w4a8_gate_up(fake, 2, 4096, fake, fake, fake, fake, 64, 128, 1, fake, fake, fake, fake, None, fake,
                            4096, None) == 1                                  # hq without hscale
    assert lib.w4a8_gate_up(fake, 2, 4096, fake, fake, fake, fake, 64, 128, 1, fake, fake, fake, fake, fake, None,
                            0, None) == 1                                     # no workspace
    assert "workspace" in w4.w4_last_error()
    assert lib.w4a8_gate_up(fake, 2, 4096, fake, fake, fake, fake, 64, 128, 1, fake, fake, fake, None, fake, None,
                            0, None) == 1                                     # hscale without hq
    assert lib.w4a8_gate_up(fake, 2, 4096, fake, fake, fake, fake, 60, 128, 1, fake, fake, fake, fake, fake, fake,
                            4096, None) == 1                                  # N not a multiple of 8
    # the product on E4M3 activations checks like the others
    assert lib.w4a8_gemm_e4m3(fake, None, 2, 4096, fake, fake, 64, 128, fake, None, 0, None) == 1   # no xscale
    assert lib.w4a8_gemm_e4m3(fake, fake, 2, 4096, fake, fake, 64, 48, fake, None, 0, None) == 2    # group size


def test_nf4_levels_match_the_oracle(lib):
    # the library computes its NF4 table on the host (bisection on erfc); the
    # oracle with scipy's inverse normal CDF: the same 16 fp32 values
    import numpy as np
    import oracle
    import w4_dequant_gemm_amd as w4
    np.testing.assert_array_equal(w4.w4_nf4_levels().view(np.uint32), oracle.nf4_levels().view(np.uint32))


def test_nf4_validation(lib):
    fake = ctypes.c_void_p(0x1000)
    assert lib.w4_nf4_quantize(fake, 4, 96, fake, fake, fake, None) == 1           # K not a multiple of 64
    assert lib.w4_nf4_gemv(fake, 65536, fake, fake, fake, 8, fake, None) == 2       # K above the LDS staging
    assert lib.w4_nf4_gemv(fake, 128, fake, None, fake, 8, fake, None) == 1         # no block scales
    assert lib.w4_nf4_quantize(None, 0, 128, None, None, None, None) == 0           # nothing to do


def test_empty_shapes_are_no_ops(lib):
    # nothing to do: OK without touching any pointer (and without a device)
    one = _fr(1.0)
    assert lib.w4_quantize_blockwise(None, 0, 96, 32, 1, one, 1, None, None, None, None, None) == 0
    assert lib.w4a16_gemm(None, 0, 96, None, None, 8, 32, None, None, 0, None) == 0
    assert lib.w4a16_gemm(None, 4, 96, None, None, 0, 32, None, None, 0, None) == 0
    assert lib.w4_quantize_rows_e4m3(None, 0, 96, None, None, None) == 0
    assert lib.w4_prepack(None, None, None, 0, 96, 32, 1, None, None, None) == 0


def test_product_path_has_no_fallback():
    # the binding raises when the library is missing instead of computing anything
    import importlib

    import w4_dequant_gemm_amd as w4
    saved_path, saved_lib = w4.library_path, w4._lib
    try:
        w4.library_path = os.path.join(ROOT, "does-not-exist", "libw4.so")
        w4._lib = None
        with pytest.raises(RuntimeError, match="not built"):
            w4.lib()
    finally:
        w4.library_path, w4._lib = saved_path, saved_lib
    importlib.reload  # noqa: B018 (module kept loaded)


def test_binding_never_imports_the_oracle():
    src = open(os.path.join(ROOT, "w4_dequant_gemm_amd", "__init__.py")).read()
    assert "oracle" not in src.replace("no CPU or PyTorch fallback", "")
    for f in os.listdir(os.path.join(ROOT, "w4_dequant_gemm_amd", "csrc")):
        text = open(os.path.join(ROOT, "w4_dequant_gemm_amd", "csrc", f)).read()
        assert "w4_oracle" not in text and "w4o_" not in text
