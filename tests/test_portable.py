"""The portable file form of a quantized weight (host only, no GPU): the
canonical arrays and the clip fractions come back bit for bit, the layout is
the documented one, and damaged or foreign files are rejected.  Follows
gowda.ai "LLM fast inference", "MSE clipping" (export once into a portable
form of codes, scales and zero terms) and "What the WMT26 paper finds"."""
import os
import struct

import numpy as np
import pytest

import oracle
import synth
from helpers import fracs_for, oracle_quant


@pytest.fixture()
def w4():
    import w4_dequant_gemm_amd as w4
    if not os.path.exists(w4.library_path):
        from w4_dequant_gemm_amd import build
        build.build()
    return w4


def _random(N, K, G, asym, clip, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.integers(0, 256, (N, K // 2), dtype=np.uint8),
            rng.integers(0, 1 << 16, (N, K // G), dtype=np.uint16),
            rng.integers(0, 1 << 16, (N, K // G), dtype=np.uint16) if asym else None,
            rng.integers(0, 20, (N, K // G), dtype=np.uint8) if clip else None)


@pytest.mark.parametrize("N,K,G,mode,clip", [(37, 256, 32, "asym", True), (16, 512, 128, "sym", False),
                                             (5, 192, 64, "asym", False), (0, 128, 32, "asym", True)])
def test_round_trip(w4, tmp_path, N, K, G, mode, clip):
    pk, sc, ze, ci = _random(N, K, G, mode == "asym", clip, seed=N + K)
    fr = synth.FRACS_11 if clip else (1.0,)
    path = str(tmp_path / "w.w4q")
    w4.w4_portable_save(path, pk, sc, ze, G, mode, fr, clip_idx=ci)
    info = w4.w4_portable_info_read(path)
    assert (info["N"], info["K"], info["G"], info["mode"], info["has_clip"]) == (N, K, G, int(mode == "asym"), clip)
    assert np.array_equal(np.array(info["fracs"], np.float32), np.array(fr, np.float32))
    out = w4.w4_portable_load(path)
    assert np.array_equal(out["packed"], pk) and np.array_equal(out["scale"], sc)
    if mode == "asym":
        assert np.array_equal(out["zero"], ze)
    else:
        assert out["zero"] is None
    if clip:
        assert np.array_equal(out["clip_idx"], ci)


def test_documented_layout(w4, tmp_path):
    # header: magic, version, header size, N, K, G, mode, n_fracs, flags,
    # payload size, payload hash, fracs; sections on 64-byte boundaries
    N, K, G = 3, 96, 32
    pk, sc, ze, ci = _random(N, K, G, True, True, seed=7)
    path = str(tmp_path / "w.w4q")
    w4.w4_portable_save(path, pk, sc, ze, G, "asym", (1.0, 0.9), clip_idx=ci)
    raw = open(path, "rb").read()
    assert raw[:8] == b"W4QPORT\0"
    version, hb, n, k, g, mode, nf, flags, pb, h = struct.unpack_from("<IIqqiiiIQQ", raw, 8)
    assert (version, hb, n, k, g, mode, nf, flags) == (1, 128, N, K, G, 1, 2, 1)
    assert struct.unpack_from("<2f", raw, 64) == (1.0, np.float32(0.9))
    assert raw[72:hb] == bytes(hb - 72)                   # zeros up to the header size
    assert len(raw) == hb + pb


def test_section_offsets(w4, tmp_path):
    N, K, G = 3, 96, 32                                   # 144 code bytes, 9 groups
    pk, sc, ze, ci = _random(N, K, G, True, True, seed=8)
    path = str(tmp_path / "w.w4q")
    w4.w4_portable_save(path, pk, sc, ze, G, "asym", (1.0,), clip_idx=ci)
    raw = open(path, "rb").read()
    hb = struct.unpack_from("<I", raw, 12)[0]
    p = raw[hb:]
    assert p[0:144] == pk.tobytes()
    assert p[192:192 + 18] == sc.tobytes()                # packed section rounded up to 192
    assert p[256:256 + 18] == ze.tobytes()
    assert p[320:320 + 9] == ci.tobytes()
    assert len(p) == 384
    # FNV-1a 64 of the payload, as documented
    h = 1469598103934665603
    for b in p:
        h = ((h ^ b) * 1099511628211) & (2 ** 64 - 1)
    assert struct.unpack_from("<Q", raw, 56)[0] == h


def test_oracle_quantized_weights_round_trip(w4, tmp_path):
    # the portable form of the oracle's own quantization of the tiny workload
    # (20 clip fractions): it comes back bit for bit and dequantizes the same
    q = oracle_quant("tiny", 0, None, "asym", 32, 20)
    fr = tuple(float(f) for f in fracs_for(20))
    path = str(tmp_path / "tiny.w4q")
    w4.w4_portable_save(path, q["packed"], q["scale"], q["zero"], 32, "asym", fr, clip_idx=q["clip"])
    out = w4.w4_portable_load(path)
    assert np.array_equal(np.array(out["fracs"], np.float32), np.array(fr, np.float32))
    for key, want in (("packed", q["packed"]), ("scale", q["scale"]), ("zero", q["zero"]), ("clip_idx", q["clip"])):
        assert np.array_equal(out[key], want), key
    W1 = oracle.dequant(out["packed"], out["scale"], out["zero"], 32, "asym")
    W0 = oracle.dequant(q["packed"], q["scale"], q["zero"], 32, "asym")
    assert np.array_equal(W1, W0)


def test_damaged_and_foreign_files(w4, tmp_path):
    N, K, G = 8, 128, 32
    pk, sc, ze, ci = _random(N, K, G, True, True, seed=9)
    path = str(tmp_path / "w.w4q")
    w4.w4_portable_save(path, pk, sc, ze, G, "asym", (1.0,), clip_idx=ci)
    good = open(path, "rb").read()

    def expect(data, status, words):
        bad = str(tmp_path / "bad.w4q")
        open(bad, "wb").write(data)
        with pytest.raises(w4.W4Error) as e:
            w4.w4_portable_load(bad)
        assert e.value.status == status
        assert words in str(e.value)

    flipped = bytearray(good)
    flipped[-100] ^= 0x10
    expect(bytes(flipped), 1, "hash")                     # one bit of the payload
    expect(good[:-1], 1, "truncated")
    expect(good + b"\0", 1, "trailing")
    expect(b"NOTAW4Q!" + good[8:], 1, "magic")
    expect(good[:8] + struct.pack("<I", 2) + good[12:], 2, "version")
    expect(good[:32] + struct.pack("<i", 48) + good[36:], 2, "group size")
    expect(good[:30], 1, "shorter than a header")
    with pytest.raises(w4.W4Error):
        w4.w4_portable_load(str(tmp_path / "missing.w4q"))
    # invalid arguments to save
    with pytest.raises(w4.W4Error):
        w4.w4_portable_save(str(tmp_path / "x.w4q"), pk[:, :50], sc, ze, 64, "asym")   # K = 100 not a multiple
    assert not os.path.exists(str(tmp_path / "x.w4q"))
