"""The E4M3 row quantization in the kernels (the row quantizer and the
in-kernel form of the one- and two-row W4A8 products) forms x / s without a
division: q1 = fl(x * fl(1/s)), corrected once by its exact residual with
fused multiply-adds, carrying the sign of x.  ``row_quotient_check.c``
compares the E4M3 code of that quotient with the code of the correctly
rounded fl(x / s) for the bf16 row maxima a (scale s = max(fl(a / 448), 1e-8))
and every bf16 x with |x| <= a; the codes must all agree.  The default run
takes every 7th row maximum (about 150 million pairs, a few seconds);
W4_QUOTIENT_STRIDE=1 checks all of them (about a billion pairs)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _build(tmp_path, src_text=None):
    src = os.path.join(HERE, "row_quotient_check.c")
    if src_text is not None:
        src = str(tmp_path / "variant.c")
        with open(src, "w") as f:
            f.write(src_text)
    exe = str(tmp_path / "row_quotient_check")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", src, "-lm", "-o", exe], check=True)
    return exe


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_division_free_quotient_gives_the_same_codes(tmp_path):
    exe = _build(tmp_path)
    stride = int(os.environ.get("W4_QUOTIENT_STRIDE", "7"))
    out = subprocess.run([exe, str(stride)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout
    assert "differing codes 0" in out.stdout
    pairs = int(out.stdout.split("pairs ")[1].split()[0])
    assert pairs > 1_000_000_000 // stride // 2


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_check_sees_a_quotient_without_the_correction(tmp_path):
    # the plain product fl(x * fl(1/s)) does move codes across E4M3 rounding
    # boundaries, and dropping the sign step turns -0 into +0: the check has
    # to report both
    with open(os.path.join(HERE, "row_quotient_check.c")) as f:
        text = f.read()
    fast = "copysignf(fmaf(fmaf(-q1, s, x), r, q1), x)"
    assert text.count(fast) == 1
    for variant in ("q1", "fmaf(fmaf(-q1, s, x), r, q1)"):
        exe = _build(tmp_path, text.replace(fast, variant))
        out = subprocess.run([exe, "61"], capture_output=True, text=True)
        assert out.returncode == 1 and "differing codes 0" not in out.stdout, variant
