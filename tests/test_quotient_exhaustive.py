"""The division-free quotient used by the HIP quantization kernels is the
correctly rounded fp32 quotient for every input the kernels can see.

The kernels compute code = rne(fl32(x / s)) with s = fl32(a / 127), a the
fp16 absmax of x's vector.  Instead of an IEEE division per element they use
one reciprocal r = fl32(1/s) per vector and Markstein's correction,
q = fma(fma(-q0, s, x), r, q0) with q0 = fl32(x*r).  tests/native/
quotient_check.c restates that formula in C and compares it bit for bit with
IEEE division over every positive finite fp16 a and every fp16 x with
0 < x <= a (about 5e8 pairs; the formula is odd in x).  The same program
with the correction removed reports mismatches, so the check can fail.
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "quotient_check.c")


def _build(tmp_path, src, name):
    exe = str(tmp_path / name)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", src, "-o", exe, "-lm"],
                   check=True)
    return exe


def test_markstein_quotient_is_exact_for_all_fp16_inputs(tmp_path):
    exe = _build(tmp_path, SRC, "qcheck")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout
    checked = int(r.stdout.split("checked ")[1].split()[0])
    # every pair 0 < x <= a of positive finite fp16 patterns 1 .. 0x7bff
    assert checked == 0x7BFF * 0x7C00 // 2


def test_uncorrected_reciprocal_product_is_not_exact(tmp_path):
    src = open(SRC).read().replace("float q1 = fmaf(e, r, q0);", "float q1 = q0; (void)e;")
    p = tmp_path / "naive.c"
    p.write_text(src)
    exe = _build(tmp_path, str(p), "naive")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 1
    assert int(r.stdout.split("mismatches ")[1]) > 0
