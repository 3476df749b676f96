"""CPU check of the division-free arithmetic inside the GPU Q8_0 quantizer.

The kernels compute d = max|x| / 127 with one multiply and a Markstein
correction, and q = roundf(x / d) from the exact product x * rcp(d) rounded
through 1.5 * 2^23, falling back to the correctly rounded division near
half-integers (Q8_0 activation blocks: minfer README on the nano-inference
page, M3.5 and M14).  ``quant_fastpath_check.c`` emulates those steps with IEEE
fp32 and fmaf -- the reciprocal anywhere within one ulp of 1/d -- and compares
them with the definitions over every scale of one binade and adversarial
near-tie values.  The GPU tests check the kernels themselves bit for bit
against the oracle.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_quantizer_fast_path_matches_division(tmp_path):
    exe = str(tmp_path / "qfc")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", os.path.join(HERE, "quant_fastpath_check.c"),
                    "-lm", "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    ok, n_fast, n_slow = r.stdout.split()
    assert ok == "ok" and int(n_fast) > 10 ** 8 and int(n_slow) > 10 ** 6
