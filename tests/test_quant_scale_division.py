"""The quantizer's group scale s = fl(fl(max - min) / (2^b - 1)) is computed
on the GPU without a division (kvq_quant.h, group_scale): q0 = fl(D c) with
c = fl(1/(2^b - 1)), the exact fma residual r = D - q0 (2^b - 1), and
q = fl(q0 + r c).  This compiles a small C check with the host compiler
(IEEE fp32 multiply and fma, as on the GPU) and runs it over every fp32 D of
the binades that fp16 extrema can produce, [2^-24, 2^17): q must equal the
correctly rounded quotient in every case.  No GPU."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
def test_fma_corrected_quotient_is_correctly_rounded(tmp_path):
    exe = str(tmp_path / "scale_division_check")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "csrc", "scale_division_check.c"), "-lm"], check=True)
    # D = fl(max - min) of fp16 values is 0 or lies in [2^-24, 131008]
    r = subprocess.run([exe, "-24", "16"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout
    assert "mismatches 0" in r.stdout
