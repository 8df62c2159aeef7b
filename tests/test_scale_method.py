"""The E4M3 block scale of the GPU codec rounds like the exact amax/6.

"NVFP4 Attention QAT Backward", §Overview: the scale of each group of 16 is
the round-to-nearest-even of amax/6 on the E4M3 grid.  The kernels form the
quotient from a reciprocal product with one FMA correction instead of a
divide and round it with the hardware FP8 conversion; ``tests/c/e4m3_scale_exhaustive.c`` checks, for every finite
non-negative fp32 amax, that this rounds to the same E4M3 value as the exact
rational quotient (and that the bare product would not).  The GPU tests
check separately that the kernels' scale bytes equal the oracle's.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_fma_corrected_quotient_rounds_exactly(tmp_path):
    exe = str(tmp_path / "e4m3_scale_exhaustive")
    src = os.path.join(HERE, "c", "e4m3_scale_exhaustive.c")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-o", exe, src, "-lm"],
                   check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=600).stdout
    fields = dict(zip(out.split()[0::2], out.split()[1::2]))
    assert int(fields["checked"]) == 0x7F800000
    assert int(fields["fma_mismatches"]) == 0
    # the uncorrected product is not enough: the correction step matters
    assert int(fields["mul_mismatches"]) > 0


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_probability_quotient_rounds_exactly(tmp_path):
    """The two-term-reciprocal quotient that the dK/dV kernel, the quantized
    forward output and the fp32 codec feed to the hardware E2M1 conversion
    gives the code of the exact x/s for every fp32 x (tests/c/
    p_quotient_exhaustive.c; the hardware reciprocal is taken within 1 ulp and
    the conversion as round to nearest even, which the GPU codec tests pin)."""
    exe = str(tmp_path / "p_quotient_exhaustive")
    src = os.path.join(HERE, "c", "p_quotient_exhaustive.c")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-o", exe, src, "-lm"],
                   check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=900).stdout
    fields = dict(zip(out.split()[0::2], out.split()[1::2]))
    assert int(fields["checked"]) == 24 * 6 * (1 << 23)
    assert int(fields["mismatches"]) == 0
