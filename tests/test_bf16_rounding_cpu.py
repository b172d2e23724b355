"""The RMSNorm kernels round each float64 value (x * r) * gamma to bf16 without a branch: add and
subtract 1.5 * 2^(p+52), where 2^p is the bf16 spacing at the value, so the float64 adder rounds to
a multiple of 2^p, ties to even; copy the sign back; convert to float32 exactly.  This compiles
bf16_rounding_check.c with the host compiler and checks that method against the bit-field
definition of the rounding (7 stored mantissa bits, carry into the exponent, subnormals below
2^-126, infinity past the largest bf16) on about 70 million doubles: edge values, every bf16 value,
its midpoint to the next one and the doubles either side of both, and random doubles from 2^-160
to 2^140."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
def test_branch_free_bf16_rounding_equals_the_bit_field_definition(tmp_path):
    exe = str(tmp_path / "bf16_rounding_check")
    subprocess.run(["gcc", "-O2", "-o", exe, os.path.join(HERE, "bf16_rounding_check.c"), "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout
    assert r.stdout.strip().endswith("0 mismatches"), r.stdout
