"""Host check of the division step inside the quantize kernel.

The kernel reaches the IEEE fp32 quotients of the quantizer — the scale
(max - min) / (2^bits - 1) and the code (x - bias) / s of the MLX page "add
fast::quantized_kv_update" (kernels/quantized.h affine_quantize), and the
Q8_0 scale amax / 127 and code x / d of the llama.cpp page "Metal: Optimize q8_0
KV - #25556" — through a reciprocal and one correction (Markstein's step)
rather than a division per element, the reciprocal of a 16-bit divisor being
the hardware estimate refined by one Newton step.  This test compiles a small C
program that checks the refined reciprocal from every start within one ulp,
and compares the quotient step with the host's IEEE division over every 16-bit
divisor at the numerators where a code could change, and over a dense sample of
all fp32 values for the constant divisors.  It tests the arithmetic argument on the
host; the GPU quantize tests compare the kernel's codes with the oracle's.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_reciprocal_correction_equals_ieee_division(tmp_path):
    exe = str(tmp_path / "division_check")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-mfma", "-o", exe,
                    os.path.join(HERE, "division_check.c"), "-lm"], check=True)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
    out = subprocess.run([exe, "211"], check=True, capture_output=True, text=True, env=env,
                         timeout=600).stdout
    parts = {ln.split()[0]: (int(ln.split()[1]), int(ln.split()[2])) for ln in out.strip().splitlines()}
    assert set(parts) == {"recip", "fp16", "bf16", "const"}
    for name, (n, bad) in parts.items():
        assert n > (100_000 if name == "recip" else 10_000_000), (name, n)
        assert bad == 0, (name, n, bad)
