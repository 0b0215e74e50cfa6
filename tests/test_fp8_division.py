"""The FP8 fp32-scale path divides by a reciprocal plus one FMA correction;
this runs tests/native/fp8_division_check.c over every bf16 significand
against every fp32 significand (2^30 pairs, split over worker processes) and
requires every quotient to equal the correctly rounded one."""
import os
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "fp8_division_check.c")


@pytest.mark.slow
def test_reciprocal_fma_quotient_is_correctly_rounded():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "check")
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe, SRC, "-lm"], check=True)
        n = max(1, min(8, os.cpu_count() or 1))
        step = (1 << 23) // n
        procs = [subprocess.Popen([exe, str(i * step), str((1 << 23) if i == n - 1 else (i + 1) * step)],
                                  stdout=subprocess.PIPE, text=True) for i in range(n)]
        outs = [p.communicate(timeout=600)[0] for p in procs]
    total = sum(int(o.split()[1]) for o in outs)
    bad = sum(int(o.split()[3]) for o in outs)
    assert total == (1 << 30) and bad == 0, outs
