"""The kernels divide by the constants 6 and 448 with a reciprocal and one FMA
correction, and take the reciprocal of an e4m3fn scale with one Newton step
from the hardware reciprocal; tests/native/const_division_check.c checks both
exhaustively (every finite bf16 numerator; every positive e4m3fn scale with a
start anywhere within 2 ulp) against an independent correctly rounded
quotient."""
import os
import re
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "native", "const_division_check.c")


def test_constant_division_and_e4m3_reciprocal_are_exact():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "check")
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe, SRC, "-lm"], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    rows = {m.group(1): (int(m.group(2)), int(m.group(3)))
            for m in re.finditer(r"(\w+) checked (\d+) bad (\d+)", out)}
    assert rows == {"div6": (32640, 0), "div448": (32640, 0), "e4m3_reciprocal": (630, 0)}, out


def test_kernel_constants_are_the_checked_ones():
    """The reciprocal literals in the device header are the ones checked."""
    with open(os.path.join(ROOT, "pack_token_amd", "csrc", "fp4idx_device.h")) as f:
        src = f.read()
    assert "kRcp6 = 0x1.555556p-3f" in src
    assert "kRcp448 = 0x1.24924ap-9f" in src
