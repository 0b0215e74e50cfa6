"""Build the CPU oracle (test infrastructure only) with gcc.

Flags keep every fp32 operation a single IEEE-754 operation: no fast-math,
no FMA contraction, no flush-to-zero.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fp4idx_oracle.c")
LIB = os.path.join(HERE, "libfp4idx_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
          "-Wall", "-Wextra"]


def build(verbose: bool = False, src: str = SRC, out: str = LIB, extra=()) -> str:
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra, "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
