"""Build libfp4idx.so (HIP kernels + C-ABI layer) for gfx950 with hipcc, in-tree.

Flags:
  -ffp-contract=off     every fp32 step is one rounded operation (no FMA fusion)
  -packed-fp32-ops off  no v_pk_{add,mul,fma}_f32: scalar fp32 VALU only
  mfma-vgpr-form        matrix-core results in VGPRs (the scorer's epilogue reads them)
Denormals stay enabled (the HIP default), which the subnormal-group and
RMSNorm semantics rely on.
"""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp4idx.so")
SOURCES = [os.path.join(CSRC, "fp4idx_kernels.hip"), os.path.join(CSRC, "fp4idx_modes.hip"),
           os.path.join(CSRC, "fp4idx_scorer.hip"), os.path.join(CSRC, "fp4idx_ceiling.hip"),
           os.path.join(CSRC, "fp4idx_api.cpp")]
ARCH = "gfx950"  # the kernels use gfx950-only instructions (scaled FP4 converters and MFMA)


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: set ROCM_PATH")


def flags():
    return ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
            "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(verbose: bool = False, extra=()) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *flags(), *extra, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that line only
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
