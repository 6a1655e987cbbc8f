"""Build libbf16opt.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Floating-point flags: -ffp-contract=off (no implicit multiply-add fusion: the
update's op sequence is fixed), correctly rounded fp32 divide/sqrt and fp32
denormals kept (HIP's defaults, stated explicitly), and packed-fp32
instructions disabled.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbf16opt.so")
SOURCES = [os.path.join(CSRC, "bfo_kernels.hip"), os.path.join(CSRC, "bfo_abi.cpp"),
           os.path.join(CSRC, "bfo_control.cpp"), os.path.join(CSRC, "bfo_checkpoint.cpp")]
ARCH = os.environ.get("BFO_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-pthread",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc():
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def build(verbose: bool = False, extra=()) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
