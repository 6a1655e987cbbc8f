"""The whole step driven from plain C on the GPU (tests/c/step_gpu.c): HIP
runtime C API for memory and graph capture, the library's C ABI for every
step, the CPU oracle for the check.  No Python or torch sits between the
caller and the kernels."""
import os
import shutil
import subprocess

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs a C compiler")
def test_step_from_c_matches_the_oracle_bit_for_bit(tmp_path):
    libdir = os.path.join(ROOT, "bf16_numerics_amd")
    oracledir = os.path.join(ROOT, "oracle")
    for lib in (os.path.join(libdir, "libbf16opt.so"), os.path.join(oracledir, "liboracle.so")):
        assert os.path.exists(lib), f"{lib} is missing: build first"
    exe = tmp_path / "step_gpu"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-o", str(exe),
                    os.path.join(ROOT, "tests", "c", "step_gpu.c"), "-L", libdir, "-lbf16opt", "-L", oracledir,
                    "-loracle", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    f"-Wl,-rpath,{libdir}:{oracledir}:{os.path.join(ROCM, 'lib')}"], check=True)
    print("running", exe, flush=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "FAIL" not in r.stdout
    assert r.stdout.count("ok  ") == 14
