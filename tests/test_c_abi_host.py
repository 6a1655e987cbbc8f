"""The C ABI from C: tests/c/abi_host.c must compile as strict C99 against
include/bf16opt.h, link against the built library and pass its host-side
checks (no GPU is touched)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "bf16_numerics_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs a C compiler")
def test_header_is_strict_c99_and_host_calls_work_from_c(tmp_path):
    assert os.path.exists(os.path.join(LIBDIR, "libbf16opt.so")), "build the library first"
    exe = tmp_path / "abi_host"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           "-o", str(exe), os.path.join(ROOT, "tests", "c", "abi_host.c"), "-L", LIBDIR, "-lbf16opt",
           f"-Wl,-rpath,{LIBDIR}", "-lm"]
    subprocess.run(cmd, check=True)
    ckpt = tmp_path / "ckpt"
    ckpt.mkdir()
    r = subprocess.run([str(exe), str(ckpt)], capture_output=True, text=True, timeout=60)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "FAIL" not in r.stdout
    assert r.stdout.count("ok  ") == 14
