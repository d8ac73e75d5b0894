"""The C ABI from a plain C99 program: include/lowbit.h compiles as C, liblowbit.so links, and the calls
that end in host-side validation return the documented statuses (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "bit_quantized_matvec_q1_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c99_consumer_compiles_links_and_validates(tmp_path):
    exe = tmp_path / "consumer"
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "c", "consumer.c"), "-L", LIBDIR, "-llowbit",
           "-Wl,-rpath," + LIBDIR, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
