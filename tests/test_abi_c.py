"""The C ABI from a plain C99 program: include/ada.h compiles as C (gcc,
-std=c99 -Wall -Werror), every function the program calls links against
libada.so, and the host-only paths return what the header documents.  No
GPU is touched: the program makes no device call."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIBDIR = os.path.join(ROOT, "compressed_kv_cache_ada_amd")


def test_c_program_links_and_runs():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    if not os.path.exists(os.path.join(LIBDIR, "libada.so")):
        pytest.skip("the library has not been built")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "c_abi_check")
        cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
               os.path.join(HERE, "c_abi_check.c"), "-o", exe, "-L", LIBDIR, "-l:libada.so",
               "-Wl,-rpath," + LIBDIR]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, (r.stdout, r.stderr)
        assert r.stdout.strip() == "ok"
