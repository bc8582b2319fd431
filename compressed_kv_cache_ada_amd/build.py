"""Compile the HIP library ``libada.so`` for gfx950 (MI355X).

Every translation unit is compiled with hipcc for gfx950 with the packed-fp32
VALU forms disabled; the encoder is compiled without floating-point
contraction so each rounding is the one written in the source.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build", "ada")
LIB = os.path.join(HERE, "libada.so")

SOURCES = {
    "ada_api.hip": [],
    "decode.hip": [],
    "encode.hip": ["-ffp-contract=off"],
    "rdr.hip": [],
    "dense.hip": [],
}
COMMON = ["-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include")]


def hipcc():
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


def _compile(name):
    src = os.path.join(CSRC, name)
    obj = os.path.join(BUILD, name.replace(".hip", ".o"))
    cmd = [hipcc()] + COMMON + SOURCES[name] + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
    return obj


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
