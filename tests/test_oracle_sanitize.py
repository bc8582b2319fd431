"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

ada_oracle.c is built with -fsanitize=address,undefined into a temporary
directory and a child Python process, with the sanitizer runtimes
preloaded, runs every oracle entry point on small workloads: the codec,
pack and append of all six tiers in both pair layouts, decode and utility,
RDR, transcoding and re-pack.  Any out-of-bounds access, use after free or
undefined behaviour in the oracle aborts the child, and the test fails with
its report.  (Small NumPy buffers handed in by the binding may come from
NumPy's own allocation cache, which the sanitizer does not see.)"""
import os
import subprocess
import sys
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "ada_oracle.c")

CHILD = r'''
with open("/proc/self/maps") as f:
    assert "libasan" in f.read()       # the instrumented runtime is in place
import numpy as np
import workloads as W
from oracle import oracle as O
from tests.util import upper_capacity

def cache(w, layout=0):
    per_row, pages, units = upper_capacity(w, 386 * w["P"] // 16, extra_pages_per_row=12)
    return O.Cache(w["P"], w["Hq"], w["Hkv"], w["B"], per_row, pages, units, pair_layout=layout)

rng = np.random.default_rng(0)
keys = rng.standard_normal((40, 128)).astype(np.float32)
for t in range(6):
    tb, sb = O.TIER_BITS[t]
    assert O.encode(keys, tb, sb)[3] == O.OK
    assert O.encode(keys, tb, sb, pair_layout=1)[3] == O.OK
assert O.v8_encode(rng.standard_normal(128).astype(np.float16).view(np.uint16))[0] == O.OK
for name, ctx, batch in (("ragged", 300, 3), ("long256k", 200, 1), ("tiny", 100, 1)):
    for layout in (0, 1):
        w = W.config(name, ctx=ctx, batch=batch)
        t = w["tiers"]
        w["tiers"] = np.where(t >= 0, t + 3 * rng.integers(0, 2, t.shape), -1).astype(np.int8)
        c = cache(w, layout)
        assert O.pack(c, w["ctx_len"], w["tiers"], w["keys"], w["values"], nthreads=2) == O.OK
        out, lse = O.decode(c, w["q"], w["scale"], nthreads=2)
        u = O.decode_utility(c, w["q"], w["scale"], nthreads=2)
        n = 50
        seq = rng.integers(0, w["B"], n).astype(np.int32)
        head = rng.integers(0, w["Hkv"], n).astype(np.int32)
        tier = rng.integers(0, 6, n).astype(np.uint8)
        k = rng.standard_normal((n, 128)).astype(np.float32)
        v = rng.standard_normal((n, 128)).astype(np.float16).view(np.uint16)
        assert O.append(c, seq, head, tier, k, v) == O.OK
        util = np.nan_to_num(O.decode_utility(c, w["q"], w["scale"], nthreads=2), nan=0.0).astype(np.float32)
        for mask in (0b111, 0b111000):
            d = cache(w, layout)
            st, _ = O.repack(c, w["B"], util, [100000] * w["B"], d, tier_mask=mask)
            assert st == O.OK
            O.decode(d, w["q"], w["scale"], nthreads=2)
        r = W.config("rdr128k", ctx=300, batch=2)
        for mask in (0b111, 0b111000, 0b111001):
            assert O.rdr_assign(r["ctx_len"], r["utility"], np.array([50000, 90000]), tier_mask=mask)[0] == O.OK
for a, b in ((0, 1), (0, 2), (1, 2), (3, 4), (0, 5)):
    O.transcode(a, b, rng.integers(0, 256, (3, 64)), rng.integers(0, 8, (3, 64)))
print("sanitized run ok")
'''


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_under_sanitizers():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    with tempfile.TemporaryDirectory() as d:
        lib = os.path.join(d, "liboracle_san.so")
        subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                               "-fno-sanitize-recover=undefined", "-ffp-contract=off", "-fPIC", "-shared",
                               "-o", lib, SRC, "-lquadmath", "-lm", "-lpthread"])
        env = dict(os.environ, ORACLE_LIB=lib, LD_PRELOAD=f"{asan}:{ubsan}",
                   ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
                   PYTHONPATH=ROOT)
        r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, env=env, capture_output=True, text=True,
                           timeout=600)
        assert r.returncode == 0 and "sanitized run ok" in r.stdout, r.stderr[-4000:]
