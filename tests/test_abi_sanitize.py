"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The C-ABI glue (ada_api.hip: argument checks, layout and workspace
arithmetic) is rebuilt with the sanitizers on its host pass only and linked,
in a temporary directory, with the device objects of the normal build.  A
child Python process, with the sanitizer runtime preloaded and the binding
pointed at that library, runs every host-only path: the checks of
test_abi_host, then every workspace query over a grid of configurations,
batch sizes and cache shapes that reaches the largest sizes the types carry,
and the null-buffer refusals of the compute entry points.  An out-of-bounds
access, a signed overflow or a float-to-integer conversion out of range in
the glue aborts the child, and the test fails with its report.  No kernel
is launched and no device memory is touched: the only HIP calls reached are
device queries, which fail without a GPU and leave the documented defaults."""
import glob
import os
import subprocess
import sys
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "compressed_kv_cache_ada_amd", "csrc")
OBJS = os.path.join(ROOT, "_build", "ada")

CHILD = r'''
import ctypes, itertools, sys
with open("/proc/self/maps") as f:
    assert "libclang_rt.asan" in f.read()
import compressed_kv_cache_ada_amd as ada
ada.LIB_PATH = sys.argv[1]
L = ada.lib()
import tests.test_abi_host as T
for name in dir(T):
    if name.startswith("test_"):
        getattr(T, name)()

sz = ctypes.c_size_t
def ws(fn, *args):
    n = sz(12345)
    st = fn(*args, ctypes.byref(n))
    assert st in (ada.OK, ada.EINVAL, ada.EUNSUPPORTED, ada.ENOSPC), (fn, st)
    if st == ada.OK:
        assert n.value <= 2 ** 48 and (n.value > 0 or args[-1] == 0 or args[-2] == 0), (fn, args, n.value)
    else:
        assert n.value == 12345             # nothing written on refusal
    return st

I32 = 2 ** 31 - 1
configs = []
for P, hq, hkv, mask, chunk, layout, vt in itertools.product(
        (16, 32), (32, 8), (8, 1), (0, 0b011, 0b111000), (0, 1, 64), (0, 1), (0, 1)):
    if hq % hkv:
        continue
    configs.append(ada.Config(128, P, hq, hkv, mask, chunk, layout, vt))
configs += [ada.Config(128, 16, 32, 8, 0, -1, 0, 0), ada.Config(128, 16, I32, 1, 0, 0, 0, 0),
            ada.Config(128, 16, 32, 8, 0, I32, 0, 0), ada.Config(-128, 16, 32, 8, 0, 0, 0, 0)]
shapes = [(1, 1, 1, 1), (2, 64, 1000, 100000), (64, 4096, 1 << 20, 1 << 40),
          (4096, 1 << 20, 1 << 40, 1 << 60), (I32, I32, 2 ** 63 - 1, 2 ** 63 - 1),
          (0, 0, 0, 0), (-1, -5, -1, -1)]
ok = 0
for cfg in configs:
    c = ctypes.byref(cfg)
    for seqs, maxp, cap, arena in shapes:
        d = ada.CacheDesc(seqs, maxp, cap, arena, 0, 0, 0, 0, 0, 0, 0)
        dp = ctypes.byref(d)
        for B in (0, 1, 3, 64, 4096, I32, -1):
            ok += ws(L.ada_decode_workspace, c, dp, B) == ada.OK
            for Q in (1, 2, 8, 0):
                ws(L.ada_decode_multi_workspace, c, dp, B, Q)
            ws(L.ada_decode_utility_workspace, c, dp, B)
            ws(L.ada_decode_append_workspace, c, dp, B)
            ws(L.ada_repack_workspace, c, dp, B)
            ws(L.ada_append_workspace, c, dp, B)
            for stride in (0, 1, 4096, 1 << 20, 2 ** 40, 2 ** 63 - 1, -1):
                ws(L.ada_pack_workspace, c, dp, B, stride)
        for B, stride in itertools.product((0, 1, 64, I32, -1), (0, 1, 1 << 18, 2 ** 40, 2 ** 63 - 1, -1)):
            ws(L.ada_rdr_workspace, c, B, stride)
        for B, mp in itertools.product((0, 1, 64, I32, -1), (0, 1, 4096, I32, -1)):
            ws(L.ada_dense_workspace, c, B, mp)
    L.ada_lut_floats(c)
assert ok > 100
for t, P in itertools.product(range(-2, 9), (0, 8, 16, 32, 64, I32, -1)):
    L.ada_block_bytes(t, P)
for s in range(-3, 12):
    L.ada_status_str(s)
for v in (float("nan"), float("inf"), -float("inf"), 1e308, -1e308, 5e-324, -0.0, 2.0 ** 64, -2.0 ** 64):
    L.ada_host_f64_to_f16(v)
# compute entry points refuse null buffers on the host
good = ada.make_config(16, 32, 8)
null = ada.CacheDesc(2, 64, 1000, 100000, 0, 0, 0, 0, 0, 0, 0)
g, n0 = ctypes.byref(good), ctypes.byref(null)
assert L.ada_cache_init(g, n0, None) == ada.EINVAL
assert L.ada_decode(g, n0, None, 2, 1.0, None, None, None, 0, None) == ada.EINVAL
assert L.ada_decode_utility(g, n0, None, 2, 1.0, None, None, None, None, 0, None) == ada.EINVAL
assert L.ada_read_status(None, None) == ada.EINVAL
print("host glue clean:", ok, "workspace queries OK")
'''


def _asan_runtime():
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return libs[-1] if libs else None


def test_abi_glue_under_sanitizers():
    runtime = _asan_runtime()
    hipcc = "/opt/rocm/bin/hipcc"
    if runtime is None or not os.path.exists(hipcc):
        pytest.skip("clang sanitizer runtime or hipcc not available")
    device_objs = [os.path.join(OBJS, n) for n in ("decode.o", "encode.o", "rdr.o", "dense.o")]
    if not all(os.path.exists(o) for o in device_objs):
        pytest.skip("the library has not been built (compressed_kv_cache_ada_amd/build.py)")
    with tempfile.TemporaryDirectory() as tmp:
        obj = os.path.join(tmp, "ada_api.o")
        so = os.path.join(tmp, "libada_san.so")
        # each sanitizer flag applies to the host pass only
        host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
        cmd = [hipcc, "-O1", "-g", "--offload-arch=gfx950", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include")] + host_san + \
              ["-c", os.path.join(CSRC, "ada_api.hip"), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        r = subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", so, obj] + device_objs,
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ, LD_PRELOAD=runtime, PYTHONPATH=ROOT,
                   ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        r = subprocess.run([sys.executable, "-c", CHILD, so], cwd=ROOT, env=env, capture_output=True,
                           text=True, timeout=600)
        assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-6000:])
        assert "host glue clean" in r.stdout
