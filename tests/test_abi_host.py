"""The C-ABI library loads, exports every function include/ada.h declares,
and its host-only paths behave as documented (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import compressed_kv_cache_ada_amd as ada

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "ada.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ada_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = ada.lib()
    names = _declared()
    assert len(names) >= 18
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(ada.ABI_SYMBOLS)


def test_block_bytes_and_lut_floats():
    # a page's block: key part (2 + 8 tb + 8 sb bytes per token), then values
    # (256 bytes per token for fp16, 132 for V8)
    assert [ada.block_bytes(t, 16) for t in (0, 1, 2)] == [16 * (130 + 256), 16 * (66 + 256), 16 * (42 + 256)]
    assert ada.block_bytes(1, 32) == 32 * (66 + 256)
    assert [ada.block_bytes(t, 16) for t in (3, 4, 5)] == [16 * (130 + 132), 16 * (66 + 132), 16 * (42 + 132)]
    assert ada.block_bytes(6, 16) == -1 and ada.block_bytes(0, 8) == -1
    assert ada.lut_floats(ada.make_config(16, 32, 8)) == 64 * (256 + 16 + 4)


def test_status_strings():
    for s in range(6):
        assert ada.status_str(s).startswith("ADA_")


def test_host_fp16_rounding_matches_numpy():
    rng = np.random.default_rng(7)
    e = rng.uniform(-30, 16, 20000)
    x = rng.uniform(1, 2, e.size) * 2.0 ** e
    x = np.concatenate([x[x < 65504], [0.0, 2 ** -25, 3 * 2 ** -25, 1 + 2 ** -11, 1 + 2 ** -11 + 2 ** -40,
                                       2 ** -14 - 2 ** -25, 65504.0, 65519.0]])
    ref = x.astype(np.float16).view(np.uint16)
    got = np.array([ada.host_f64_to_f16(v) for v in x], np.uint16)
    assert np.array_equal(got, ref)
    assert ada.host_f64_to_f16(65520.0) == 0x7BFF and ada.host_f64_to_f16(1e300) == 0x7BFF


def _size(fn, *args):
    n = ctypes.c_size_t(0)
    st = fn(*args, ctypes.byref(n))
    return st, n.value


def test_host_validation_without_gpu():
    L = ada.lib()
    good = ada.make_config(16, 32, 8)
    desc = ada.CacheDesc(2, 64, 1000, 100000, 0, 0, 0, 0, 0, 0, 0)
    st, n = _size(L.ada_decode_workspace, ctypes.byref(good), ctypes.byref(desc), 2)
    assert st == ada.OK and n > 0
    bad = [(ada.make_config(16, 32, 8), None),
           (ada.Config(64, 16, 32, 8, 0, 0), ada.EUNSUPPORTED),
           (ada.Config(128, 24, 32, 8, 0, 0), ada.EUNSUPPORTED),
           (ada.Config(128, 16, 48, 8, 0, 0), ada.EUNSUPPORTED),
           (ada.Config(128, 16, 30, 8, 0, 0), ada.EINVAL),
           (ada.Config(128, 16, 32, 0, 0, 0), ada.EINVAL),
           (ada.Config(128, 16, 32, 8, 9, 0), ada.EINVAL),
           (ada.Config(128, 16, 32, 8, 0, 0, 2), ada.EINVAL),
           (ada.Config(128, 16, 32, 8, 0b111000, 0, 0, 0), ada.EINVAL),   # V8 tiers without value_tiers
           (ada.Config(128, 16, 32, 8, 1 << 6, 0, 0, 1), ada.EINVAL),
           (ada.Config(128, 16, 32, 8, 0, 0, 0, 2), ada.EINVAL)]
    for cfg, want in bad[1:]:
        assert _size(L.ada_decode_workspace, ctypes.byref(cfg), ctypes.byref(desc), 2)[0] == want
    # decode refuses a cache with null buffers before touching the device
    null_cache = ada.CacheDesc(2, 64, 1000, 100000, 0, 0, 0, 0, 0, 0, 0)
    assert L.ada_decode(ctypes.byref(good), ctypes.byref(null_cache), None, 2, 1.0, None, None, None, 0, None) \
        == ada.EINVAL
    # multi-query: Q must be a power of two with Q * (Hq / Hkv) <= 64
    L_ws = L.ada_decode_multi_workspace
    st2, n2 = _size(L_ws, ctypes.byref(good), ctypes.byref(desc), 2, 2)
    assert st2 == ada.OK and n2 > n   # twice the partial rows
    assert _size(L_ws, ctypes.byref(good), ctypes.byref(desc), 2, 1) == (ada.OK, n)
    for Q, want in [(0, ada.EINVAL), (-1, ada.EINVAL), (3, ada.EUNSUPPORTED), (4, ada.OK), (16, ada.OK),
                    (32, ada.EUNSUPPORTED)]:
        assert _size(L_ws, ctypes.byref(good), ctypes.byref(desc), 2, Q)[0] == want
    g1 = ada.make_config(16, 8, 8)
    assert _size(L_ws, ctypes.byref(g1), ctypes.byref(desc), 2, 64)[0] == ada.OK
    assert _size(L_ws, ctypes.byref(g1), ctypes.byref(desc), 2, 128)[0] == ada.EUNSUPPORTED
    assert L.ada_decode_multi(ctypes.byref(good), ctypes.byref(desc), None, 2, 3, 1.0, None, None, None, 0,
                              None) == ada.EUNSUPPORTED
    # RDR: unsupported tier set is caught on the host (T8 + T4 only is fine; 0 = all)
    assert _size(L.ada_rdr_workspace, ctypes.byref(good), 2, 100)[0] == ada.OK
    assert L.ada_probe_copy(None, None, 16, None) == ada.EINVAL


def test_shape_limits_and_workspace_ceiling():
    """Shapes the kernels index with 32-bit integers, and workspaces past
    2^48 bytes, are refused on the host (ADA_EUNSUPPORTED) rather than
    reported as a wrapped size."""
    L = ada.lib()
    cfg = ada.make_config(16, 32, 8)
    c = ctypes.byref(cfg)
    I32 = 2 ** 31 - 1
    big = ada.CacheDesc(64, 4096, 1 << 20, 1 << 30, 0, 0, 0, 0, 0, 0, 0)
    assert _size(L.ada_decode_workspace, c, ctypes.byref(big), 64)[0] == ada.OK
    # B * Hq past int32
    assert _size(L.ada_decode_workspace, c, ctypes.byref(big), I32 // 32 + 1)[0] == ada.EUNSUPPORTED
    assert _size(L.ada_decode_workspace, c, ctypes.byref(big), I32 // 32)[0] == ada.OK
    # max_pages_per_head * P past int32
    wide = ada.CacheDesc(1, I32 // 16 + 1, 1 << 20, 1 << 30, 0, 0, 0, 0, 0, 0, 0)
    assert _size(L.ada_decode_workspace, c, ctypes.byref(wide), 1)[0] == ada.EUNSUPPORTED
    assert _size(L.ada_dense_workspace, c, 1, I32 // 16 + 1)[0] == ada.EUNSUPPORTED
    # the utility logit buffer: page_capacity * P * G within uint32
    G = 4
    cap_ok = (2 ** 32 - 1) // (16 * G)
    for cap, want in ((cap_ok, ada.OK), (cap_ok + 1, ada.EUNSUPPORTED)):
        d = ada.CacheDesc(2, 64, cap, 1 << 30, 0, 0, 0, 0, 0, 0, 0)
        assert _size(L.ada_decode_utility_workspace, c, ctypes.byref(d), 2)[0] == want
    # a pack workspace that would pass 2^48 bytes
    assert _size(L.ada_pack_workspace, c, ctypes.byref(big), 64, 2 ** 40)[0] == ada.EUNSUPPORTED
    st, n = _size(L.ada_pack_workspace, c, ctypes.byref(big), 64, 1 << 20)
    assert st == ada.OK and 0 < n <= 2 ** 48
    assert _size(L.ada_rdr_workspace, c, I32, 2 ** 62)[0] == ada.EUNSUPPORTED


def test_workspace_sizes_cover_what_the_kernels_write():
    """Property check of the workspace arithmetic: for explicit chunk lengths,
    the decode workspace holds the split-K partials (m, l and 128 values per
    (sequence, query, query head, chunk)), grows with the batch, and the
    pack and RDR workspaces hold their per-item arrays."""
    hyp = pytest.importorskip("hypothesis")
    st = hyp.strategies
    L = ada.lib()

    @hyp.settings(max_examples=300, deadline=None)
    @hyp.given(P=st.sampled_from([16, 32]), G=st.sampled_from([1, 2, 4, 8]), Hkv=st.integers(1, 16),
               B=st.integers(1, 300), maxp=st.integers(1, 20000), chunk=st.integers(1, 400),
               Q=st.sampled_from([1, 2, 4, 8, 16]), stride=st.integers(1, 1 << 18))
    def check(P, G, Hkv, B, maxp, chunk, Q, stride):
        if Q * G > 64:
            return
        cfg = ada.make_config(P, G * Hkv, Hkv, decode_chunk_pages=chunk)
        desc = ada.CacheDesc(B, maxp, 1 << 20, 1 << 30, 0, 0, 0, 0, 0, 0, 0)
        s1, n1 = _size(L.ada_decode_multi_workspace, ctypes.byref(cfg), ctypes.byref(desc), B, Q)
        assert s1 == ada.OK
        tpg = 64 // P
        cp = min(-(-chunk // tpg) * tpg, 256)
        S = -(-maxp // cp)
        assert n1 >= B * Q * G * Hkv * S * 130 * 4
        s2, n2 = _size(L.ada_decode_multi_workspace, ctypes.byref(cfg), ctypes.byref(desc), B + 1, Q)
        assert s2 == ada.OK and n2 >= n1
        s3, n3 = _size(L.ada_pack_workspace, ctypes.byref(cfg), ctypes.byref(desc), B, stride)
        assert s3 == ada.OK and n3 >= 2 * 4 * B * Hkv * stride   # destination page and slot per item
        s4, n4 = _size(L.ada_rdr_workspace, ctypes.byref(cfg), B, stride)
        assert s4 == ada.OK and n4 >= B * Hkv * stride           # one tie byte per item

    check()
