"""Helpers for the GPU parity tests: upload a workload, pack it with the HIP
library and with the oracle, compare caches byte by byte and decode outputs
within the stated tolerance."""
import numpy as np
import torch

import compressed_kv_cache_ada_amd as ada
from oracle import oracle as O
from tests.util import upper_capacity

# output tolerance: per (sequence, query head) row,
#   max_d |o_gpu - o_ref| <= TOL * max_d |o_ref|,  |lse_gpu - lse_ref| <= TOL
TOL = 2e-3


def log(msg):
    print(msg, flush=True)


def dims(w):
    block16_max = ada.block_bytes(0, w["P"]) // 16
    return upper_capacity(w, block16_max)


def gpu_cache(w, cfg=None, dims_override=None):
    cfg = cfg or ada.make_config(w["P"], w["Hq"], w["Hkv"])
    per_row, pages, units = dims_override or dims(w)
    c = ada.Cache(cfg, w["B"], per_row, pages, units)
    ada.cache_init(c)
    return c


def oracle_cache(w, dims_override=None):
    per_row, pages, units = dims_override or dims(w)
    return O.Cache(w["P"], w["Hq"], w["Hkv"], w["B"], per_row, pages, units)


def to_dev(w):
    return {
        "keys": torch.from_numpy(w["keys"]).cuda(),
        "values": torch.from_numpy(w["values"].view(np.int16)).cuda(),
        "q": torch.from_numpy(w["q"]).cuda(),
    }


def gpu_pack(w, tiers=None, dev=None):
    dev = dev or to_dev(w)
    tiers = w["tiers"] if tiers is None else tiers
    c = gpu_cache(w)
    ada.pack(c, w["ctx_len"], torch.from_numpy(tiers).cuda(), dev["keys"], dev["values"])
    st = ada.read_status(c.status)
    assert st == ada.OK, ada.status_str(st)
    return c, dev


def compare_caches(gc, oc, P):
    """Byte equality of every used part of a GPU cache and an oracle cache."""
    g = gc.host()
    assert np.array_equal(g["alloc"], oc.alloc), (g["alloc"], oc.alloc)
    npg, units = int(oc.alloc[0]), int(oc.alloc[1])
    assert np.array_equal(g["num_pages"], oc.num_pages)
    assert np.array_equal(g["open_page"], oc.open_page)
    for r in range(oc.num_pages.size):
        n = oc.num_pages[r]
        assert np.array_equal(g["page_table"][r, :n], oc.page_table[r, :n]), r
    assert np.array_equal(g["page_meta"][:npg], oc.page_meta[:npg])
    a, b = g["arena"][: units * 16], oc.arena[: units * 16]
    if not np.array_equal(a, b):
        bad = np.nonzero(a != b)[0]
        raise AssertionError(f"arena differs at {bad.size} bytes, first at {bad[:8]}")


def check_outputs(out, lse, o_ref, lse_ref, tol=TOL):
    out = np.asarray(out, np.float64)
    lse = np.asarray(lse, np.float64)
    worst = 0.0
    for idx in np.ndindex(o_ref.shape[:-1]):
        ref = o_ref[idx]
        if not np.isfinite(lse_ref[idx]):
            assert lse[idx] == -np.inf and np.all(out[idx] == 0), idx
            continue
        err = np.max(np.abs(out[idx] - ref)) / max(np.max(np.abs(ref)), 1e-30)
        worst = max(worst, err)
        assert err <= tol, (idx, err)
        assert abs(lse[idx] - lse_ref[idx]) <= tol, (idx, lse[idx], lse_ref[idx])
    return worst
