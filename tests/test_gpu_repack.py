"""GPU parity of the RDR re-pack (ada_repack) against the oracle.

Bit-exact: the re-packed cache (page table, page counts, open pages, page
metadata, code arena, value pool, allocation counters) for the same source,
utilities and budgets, including utilities emitted by ada_decode_utility.
An unlimited budget reproduces the source; errors leave the destination
untouched."""
import numpy as np
import pytest
import torch

import compressed_kv_cache_ada_amd as ada
import workloads as W
from oracle import oracle as O
from tests.gpu_util import check_outputs, compare_caches, gpu_cache, gpu_pack, log, oracle_cache

pytestmark = pytest.mark.gpu

RATE = {-1: 0, 2: 298, 1: 322, 0: 386}


def _budgets(w, frac):
    return [int(frac * sum(RATE[int(x)] for x in w["tiers"][b].ravel())) for b in range(w["B"])]


def _sources(w):
    gsrc, dev = gpu_pack(w)
    osrc = oracle_cache(w)
    assert O.pack(osrc, w["ctx_len"], w["tiers"], w["keys"], w["values"]) == O.OK
    return gsrc, osrc, dev


@pytest.mark.parametrize("name,ctx,batch,frac", [("llama8b", 900, 2, 0.45), ("ragged", 1200, 3, 0.3),
                                                 ("long256k", 1500, 1, 0.6), ("tiny", 2000, 1, 0.8)])
def test_repack_matches_oracle(name, ctx, batch, frac):
    w = W.config(name, ctx=ctx, batch=batch)
    log(f"repack {name} ctx {ctx} batch {batch} budget {frac}")
    gsrc, osrc, dev = _sources(w)
    util = np.exp(np.random.default_rng(8).standard_normal((osrc.page_capacity, w["P"]))).astype(np.float32)
    budget = _budgets(w, frac)
    gdst = gpu_cache(w)
    ada.repack(gsrc, w["B"], torch.from_numpy(util).cuda(), budget, gdst)
    assert ada.read_status(gdst.status) == ada.OK
    odst = oracle_cache(w)
    st, _ = O.repack(osrc, w["B"], util, budget, odst)
    assert st == O.OK
    compare_caches(gdst, odst, w["P"])
    out, lse = ada.decode(gdst, dev["q"], w["scale"])
    o_ref, l_ref = O.decode(odst, w["q"], w["scale"])
    check_outputs(out.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref)


def test_repack_from_emitted_utility():
    w = W.config("llama8b", ctx=1200, batch=2)
    gsrc, osrc, dev = _sources(w)
    util = torch.zeros((gsrc.desc.page_capacity, w["P"]), dtype=torch.float32, device="cuda")
    ada.decode_utility(gsrc, dev["q"], w["scale"], util)
    budget = _budgets(w, 0.4)
    gdst = gpu_cache(w)
    ada.repack(gsrc, w["B"], util, budget, gdst)
    assert ada.read_status(gdst.status) == ada.OK
    odst = oracle_cache(w)
    assert O.repack(osrc, w["B"], util.cpu().numpy(), budget, odst)[0] == O.OK
    compare_caches(gdst, odst, w["P"])


def test_repack_unlimited_budget_reproduces_source():
    w = W.config("ragged", ctx=1000, batch=3)
    gsrc, _, _ = _sources(w)
    util = torch.ones((gsrc.desc.page_capacity, w["P"]), dtype=torch.float32, device="cuda")
    gdst = gpu_cache(w)
    ada.repack(gsrc, w["B"], util, [1 << 40] * w["B"], gdst)
    assert ada.read_status(gdst.status) == ada.OK
    hs, hd = gsrc.host(), gdst.host()
    n = int(hs["alloc"][0])
    assert np.array_equal(hs["alloc"], hd["alloc"])
    for k in ("page_table", "num_pages", "open_page"):
        assert np.array_equal(hs[k], hd[k]), k
    assert np.array_equal(hs["page_meta"][:n], hd["page_meta"][:n])
    units = int(hs["alloc"][1])
    assert np.array_equal(hs["arena"][: units * 16], hd["arena"][: units * 16])


def test_repack_errors_write_nothing():
    w = W.config("llama8b", ctx=400, batch=2)
    gsrc, _, _ = _sources(w)
    util = torch.ones((gsrc.desc.page_capacity, w["P"]), dtype=torch.float32, device="cuda")
    util[3, 2] = -1.0                                    # a bad utility (page 3 holds kept tokens)
    gdst = gpu_cache(w)
    before = gdst.host()
    ada.repack(gsrc, w["B"], util, _budgets(w, 0.5), gdst)
    assert ada.read_status(gdst.status) == ada.EINVAL
    after = gdst.host()
    for k in before:
        assert np.array_equal(before[k], after[k]), k
    util[3, 2] = 1.0
    small = gpu_cache(w, dims_override=(2, 4, 4 * 386))  # far too small for the kept tokens
    ada.repack(gsrc, w["B"], util, [1 << 40] * w["B"], small)
    assert ada.read_status(small.status) == ada.ENOSPC
