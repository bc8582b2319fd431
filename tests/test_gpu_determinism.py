"""Run-twice determinism on the GPU: the same call on the same inputs gives
the same bytes -- pack and append (atomics-based booking included), RDR,
re-pack, decode and utility outputs (the split-K merge order is fixed, no
float atomics).  Catches races and order-dependent reductions that a single
comparison against the oracle could pass by luck."""
import numpy as np
import pytest
import torch

import compressed_kv_cache_ada_amd as ada
import workloads as W
from tests.gpu_util import dims, log, to_dev

pytestmark = pytest.mark.gpu


def _cache(w, **kw):
    c = ada.Cache(ada.make_config(w["P"], w["Hq"], w["Hkv"], value_tiers=True, **kw), w["B"], *dims(w))
    ada.cache_init(c)
    return c


def _same(a, b):
    ha, hb = a.host(), b.host()
    for k in ha:
        assert np.array_equal(ha[k], hb[k]), k


def test_runs_repeat_bit_for_bit():
    w = W.config("ragged", ctx=2000, batch=6)
    t = w["tiers"]
    w["tiers"] = np.where(t >= 0, t + 3 * (np.random.default_rng(1).random(t.shape) < 0.4), -1).astype(np.int8)
    dev = to_dev(w)
    log("determinism ragged ctx 2000 batch 6")
    caches = []
    for _ in range(2):
        c = _cache(w)
        ada.pack(c, w["ctx_len"], torch.from_numpy(w["tiers"]).cuda(), dev["keys"], dev["values"])
        assert ada.read_status(c.status) == ada.OK
        caches.append(c)
    _same(*caches)
    rng = np.random.default_rng(2)
    n = 3000
    req = [torch.from_numpy(x).cuda() for x in (rng.integers(0, w["B"], n).astype(np.int32),
                                                  rng.integers(0, w["Hkv"], n).astype(np.int32),
                                                  rng.integers(0, 6, n).astype(np.uint8),
                                                  rng.standard_normal((n, 128), dtype=np.float32),
                                                  rng.standard_normal((n, 128)).astype(np.float16).view(np.int16))]
    for c in caches:
        ada.encode_append(c, *req)
        assert ada.read_status(c.status) == ada.OK
    _same(*caches)
    outs = [ada.decode_utility(c, dev["q"], w["scale"]) for c in caches]
    for x, y in zip(*outs):
        assert torch.equal(torch.nan_to_num(x, nan=-7.0), torch.nan_to_num(y, nan=-7.0))
    util = torch.nan_to_num(outs[0][2], nan=0.0)
    cur = [int(x) for x in np.full(w["B"], 2_000_000)]
    dsts = []
    for c in caches:
        c.cfg = ada.make_config(w["P"], w["Hq"], w["Hkv"], value_tiers=True, rdr_tier_mask=0b111000)
        d = _cache(w, rdr_tier_mask=0b111000)
        ada.repack(c, w["B"], util, cur, d)
        assert ada.read_status(d.status) == ada.OK
        dsts.append(d)
    _same(*dsts)
    r = W.config("rdr128k", ctx=5000, batch=3)
    cfg = ada.make_config(r["P"], r["Hq"], r["Hkv"])
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ut = torch.from_numpy(r["utility"]).cuda()
    a = ada.rdr_assign(cfg, r["ctx_len"], ut, r["budget"], status)
    b = ada.rdr_assign(cfg, r["ctx_len"], ut, r["budget"], status)
    assert ada.read_status(status) == ada.OK and torch.equal(a, b)
