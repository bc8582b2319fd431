"""GPU parity of utility emission (ada_decode_utility) against the oracle.

Every kept token's utility (its softmax weights summed over the KV head's
query heads) must match the oracle per KV row within 2e-3 of the row's
largest utility, rows must sum to G, slots holding no kept token must stay
untouched, and out / lse must be bit-identical to ada_decode."""
import numpy as np
import pytest
import torch

import compressed_kv_cache_ada_amd as ada
import workloads as W
from oracle import oracle as O
from tests.gpu_util import TOL, gpu_pack, log, oracle_cache

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,ctx,batch", [("llama8b", 1500, 2), ("long256k", 2000, 1), ("ragged", 2500, 4),
                                            ("tiny", 3000, 1)])
def test_utility_matches_oracle(name, ctx, batch):
    w = W.config(name, ctx=ctx, batch=batch)
    log(f"utility {name} ctx {ctx} batch {batch}")
    gc, dev = gpu_pack(w)
    oc = oracle_cache(w)
    assert O.pack(oc, w["ctx_len"], w["tiers"], w["keys"], w["values"]) == O.OK
    out, lse, util = ada.decode_utility(gc, dev["q"], w["scale"])
    o2, l2 = ada.decode(gc, dev["q"], w["scale"])
    assert torch.equal(out, o2) and torch.equal(lse, l2)
    u = util.cpu().numpy().astype(np.float64)
    ref = O.decode_utility(oc, w["q"], w["scale"])
    kept = ~np.isnan(ref)
    assert np.array_equal(kept, ~np.isnan(u))          # exactly the kept slots written
    G = w["Hq"] // w["Hkv"]
    for row in range(w["B"] * w["Hkv"]):
        pages = oc.page_table[row, : oc.num_pages[row]]
        if pages.size == 0:
            continue
        ur, ug = ref[pages][kept[pages]], u[pages][kept[pages]]
        assert np.max(np.abs(ug - ur)) <= TOL * np.max(ur), row
        assert abs(ug.sum() - G) <= 1e-3 * G, row
