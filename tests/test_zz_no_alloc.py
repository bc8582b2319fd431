"""ada_decode_noalloc: the decode without a workspace argument (for callers
that cannot allocate) against ada_decode, the entry point it shares its
kernels with.  Two calls in a row on different caches, the second smaller
(fewer sequences, shorter context, another head grouping), so partials left
in the library's array by the first call must not leak into the second.
Each call must equal ada_decode bit for bit and the oracle within 2e-3 per
row; a call whose partials would not fit the array is refused before any
launch."""
import numpy as np
import pytest
import torch

import compressed_kv_cache_ada_amd as ada
import workloads as W
from oracle import oracle as O
from tests.gpu_util import check_outputs, gpu_pack, log, oracle_cache

pytestmark = pytest.mark.gpu


def _one(name, ctx, batch):
    w = W.config(name, ctx=ctx, batch=batch)
    log(f"noalloc {name} ctx {ctx} batch {batch}")
    gc, dev = gpu_pack(w)
    o1, l1 = ada.decode_noalloc(gc, dev["q"], w["scale"])
    o2, l2 = ada.decode(gc, dev["q"], w["scale"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    oc = oracle_cache(w)
    assert O.pack(oc, w["ctx_len"], w["tiers"], w["keys"], w["values"]) == O.OK
    o_ref, l_ref = O.decode(oc, w["q"], w["scale"])
    check_outputs(o1.cpu().numpy(), l1.cpu().numpy(), o_ref, l_ref)


def test_noalloc_decode_twice_second_smaller():
    _one("ragged", 3000, 6)
    _one("llama8b", 900, 2)


def test_noalloc_refuses_partials_past_the_array():
    cfg = ada.make_config(16, 32, 8, decode_chunk_pages=4)
    cache = ada.Cache(cfg, 8, 16384, 64, 64 * 386)   # 8 x 32 query heads x 4096 chunks of partials
    ada.cache_init(cache)
    q = torch.zeros((8, 32, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(ada.AdaError) as e:
        ada.decode_noalloc(cache, q, 0.1)
    assert e.value.status == ada.EUNSUPPORTED
