"""GPU parity of multi-query decode (ada_decode_multi): Q queries per
sequence against the same cache, up to Q * G = 64 virtual heads (beyond 8 the
heads are cut into slices of 8, one work-group each).  Each query's output
must match the oracle's single-query decode of that query (2e-3 per row, as
for ada_decode), and ada_decode_multi with Q = 1 must equal ada_decode
exactly."""
import numpy as np
import pytest
import torch

import compressed_kv_cache_ada_amd as ada
import workloads as W
from oracle import oracle as O
from tests.gpu_util import check_outputs, gpu_pack, log, oracle_cache

pytestmark = pytest.mark.gpu


def _queries(w, Q, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((w["B"], Q, w["Hq"], 128), dtype=np.float32)


@pytest.mark.parametrize("name,ctx,batch,Q", [("llama8b", 1500, 2, 2),    # G = 4 -> 8 virtual heads
                                              ("tiny", 3000, 2, 8),       # G = 1
                                              ("tiny", 700, 3, 2),
                                              ("ragged", 2200, 4, 2),
                                              # more than 8 virtual heads: slices of 8 per work-group
                                              ("llama8b", 1300, 2, 4),    # G = 4 -> 16
                                              ("llama8b", 900, 1, 8),     # G = 4 -> 32
                                              ("ragged", 1700, 3, 4),
                                              ("long256k", 2100, 1, 2),   # G = 8 -> 16
                                              ("long256k", 1500, 1, 4),   # G = 8 -> 32
                                              ("tiny", 1100, 2, 16)])     # G = 1 -> 16
def test_multi_query_matches_oracle(name, ctx, batch, Q):
    w = W.config(name, ctx=ctx, batch=batch)
    log(f"multi {name} ctx {ctx} batch {batch} Q {Q}")
    gc, dev = gpu_pack(w)
    oc = oracle_cache(w)
    assert O.pack(oc, w["ctx_len"], w["tiers"], w["keys"], w["values"]) == O.OK
    qs = _queries(w, Q, 7 + Q)
    out, lse = ada.decode_multi(gc, torch.from_numpy(qs).cuda(), w["scale"])
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for qi in range(Q):
        o_ref, l_ref = O.decode(oc, qs[:, qi], w["scale"])
        check_outputs(out[:, qi], lse[:, qi], o_ref, l_ref)


def test_multi_query_q1_is_decode():
    w = W.config("ragged", ctx=1800, batch=3)
    gc, dev = gpu_pack(w)
    o1, l1 = ada.decode(gc, dev["q"], w["scale"])
    o2, l2 = ada.decode_multi(gc, dev["q"][:, None].contiguous(), w["scale"])
    assert torch.equal(o1, o2[:, 0]) and torch.equal(l1, l2[:, 0])


def test_multi_query_unsupported_shape():
    w = W.config("long256k", ctx=500)            # G = 8: Q * G at most 64
    gc, dev = gpu_pack(w)
    qs = torch.from_numpy(_queries(w, 16, 1)).cuda()
    with pytest.raises(ada.AdaError):
        ada.decode_multi(gc, qs, w["scale"])
