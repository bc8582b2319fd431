"""GPU parity of the fused append + decode step (ada_decode_append).

Each call appends one token per (sequence, KV head) and decodes over the
cache including it.  It must equal the oracle's append of the same requests
in row order followed by its decode: cache bytes bit-exact, outputs within
2e-3 per row.  It must also be bit-identical to the library's own
ada_encode_append + ada_decode, and write nothing on a booking error."""
import numpy as np
import pytest
import torch

import compressed_kv_cache_ada_amd as ada
import workloads as W
from oracle import oracle as O
from tests.gpu_util import check_outputs, compare_caches, gpu_cache, gpu_pack, log, oracle_cache

pytestmark = pytest.mark.gpu


def _oracle_pack(w, tiers=None):
    oc = oracle_cache(w)
    assert O.pack(oc, w["ctx_len"], w["tiers"] if tiers is None else tiers, w["keys"], w["values"]) == O.OK
    return oc


def _step(w, rng):
    B, Hkv = w["B"], w["Hkv"]
    keys = (rng.standard_normal((B, Hkv, 128)) * 2).astype(np.float32)
    vals = rng.standard_normal((B, Hkv, 128)).astype(np.float16).view(np.uint16)
    tiers = rng.integers(0, 3, (B, Hkv)).astype(np.uint8)
    q = rng.standard_normal((B, w["Hq"], 128)).astype(np.float32)
    return keys, vals, tiers, q


def _dev(keys, vals, tiers, q):
    return (torch.from_numpy(keys).cuda(), torch.from_numpy(vals.view(np.int16)).cuda(),
            torch.from_numpy(tiers).cuda(), torch.from_numpy(q).cuda())


def _rows(w):
    return np.repeat(np.arange(w["B"]), w["Hkv"]), np.tile(np.arange(w["Hkv"]), w["B"])


@pytest.mark.parametrize("name,ctx,batch", [("llama8b", 700, 2), ("tiny", 1000, 2), ("long256k", 900, 1),
                                            ("ragged", 1500, 3),
                                            ("llama8b", 48, 130)])   # 1040 rows: two booking tiles
def test_decode_append_matches_oracle(name, ctx, batch):
    w = W.config(name, ctx=ctx, batch=batch)
    log(f"decode_append {name} ctx {ctx} batch {batch}")
    gc, _ = gpu_pack(w)
    oc = _oracle_pack(w)
    seq, head = _rows(w)
    rng = np.random.default_rng(31)
    for step in range(3):
        keys, vals, tiers, q = _step(w, rng)
        kd, vd, td, qd = _dev(keys, vals, tiers, q)
        out, lse = ada.decode_append(gc, qd, w["scale"], kd, vd, td)
        assert ada.read_status(gc.status) == ada.OK
        assert O.append(oc, seq, head, tiers.ravel(), keys.reshape(-1, 128), vals.reshape(-1, 128)) == O.OK
        compare_caches(gc, oc, w["P"])
        o_ref, l_ref = O.decode(oc, q, w["scale"])
        check_outputs(out.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref)


def test_decode_append_equals_append_then_decode():
    w = W.config("llama8b", ctx=900, batch=2)
    g1, dev = gpu_pack(w)
    g2, _ = gpu_pack(w, dev=dev)
    seq, head = _rows(w)
    seq_d = torch.from_numpy(seq.astype(np.int32)).cuda()
    head_d = torch.from_numpy(head.astype(np.int32)).cuda()
    rng = np.random.default_rng(5)
    for step in range(2):
        keys, vals, tiers, q = _step(w, rng)
        kd, vd, td, qd = _dev(keys, vals, tiers, q)
        o1, l1 = ada.decode_append(g1, qd, w["scale"], kd, vd, td)
        ada.encode_append(g2, seq_d, head_d, td.reshape(-1), kd.reshape(-1, 128), vd.reshape(-1, 128))
        o2, l2 = ada.decode(g2, qd, w["scale"])
        assert ada.read_status(g1.status) == ada.OK and ada.read_status(g2.status) == ada.OK
        h1, h2 = g1.host(), g2.host()
        for k in h1:
            assert np.array_equal(h1[k], h2[k]), k
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_append_into_empty_rows():
    w = W.config("llama8b", ctx=200, batch=2)
    t = w["tiers"].copy()
    t[1, :, :] = -1                     # sequence 1 has no cached token
    gc, _ = gpu_pack(w, tiers=t)
    oc = _oracle_pack(w, tiers=t)
    keys, vals, tiers, q = _step(w, np.random.default_rng(2))
    kd, vd, td, qd = _dev(keys, vals, tiers, q)
    out, lse = ada.decode_append(gc, qd, w["scale"], kd, vd, td)
    assert ada.read_status(gc.status) == ada.OK
    seq, head = _rows(w)
    assert O.append(oc, seq, head, tiers.ravel(), keys.reshape(-1, 128), vals.reshape(-1, 128)) == O.OK
    compare_caches(gc, oc, w["P"])
    # one kept token: the output is its value exactly
    G = w["Hq"] // w["Hkv"]
    v1 = torch.from_numpy(vals[1].view(np.float16).astype(np.float32)).cuda()
    assert torch.equal(out[1], v1.repeat_interleave(G, dim=0))


def test_decode_append_errors_write_nothing():
    w = W.config("tiny", ctx=64)
    gc = gpu_cache(w, dims_override=(4, 4, 4 * (66 + 256)))   # exactly the 4 full T4 pages of the context
    ada.pack(gc, w["ctx_len"], torch.from_numpy(w["tiers"]).cuda(), torch.from_numpy(w["keys"]).cuda(),
             torch.from_numpy(w["values"].view(np.int16)).cuda())
    assert ada.read_status(gc.status) == ada.OK
    before = gc.host()
    q = torch.from_numpy(w["q"]).cuda()
    o_old, l_old = ada.decode(gc, q, w["scale"])
    keys, vals, tiers, _ = _step(w, np.random.default_rng(3))
    tiers[:] = 1
    kd, vd, td, _ = _dev(keys, vals, tiers, w["q"])
    out, lse = ada.decode_append(gc, q, w["scale"], kd, vd, td)    # needs a fifth page
    assert ada.read_status(gc.status) == ada.ENOSPC
    after = gc.host()
    for k in before:
        assert np.array_equal(before[k], after[k]), k
    assert torch.equal(out, o_old) and torch.equal(lse, l_old)
    keys[0, 0, 7] = np.nan
    kd, vd, td, _ = _dev(keys, vals, tiers, w["q"])
    ada.decode_append(gc, q, w["scale"], kd, vd, td)
    assert ada.read_status(gc.status) == ada.EINVAL
    after = gc.host()
    for k in before:
        assert np.array_equal(before[k], after[k]), k
