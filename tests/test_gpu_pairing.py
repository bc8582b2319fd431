"""GPU parity of the half-split pair layout (pair j = (x[j], x[j+64]) for
keys and queries) against the oracle with the same layout: pack, append and
fused append + decode byte for byte, adversarial keys next to every angle
boundary, decode and multi-query outputs within the tolerance, the
stand-alone LUT within 1e-6."""
import numpy as np
import pytest
import torch

import compressed_kv_cache_ada_amd as ada
import workloads as W
from oracle import oracle as O
from tests.gpu_util import check_outputs, compare_caches, dims, log, to_dev
from tests.util import near_boundary_pairs

pytestmark = pytest.mark.gpu

HALF = ada.PAIRS_HALF_SPLIT


def _caches(w, dims_override=None):
    per_row, pages, units = dims_override or dims(w)
    cfg = ada.make_config(w["P"], w["Hq"], w["Hkv"], pair_layout=HALF)
    gc = ada.Cache(cfg, w["B"], per_row, pages, units)
    ada.cache_init(gc)
    oc = O.Cache(w["P"], w["Hq"], w["Hkv"], w["B"], per_row, pages, units, pair_layout=O.PAIRS_HALF)
    return gc, oc


def _pack_both(w, dev):
    gc, oc = _caches(w)
    ada.pack(gc, w["ctx_len"], torch.from_numpy(w["tiers"]).cuda(), dev["keys"], dev["values"])
    assert ada.read_status(gc.status) == ada.OK
    assert O.pack(oc, w["ctx_len"], w["tiers"], w["keys"], w["values"]) == O.OK
    return gc, oc


@pytest.mark.parametrize("name,ctx,batch", [("llama8b", 1200, 2), ("ragged", 1500, 3), ("long256k", 2000, 1)])
def test_pack_and_decode(name, ctx, batch):
    w = W.config(name, ctx=ctx, batch=batch)
    log(f"half-split pack/decode {name} ctx {ctx} batch {batch}")
    dev = to_dev(w)
    gc, oc = _pack_both(w, dev)
    compare_caches(gc, oc, w["P"])
    out, lse = ada.decode(gc, dev["q"], w["scale"])
    o_ref, l_ref = O.decode(oc, w["q"], w["scale"])
    check_outputs(out.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref)


def test_layouts_differ():
    w = W.config("llama8b", ctx=300, batch=1)
    dev = to_dev(w)
    gh, _ = _pack_both(w, dev)
    ga = ada.Cache(ada.make_config(w["P"], w["Hq"], w["Hkv"]), w["B"], *dims(w))
    ada.cache_init(ga)
    ada.pack(ga, w["ctx_len"], torch.from_numpy(w["tiers"]).cuda(), dev["keys"], dev["values"])
    assert ada.read_status(ga.status) == ada.OK
    n = int(gh.host()["alloc"][1]) * 16
    assert not np.array_equal(gh.host()["arena"][:n], ga.host()["arena"][:n])


@pytest.mark.parametrize("tier", [0, 1, 2])
def test_adversarial_codec(tier):
    tb, sb = O.TIER_BITS[tier]
    keys = []
    pairs = near_boundary_pairs(max(tb, 3))
    for start in range(0, len(pairs), 64):
        chunk = pairs[start:start + 64] + [(0.0, 0.0)] * (64 - len(pairs[start:start + 64]))
        k = np.zeros(128, np.float32)
        for j, (x, y) in enumerate(chunk):
            k[j], k[j + 64] = x, y
        keys.append(k)
    diag = np.zeros(128, np.float32)
    diag[:64] = [1, -1, -1, 1] * 16
    diag[64:] = [1, 1, -1, -1] * 16
    keys.append(diag)                                   # 2-bit diagonal ties
    rng = np.random.default_rng(40 + tier)
    keys.extend((rng.standard_normal((100, 128)) * np.exp(2 * rng.standard_normal((100, 128)))).astype(np.float32))
    keys = np.array(keys, np.float32)
    n = keys.shape[0]
    vals = rng.standard_normal((n, 128)).astype(np.float16).view(np.uint16)
    w = W.config("tiny", ctx=max(n, 16))
    gc, oc = _caches(w)
    zeros = np.zeros(n, np.int32)
    ada.encode_append(gc, torch.from_numpy(zeros).cuda(), torch.from_numpy(zeros).cuda(),
                      torch.from_numpy(np.full(n, tier, np.uint8)).cuda(), torch.from_numpy(keys).cuda(),
                      torch.from_numpy(vals.view(np.int16)).cuda())
    assert ada.read_status(gc.status) == ada.OK
    assert O.append(oc, zeros, zeros, np.full(n, tier, np.uint8), keys, vals) == O.OK
    compare_caches(gc, oc, w["P"])


def test_fused_append_decode():
    w = W.config("llama8b", ctx=700, batch=2)
    dev = to_dev(w)
    gc, oc = _pack_both(w, dev)
    rows = w["B"] * w["Hkv"]
    seq, head = np.repeat(np.arange(w["B"]), w["Hkv"]), np.tile(np.arange(w["Hkv"]), w["B"])
    rng = np.random.default_rng(12)
    for step in range(2):
        keys = rng.standard_normal((w["B"], w["Hkv"], 128), dtype=np.float32)
        vals = rng.standard_normal((w["B"], w["Hkv"], 128)).astype(np.float16).view(np.uint16)
        tiers = rng.integers(0, 3, (w["B"], w["Hkv"])).astype(np.uint8)
        q = rng.standard_normal((w["B"], w["Hq"], 128), dtype=np.float32)
        out, lse = ada.decode_append(gc, torch.from_numpy(q).cuda(), w["scale"], torch.from_numpy(keys).cuda(),
                                     torch.from_numpy(vals.view(np.int16)).cuda(), torch.from_numpy(tiers).cuda())
        assert ada.read_status(gc.status) == ada.OK
        assert O.append(oc, seq, head, tiers.ravel(), keys.reshape(rows, 128), vals.reshape(rows, 128)) == O.OK
        compare_caches(gc, oc, w["P"])
        o_ref, l_ref = O.decode(oc, q, w["scale"])
        check_outputs(out.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref)


def test_multi_query():
    w = W.config("llama8b", ctx=900, batch=2)
    dev = to_dev(w)
    gc, oc = _pack_both(w, dev)
    q2 = np.random.default_rng(3).standard_normal((w["B"], 2, w["Hq"], 128), dtype=np.float32)
    out, lse = ada.decode_multi(gc, torch.from_numpy(q2).cuda(), w["scale"])
    for qi in range(2):
        o_ref, l_ref = O.decode(oc, np.ascontiguousarray(q2[:, qi]), w["scale"])
        check_outputs(out[:, qi].cpu().numpy(), lse[:, qi].cpu().numpy(), o_ref, l_ref)


def test_lut():
    w = W.config("llama8b", ctx=16, batch=2)
    cfg = ada.make_config(16, w["Hq"], w["Hkv"], pair_layout=HALF)
    lut = ada.build_lut(cfg, torch.from_numpy(w["q"]).cuda()).cpu().numpy()
    for b in range(w["B"]):
        for hq in range(w["Hq"]):
            q = w["q"][b, hq]
            ref = np.concatenate([O.lut(q, tb, O.PAIRS_HALF).ravel() for tb in (8, 4, 2)])
            assert np.max(np.abs(lut[b, hq] - ref)) <= 1e-6 * np.max(np.abs(ref)), (b, hq)
