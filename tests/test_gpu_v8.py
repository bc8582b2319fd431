"""GPU parity of the value tiers (ids 3-5: T8 / T4 / T2 keys with V8 values)
against the oracle: pack, append and fused append + decode byte for byte
(values next to every rounding case of the codec included), decode,
multi-query and utility outputs within the tolerance, RDR over a V8 chain
and re-pack from fp16 tiers into V8 tiers byte for byte, and the errors."""
import numpy as np
import pytest
import torch

import compressed_kv_cache_ada_amd as ada
import workloads as W
from oracle import oracle as O
from tests.gpu_util import TOL, check_outputs, compare_caches, dims, log, oracle_cache, to_dev

pytestmark = pytest.mark.gpu


def _cfg(w, **kw):
    return ada.make_config(w["P"], w["Hq"], w["Hkv"], value_tiers=True, **kw)


def _gcache(w, cfg=None, dims_override=None):
    c = ada.Cache(cfg or _cfg(w), w["B"], *(dims_override or dims(w)))
    ada.cache_init(c)
    return c


def _v8(w, frac, seed=3):
    """a copy of the workload with about `frac` of the kept tokens in V8 tiers"""
    w = dict(w)
    t = w["tiers"]
    rng = np.random.default_rng(seed)
    shift = (rng.random(t.shape) < frac) * 3
    w["tiers"] = np.where(t >= 0, t + shift, -1).astype(np.int8)
    return w


def _pack_both(w, dev):
    gc = _gcache(w)
    ada.pack(gc, w["ctx_len"], torch.from_numpy(w["tiers"]).cuda(), dev["keys"], dev["values"])
    assert ada.read_status(gc.status) == ada.OK
    oc = oracle_cache(w)
    assert O.pack(oc, w["ctx_len"], w["tiers"], w["keys"], w["values"]) == O.OK
    return gc, oc


CASES = [("llama8b", 1200, 2, 0.5), ("ragged", 1500, 3, 0.5), ("long256k", 2000, 1, 1.0), ("tiny", 3000, 1, 1.0),
         ("llama8b", 700, 2, 1.0)]


@pytest.mark.parametrize("name,ctx,batch,frac", CASES)
def test_pack_and_decode(name, ctx, batch, frac):
    w = _v8(W.config(name, ctx=ctx, batch=batch), frac)
    log(f"v8 pack/decode {name} ctx {ctx} batch {batch} frac {frac}")
    dev = to_dev(w)
    gc, oc = _pack_both(w, dev)
    compare_caches(gc, oc, w["P"])
    out, lse = ada.decode(gc, dev["q"], w["scale"])
    o_ref, l_ref = O.decode(oc, w["q"], w["scale"])
    check_outputs(out.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref)


@pytest.mark.parametrize("edge", ["inside", "below", "above"])
def test_fused_conversion_range_edges(edge):
    """A group whose V8 tokens all have block maxima in [2^-8, 2^12) (scale
    bytes 119..138) has its codes converted with one fused multiply-add per
    pair, any other group with a subtract and a multiply; the two give the
    same fp16 values.  Blocks exactly at the range's edges (maxima 2^-8 and
    4094), and one token in 37 one step outside it (maxima 0.75 * 2^-8 or
    4096), decoded against the oracle."""
    w = _v8(W.config("llama8b", ctx=900, batch=2), 1.0)
    rng = np.random.default_rng(23)
    shape = w["values"].shape
    u = rng.uniform(-1, 1, shape[:-1] + (4, 32))
    u[..., 0] = np.sign(u[..., 0])                      # each block's maximum is its magnitude
    mag = np.where(rng.random(shape[:-1] + (4,)) < 0.5, 2.0 ** -8, 4094.0)
    if edge != "inside":
        odd = (np.arange(shape[2]) % 37 == 5)[None, None, :, None] & (rng.random(shape[:-1] + (4,)) < 0.5)
        mag = np.where(odd, 0.75 * 2.0 ** -8 if edge == "below" else 4096.0, mag)
    v = (u * mag[..., None]).reshape(shape).astype(np.float16)
    w["values"] = v.view(np.uint16)
    log(f"v8 fused conversion edges: {edge}")
    dev = to_dev(w)
    gc, oc = _pack_both(w, dev)
    compare_caches(gc, oc, w["P"])
    out, lse = ada.decode(gc, dev["q"], w["scale"])
    o_ref, l_ref = O.decode(oc, w["q"], w["scale"])
    check_outputs(out.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref)


def test_decode_chunkings_agree():
    w = _v8(W.config("llama8b", ctx=1500, batch=2), 0.5)
    dev = to_dev(w)
    gc, oc = _pack_both(w, dev)
    o_ref, l_ref = O.decode(oc, w["q"], w["scale"])
    for cp in (1, 4, 7, 1000):
        gc.cfg = _cfg(w, decode_chunk_pages=cp)
        out, lse = ada.decode(gc, dev["q"], w["scale"])
        check_outputs(out.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref)


def _codec_values(rng, n):
    """value rows exercising the codec: half-way cases, the clamp, zero,
    subnormal and large blocks, and random magnitudes per block"""
    rows = []
    for i in range(n):
        v = (rng.standard_normal(128) * np.exp(rng.uniform(-6, 6, 4)).repeat(32)).astype(np.float16)
        kind = i % 6
        if kind == 1:                                           # exact half steps of the 2^-6 grid
            v[:32] = np.float16(1.0)
            v[1:32] = (np.arange(31) + 0.5).astype(np.float16) / 64
        elif kind == 2:                                         # the clamp (127.5 steps)
            v[32:64] = np.float16(255 / 128) * np.sign(rng.standard_normal(32)).astype(np.float16)
        elif kind == 3:
            v[64:96] = 0
            v[96:] = np.float16(2 ** -20) * rng.integers(-3, 4, 32).astype(np.float16)
        elif kind == 4:
            v[:] = (rng.standard_normal(128) * 3e4).clip(-65000, 65000).astype(np.float16)
        rows.append(v.view(np.uint16))
    return np.array(rows)


def test_append_codec_cases_bit_exact():
    w = W.config("ragged", ctx=400, batch=3)
    gc = _gcache(w)
    oc = oracle_cache(w)
    rng = np.random.default_rng(9)
    flat_k = w["keys"].reshape(-1, 128)
    for n in [1, 37, 700, 1500]:
        seq = rng.integers(0, w["B"], n).astype(np.int32)
        head = rng.integers(0, w["Hkv"], n).astype(np.int32)
        tier = rng.integers(0, 6, n).astype(np.uint8)
        keys = flat_k[rng.integers(0, flat_k.shape[0], n)]
        vals = _codec_values(rng, n)
        ada.encode_append(gc, torch.from_numpy(seq).cuda(), torch.from_numpy(head).cuda(),
                          torch.from_numpy(tier).cuda(), torch.from_numpy(keys).cuda(),
                          torch.from_numpy(vals.view(np.int16)).cuda())
        assert ada.read_status(gc.status) == ada.OK
        assert O.append(oc, seq, head, tier, keys, vals) == O.OK
        compare_caches(gc, oc, w["P"])
    dev_q = torch.from_numpy(w["q"]).cuda()
    out, lse = ada.decode(gc, dev_q, w["scale"])
    o_ref, l_ref = O.decode(oc, w["q"], w["scale"])
    check_outputs(out.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref)


def test_fused_append_decode():
    w = _v8(W.config("llama8b", ctx=700, batch=2), 0.5)
    dev = to_dev(w)
    gc, oc = _pack_both(w, dev)
    rows = w["B"] * w["Hkv"]
    seq, head = np.repeat(np.arange(w["B"]), w["Hkv"]), np.tile(np.arange(w["Hkv"]), w["B"])
    rng = np.random.default_rng(12)
    for step in range(3):
        keys = rng.standard_normal((w["B"], w["Hkv"], 128), dtype=np.float32)
        vals = _codec_values(rng, rows).reshape(w["B"], w["Hkv"], 128)
        tiers = rng.integers(0, 6, (w["B"], w["Hkv"])).astype(np.uint8)
        q = rng.standard_normal((w["B"], w["Hq"], 128), dtype=np.float32)
        out, lse = ada.decode_append(gc, torch.from_numpy(q).cuda(), w["scale"], torch.from_numpy(keys).cuda(),
                                     torch.from_numpy(vals.view(np.int16)).cuda(), torch.from_numpy(tiers).cuda())
        assert ada.read_status(gc.status) == ada.OK
        assert O.append(oc, seq, head, tiers.ravel(), keys.reshape(rows, 128), vals.reshape(rows, 128)) == O.OK
        compare_caches(gc, oc, w["P"])
        o_ref, l_ref = O.decode(oc, q, w["scale"])
        check_outputs(out.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref)


def test_multi_query_and_utility():
    w = _v8(W.config("llama8b", ctx=900, batch=2), 0.5)
    dev = to_dev(w)
    gc, oc = _pack_both(w, dev)
    q2 = np.random.default_rng(3).standard_normal((w["B"], 2, w["Hq"], 128), dtype=np.float32)
    out, lse = ada.decode_multi(gc, torch.from_numpy(q2).cuda(), w["scale"])
    for qi in range(2):
        o_ref, l_ref = O.decode(oc, np.ascontiguousarray(q2[:, qi]), w["scale"])
        check_outputs(out[:, qi].cpu().numpy(), lse[:, qi].cpu().numpy(), o_ref, l_ref)
    out, lse, util = ada.decode_utility(gc, dev["q"], w["scale"])
    ref = O.decode_utility(oc, w["q"], w["scale"])
    u = util.cpu().numpy().astype(np.float64)
    kept = ~np.isnan(ref)
    assert np.array_equal(kept, ~np.isnan(u))
    for row in range(w["B"] * w["Hkv"]):
        pages = oc.page_table[row, : oc.num_pages[row]]
        if pages.size:
            ur, ug = ref[pages][kept[pages]], u[pages][kept[pages]]
            assert np.max(np.abs(ug - ur)) <= TOL * np.max(ur), row


def test_rdr_v8_chain_matches_oracle():
    w = W.config("rdr128k", ctx=3000, batch=2)
    mask = 0b111001                                      # T2V8, T4V8, T8V8, T8
    cfg = _cfg(w, rdr_tier_mask=mask)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    # 40% and 95% of the all-T8 bytes: the second reaches the T8 step
    budget = [int(f * O.tier_rate(0) * w["Hkv"] * int(c)) for f, c in zip((0.4, 0.95), w["ctx_len"])]
    t = ada.rdr_assign(cfg, w["ctx_len"], torch.from_numpy(w["utility"]).cuda(), budget, status)
    assert ada.read_status(status) == ada.OK
    st, t_ref = O.rdr_assign(w["ctx_len"], w["utility"], np.array(budget), tier_mask=mask)
    assert st == O.OK
    assert np.array_equal(t.cpu().numpy(), t_ref)
    assert (t_ref >= 3).any() and (t_ref == 0).any()


@pytest.mark.parametrize("name,ctx,batch,frac", [("llama8b", 900, 2, 0.45), ("ragged", 1200, 3, 0.35)])
def test_repack_into_v8_chain(name, ctx, batch, frac):
    w = W.config(name, ctx=ctx, batch=batch)
    dev = to_dev(w)
    gsrc, osrc = _pack_both(w, dev)
    util = np.exp(np.random.default_rng(8).standard_normal((osrc.page_capacity, w["P"]))).astype(np.float32)
    cur = [sum(O.tier_rate(int(x)) for x in w["tiers"][b].ravel() if x >= 0) for b in range(w["B"])]
    budget = [int(frac * r) for r in cur]
    mask = 0b111000
    gdst = _gcache(w, cfg=_cfg(w, rdr_tier_mask=mask))
    gsrc.cfg = _cfg(w, rdr_tier_mask=mask)
    ada.repack(gsrc, w["B"], torch.from_numpy(util).cuda(), budget, gdst)
    assert ada.read_status(gdst.status) == ada.OK
    odst = oracle_cache(w)
    st, tv = O.repack(osrc, w["B"], util, budget, odst, tier_mask=mask)
    assert st == O.OK and (tv >= 3).any()
    compare_caches(gdst, odst, w["P"])
    out, lse = ada.decode(gdst, dev["q"], w["scale"])
    o_ref, l_ref = O.decode(odst, w["q"], w["scale"])
    check_outputs(out.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref)
    # V8 -> V8 with an unlimited budget reproduces the re-packed cache
    g2 = _gcache(w, cfg=_cfg(w, rdr_tier_mask=mask))
    gdst.cfg = _cfg(w, rdr_tier_mask=mask)
    ada.repack(gdst, w["B"], torch.from_numpy(util).cuda(), [1 << 40] * w["B"], g2)
    assert ada.read_status(g2.status) == ada.OK
    compare_caches(g2, odst, w["P"])


def test_errors():
    w = W.config("llama8b", ctx=64, batch=1)
    dev = to_dev(w)
    t = np.where(w["tiers"] >= 0, w["tiers"] + 3, -1).astype(np.int8)
    # a cache without value tiers rejects tiers 3-5
    plain = ada.Cache(ada.make_config(w["P"], w["Hq"], w["Hkv"]), w["B"], *dims(w))
    ada.cache_init(plain)
    ada.pack(plain, w["ctx_len"], torch.from_numpy(t).cuda(), dev["keys"], dev["values"])
    assert ada.read_status(plain.status) == ada.EINVAL
    # a non-finite value of a V8 token: nothing written
    gc = _gcache(w)
    before = gc.host()
    vals = w["values"].copy()
    kept = np.argwhere(t[0, 0] >= 0)[0, 0]
    vals[0, 0, kept, 5] = np.float16(np.nan).view(np.uint16)
    ada.pack(gc, w["ctx_len"], torch.from_numpy(t).cuda(), dev["keys"], torch.from_numpy(vals.view(np.int16)).cuda())
    assert ada.read_status(gc.status) == ada.EINVAL
    after = gc.host()
    for k in before:
        assert np.array_equal(before[k], after[k]), k
    # V8 tiers in the RDR mask need value_tiers
    with pytest.raises(ada.AdaError):
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        ada.rdr_assign(ada.make_config(w["P"], w["Hq"], w["Hkv"], rdr_tier_mask=0b111000), w["ctx_len"],
                       torch.ones((1, w["Hkv"], 64), dtype=torch.float32, device="cuda"), [1000], status)


def test_fullsize_llama8b_all_v8():
    """The full llama8b layer with every kept token's values in V8 (the
    configuration `bench.py --v8` times, automatic chunking): pages byte
    for byte and every output row within the tolerance."""
    w = _v8(W.config("llama8b"), 1.0)
    log("v8 full llama8b: pack both")
    dev = to_dev(w)
    gc, oc = _pack_both(w, dev)
    compare_caches(gc, oc, w["P"])
    # footprint: a V8 page's block is its key part plus 132 value bytes per
    # slot, so the arena holds exactly that for every page
    P = w["P"]
    n_pages = int(gc.alloc[0].item())
    tiers = gc.page_meta[:n_pages, 0].cpu().numpy()
    assert (tiers >= 3).all()
    key_bytes = {3: 130, 4: 66, 5: 42}
    assert int(gc.alloc[1].item()) * 16 == sum(P * (key_bytes[int(t)] + 132) for t in tiers)
    kept = int((w["tiers"] >= 0).sum())
    log(f"  arena bytes per kept token-head {int(gc.alloc[1].item()) * 16 / kept:.1f}")
    log("  decode")
    out, lse = ada.decode(gc, dev["q"], w["scale"])
    o_ref, l_ref = O.decode(oc, w["q"], w["scale"])
    worst = check_outputs(out.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref)
    log(f"  worst row rel err {worst:.2e}")
