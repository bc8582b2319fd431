"""Pins of the oracle's page layout, bulk pack and append: a hand-derived
page, an address computation written independently from the layout rules,
structural invariants, pack == sequential append, and all-or-nothing errors.

The pages (SPHERICAL KV abstract, newx.sg and searcharxiv pages) ask for
tier-homogeneous pages with lightweight metadata and coalesced reads; the
concrete byte layout is this library's reading of that."""
import json
import os

import numpy as np
import pytest

import workloads as W
from oracle import oracle as O
from tests.util import kept_tokens, upper_capacity

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BLOCK16_MAX = {16: 386, 32: 772}   # T8 key part + fp16 values, in 16-byte units


def _cache_for(w, per_row=None, pages=None, units=None):
    a, b, c = upper_capacity(w, BLOCK16_MAX[w["P"]])
    return O.Cache(w["P"], w["Hq"], w["Hkv"], w["B"], per_row or a, pages or b, units or c)


def test_block_sizes_closed_form():
    # key part: radius 2 B + angle 8*tb B + magnitude 8*sb B per token;
    # value part: 256 B (fp16) or 132 B (V8) per token
    assert [O.key_bytes(t, 16) for t in (0, 1, 2)] == [2080, 1056, 672]
    assert [O.key_bytes(t, 32) for t in (0, 1, 2)] == [4160, 2112, 1344]
    assert [O.block_bytes(t, 16) for t in (0, 1, 2)] == [2080 + 4096, 1056 + 4096, 672 + 4096]
    assert [O.block_bytes(t, 32) for t in (0, 1, 2)] == [4160 + 8192, 2112 + 8192, 1344 + 8192]
    assert [O.block_bytes(t, 16) for t in (3, 4, 5)] == [2080 + 2112, 1056 + 2112, 672 + 2112]
    assert [O.key_bytes(t, 16) for t in (3, 4, 5)] == [2080, 1056, 672]


def test_hand_derived_t2_page():
    with open(os.path.join(GOLDEN, "t2_page_block.json")) as f:
        g = json.load(f)
    w = W.config("tiny", ctx=4)
    w["keys"][:] = 0
    k3 = np.zeros(128, np.float32)
    k3[0:126:2] = -1.0
    k3[127] = 1.0
    w["keys"][0, 0, 3] = k3
    tiers = np.full((1, 1, 4), 2, np.int8)
    c = _cache_for(w)
    assert O.pack(c, w["ctx_len"], tiers, w["keys"], w["values"]) == O.OK
    expect = np.zeros(g["block_bytes"], np.uint8)
    for start, vals in g["ranges"]:
        expect[start:start + len(vals)] = vals
    tier, count, off16 = c.meta(0)
    assert (tier, count, off16) == (2, 4, 0)
    assert np.array_equal(c.arena[: g["block_bytes"]], expect)


def _spec_addr(tier, P, slot, comp, byte):
    """byte address inside a page's code block, computed from the layout
    rules (radius | angle units | magnitude units, token-minor units)."""
    tb, sb = O.TIER_BITS[tier]
    Bt, Bs = 8 * tb, 8 * sb
    base = 2 * P if comp == "theta" else 2 * P + P * Bt
    Bc = Bt if comp == "theta" else Bs
    unit, within = divmod(byte, 16)
    if unit < Bc // 16:
        return base + unit * 16 * P + slot * 16 + within
    return base + (Bc // 16) * 16 * P + slot * 8 + within


@pytest.mark.parametrize("name,ctx,batch", [("llama8b", 300, 2), ("long256k", 160, 1), ("ragged", 200, 3)])
def test_pack_structure(name, ctx, batch):
    w = W.config(name, ctx=ctx, batch=batch)
    c = _cache_for(w)
    assert O.pack(c, w["ctx_len"], w["tiers"], w["keys"], w["values"]) == O.OK
    P = w["P"]
    next_page, next_unit = 0, 0
    seen = 0
    for b in range(w["B"]):
        for h in range(w["Hkv"]):
            row = b * w["Hkv"] + h
            toks = kept_tokens(w, b, h)
            pages = c.page_table[row, : c.num_pages[row]]
            i = 0
            for pi, page in enumerate(pages):
                assert page == next_page                        # consecutive page ids
                next_page += 1
                tier, count, off16 = c.meta(page)
                assert off16 == next_unit                       # consecutive code blocks
                next_unit += O.block_bytes(tier, P) // 16
                assert 1 <= count <= P
                block = c.arena[off16 * 16: off16 * 16 + O.block_bytes(tier, P)]
                for slot in range(P):
                    if slot >= count:                           # unused slots are zero
                        assert block[2 * slot] == 0 and block[2 * slot + 1] == 0
                        continue
                    pos, tau = toks[i]
                    i += 1
                    assert tau == tier                          # tier-homogeneous
                    tb, sb = O.TIER_BITS[tier]
                    r16, th, s, _ = O.encode(w["keys"][b, h, pos], tb, sb)
                    assert int(block[2 * slot]) | (int(block[2 * slot + 1]) << 8) == int(r16[0])
                    bt = bytes(block[_spec_addr(tier, P, slot, "theta", k)] for k in range(8 * tb))
                    bs = bytes(block[_spec_addr(tier, P, slot, "s", k)] for k in range(8 * sb))
                    assert bt == O.bits_put(th[0], tb).tobytes()
                    assert bs == O.bits_put(s[0], sb).tobytes()
                    # values: element (slot, d) at (slot/8)*1024 + d*8 + slot%8
                    vp = O.value_part(c, page).view(np.uint16).reshape(P // 8, 128, 8)
                    assert np.array_equal(vp[slot // 8, :, slot % 8], w["values"][b, h, pos])
                    seen += 1
            assert i == len(toks)                               # each kept token exactly once
            # open pages: last page of each tier if not full
            for tau in range(3):
                tp = [p for p in pages if c.meta(p)[0] == tau]
                want = tp[-1] if tp and c.meta(tp[-1])[1] < P else -1
                assert c.open_page[row, tau] == want
    assert c.alloc[0] == next_page and c.alloc[1] == next_unit
    assert seen == int((w["tiers"] >= 0).sum())


def test_pack_equals_sequential_append():
    w = W.config("ragged", ctx=150, batch=3)
    c1 = _cache_for(w)
    assert O.pack(c1, w["ctx_len"], w["tiers"], w["keys"], w["values"]) == O.OK
    c2 = _cache_for(w)
    seq, head, tier, ks, vs = [], [], [], [], []
    for b in range(w["B"]):
        for h in range(w["Hkv"]):
            for pos, tau in kept_tokens(w, b, h):
                seq.append(b); head.append(h); tier.append(tau)
                ks.append(w["keys"][b, h, pos]); vs.append(w["values"][b, h, pos])
    # append in several calls to exercise state carried between calls
    n = len(seq)
    for a, z in [(0, n // 3), (n // 3, n // 2), (n // 2, n)]:
        assert O.append(c2, seq[a:z], head[a:z], tier[a:z], np.array(ks[a:z]), np.array(vs[a:z])) == O.OK
    for name in ("page_table", "num_pages", "open_page", "page_meta", "arena", "alloc"):
        assert np.array_equal(getattr(c1, name), getattr(c2, name)), name


def test_append_interleaved_tiers_and_open_pages():
    w = W.config("tiny", ctx=64)
    c = _cache_for(w)
    rng = np.random.default_rng(0)
    tiers = rng.integers(0, 3, 50).astype(np.uint8)
    st = O.append(c, np.zeros(50, np.int32), np.zeros(50, np.int32), tiers,
                  w["keys"][0, 0, :50], w["values"][0, 0, :50])
    assert st == O.OK
    # row order = order in which pages were opened; each tier's tokens in request order
    P = 16
    counts = {t: int((tiers == t).sum()) for t in range(3)}
    pages = c.page_table[0, : c.num_pages[0]]
    assert len(pages) == sum(-(-n // P) for n in counts.values())
    for t in range(3):
        tp = [p for p in pages if c.meta(p)[0] == t]
        assert sum(c.meta(p)[1] for p in tp) == counts[t]
        assert c.open_page[0, t] == (tp[-1] if counts[t] % P else -1)


def test_capacity_errors_write_nothing():
    w = W.config("llama8b", ctx=256, batch=1)
    a, b, u = upper_capacity(w, 386)
    for kw in [dict(pages=5), dict(units=100), dict(per_row=3)]:
        c = _cache_for(w, **kw)
        before = c.copy()
        assert O.pack(c, w["ctx_len"], w["tiers"], w["keys"], w["values"]) == O.ENOSPC
        for name in ("page_table", "num_pages", "open_page", "page_meta", "arena", "alloc"):
            assert np.array_equal(getattr(c, name), getattr(before, name))
    c = _cache_for(w, pages=2)
    before = c.copy()
    keys = w["keys"][0, 0, :40]
    assert O.append(c, np.zeros(40, np.int32), np.zeros(40, np.int32), np.ones(40, np.uint8),
                    keys, w["values"][0, 0, :40]) == O.ENOSPC
    assert np.array_equal(c.alloc, before.alloc) and np.array_equal(c.arena, before.arena)


def test_invalid_inputs_write_nothing():
    w = W.config("llama8b", ctx=128, batch=1)
    c = _cache_for(w)
    before = c.copy()
    bad = w["tiers"].copy()
    bad[0, 0, 5] = O.NUM_TIERS
    assert O.pack(c, w["ctx_len"], bad, w["keys"], w["values"]) == O.EINVAL
    # a non-finite value cannot be put into a V8 tier (fp16 tiers store it as is)
    vals = w["values"].copy()
    kept = np.argwhere(w["tiers"][0, 0] >= 0)[0, 0]
    vals[0, 0, kept, 7] = np.float16(np.inf).view(np.uint16)
    v8 = np.where(w["tiers"] >= 0, w["tiers"] + 3, -1).astype(np.int8)
    assert O.pack(c, w["ctx_len"], v8, w["keys"], vals) == O.EINVAL
    keys = w["keys"].copy()
    kept = np.argwhere(w["tiers"][0, 0] >= 0)[0, 0]
    keys[0, 0, kept, 3] = np.nan
    assert O.pack(c, w["ctx_len"], w["tiers"], keys, w["values"]) == O.EINVAL
    assert np.array_equal(c.arena, before.arena) and np.array_equal(c.alloc, before.alloc)
    # a non-finite key at a dropped position is never read
    dropped = np.argwhere(w["tiers"][0, 0] < 0)[0, 0]
    keys = w["keys"].copy()
    keys[0, 0, dropped, :] = np.inf
    assert O.pack(c, w["ctx_len"], w["tiers"], keys, w["values"]) == O.OK
    # append: out-of-range sequence / head / tier
    for s, h, t in [(1, 0, 0), (0, 8, 0), (0, 0, O.NUM_TIERS)]:
        c2 = _cache_for(w)
        assert O.append(c2, [s], [h], [t], w["keys"][0, 0, :1], w["values"][0, 0, :1]) == O.EINVAL
