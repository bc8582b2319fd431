"""Pins of the oracle's value tiers (ids 3-5: keys of T8 / T4 / T2 with V8
values) and their V8 value codec: blocks of 32 values share a power-of-two
scale 2^(e-6), e = floor(log2 max|v|) (at least -18), elements are
round-half-even(v 2^(6-e)) clamped to +-127.

The codec is pinned by closed forms (powers of two, exact half-way cases,
the clamp, zero and tiny blocks), by its error bound (at most half a step,
one step where clamped), by idempotence (decoded values re-encode to the
same bytes) and by block independence.  Pages: the V8 page bytes sit where
the layout puts them, decode equals dense attention over the dequantised
keys and decoded values, RDR over a V8 chain is optimal by brute force, and
re-packing fp16 tiers into V8 tiers quantises the values as the codec does."""
import itertools

import numpy as np
import pytest

import workloads as W
from oracle import oracle as O
from tests.util import dense_attention, dequantize, kept_tokens, upper_capacity

F16 = lambda x: np.asarray(x, np.float16).view(np.uint16)


def _block(vals, k=0):
    v = np.zeros(128, np.float16)
    v[32 * k: 32 * k + len(vals)] = vals
    return v.view(np.uint16)


def test_powers_of_two_and_full_scale():
    for e in (-10, -3, 0, 4, 15):
        v = _block([2.0 ** e, -(127 / 64) * 2.0 ** e, 2.0 ** (e - 6), 0.0])
        st, sb, c = O.v8_encode(v)
        assert st == O.OK and sb[0] == e + 127
        assert list(c[:4]) == [64, -127, 1, 0]
        assert np.array_equal(O.v8_decode(sb, c)[:4], np.float16(v[:4].view(np.float16)).astype(np.float64))


def test_half_way_rounds_to_even_and_clamp():
    # amax 1 -> step 2^-6: 1.5, 2.5, -3.5 steps round to 2, 2, -4
    v = _block([1.0, 1.5 / 64, 2.5 / 64, -3.5 / 64])
    st, sb, c = O.v8_encode(v)
    assert st == O.OK and list(c[:4]) == [64, 2, 2, -4]
    # amax 255/128 -> 127.5 steps -> clamped to 127, both signs
    v = _block([255 / 128, -255 / 128])
    st, sb, c = O.v8_encode(v)
    assert sb[0] == 127 and list(c[:2]) == [127, -127]


def test_zero_and_tiny_blocks():
    st, sb, c = O.v8_encode(np.zeros(128, np.uint16))
    assert st == O.OK and list(sb) == [109] * 4 and not c.any()
    tiny = _block([2.0 ** -20, -3 * 2.0 ** -24], k=2)     # fp16 subnormals; the exponent floor is -18
    st, sb, c = O.v8_encode(tiny)
    assert sb[2] == 109 and list(c[64:66]) == [16, -3]
    assert np.array_equal(O.v8_decode(sb, c)[64:66], [2.0 ** -20, -3 * 2.0 ** -24])


def test_non_finite_rejected():
    for bad in (np.inf, -np.inf, np.nan):
        v = np.zeros(128, np.float16)
        v[77] = bad
        assert O.v8_encode(v.view(np.uint16))[0] == O.EINVAL


def test_error_bound_idempotence_and_block_independence():
    rng = np.random.default_rng(0)
    for _ in range(300):
        v = (rng.standard_normal(128) * np.exp(rng.uniform(-8, 8, 4)).repeat(32)).astype(np.float16)
        bits = v.view(np.uint16)
        st, sb, c = O.v8_encode(bits)
        assert st == O.OK
        d = O.v8_decode(sb, c)
        x = v.astype(np.float64)
        for k in range(4):
            blk = slice(32 * k, 32 * k + 32)
            e = int(sb[k]) - 127
            step = 2.0 ** (e - 6)
            err = np.abs(x[blk] - d[blk])
            clamped = np.abs(c[blk]) == 127
            assert np.all(err[~clamped] <= step / 2) and np.all(err[clamped] <= step)
            amax = np.max(np.abs(x[blk]))
            assert amax == 0 or 2.0 ** e <= amax < 2.0 ** (e + 1) or e == -18
        # decoded values are fp16 numbers and re-encode to the same bytes
        d16 = d.astype(np.float16)
        assert np.array_equal(d16.astype(np.float64), d)
        st2, sb2, c2 = O.v8_encode(d16.view(np.uint16))
        assert np.array_equal(sb2, sb) and np.array_equal(c2, c)
        # another block's values do not change this block's bytes
        v2 = v.copy()
        v2[32:64] *= np.float16(3)
        _, sb3, c3 = O.v8_encode(v2.view(np.uint16))
        assert sb3[0] == sb[0] and np.array_equal(c3[:32], c[:32])


def _v8_workload(name, ctx, batch):
    w = W.config(name, ctx=ctx, batch=batch)
    t = w["tiers"].copy()
    rng = np.random.default_rng(3)
    shift = rng.integers(0, 2, t.shape) * 3                 # about half the kept tokens get V8 values
    w["tiers"] = np.where(t >= 0, t + shift, -1).astype(np.int8)
    return w


def _pack(w):
    per_row, pages, units = upper_capacity(w, 386 * w["P"] // 16)
    c = O.Cache(w["P"], w["Hq"], w["Hkv"], w["B"], per_row, pages, units)
    assert O.pack(c, w["ctx_len"], w["tiers"], w["keys"], w["values"]) == O.OK
    return c


def test_v8_page_bytes_follow_the_layout():
    w = _v8_workload("llama8b", 64, 1)
    c = _pack(w)
    P = w["P"]
    for row in range(w["Hkv"]):
        toks = iter(kept_tokens(w, 0, row))
        for i in range(c.num_pages[row]):
            page = c.page_table[row, i]
            tier, count, _ = c.meta(page)
            raw = O.value_part(c, page)
            assert raw.size == (256 if O.VALUE_BITS[tier] == 16 else 132) * P   # value bytes per token
            for slot in range(count):
                pos, tau = next(toks)
                assert tau == tier
                if O.VALUE_BITS[tier] == 16:
                    continue
                st, sb, codes = O.v8_encode(w["values"][0, row, pos])
                # 16-token groups of 2112 bytes: [16 tokens][4] scale bytes,
                # then [128 dims][16 tokens] code bytes
                g, r = slot // 16, slot % 16
                assert [raw[g * 2112 + r * 4 + k] for k in range(4)] == list(sb)
                assert np.array_equal(raw[g * 2112 + 64 + np.arange(128) * 16 + r].astype(np.int16) - 128, codes)
            if O.VALUE_BITS[tier] == 8:   # bytes of empty slots and past the V8 layout stay zero
                used = np.zeros(raw.size, bool)
                for slot in range(count):
                    g, r = slot // 16, slot % 16
                    used[g * 2112 + r * 4 + np.arange(4)] = True
                    used[g * 2112 + 64 + np.arange(128) * 16 + r] = True
                assert not raw[~used].any()


def test_decode_equals_dense_attention_over_decoded_values():
    w = _v8_workload("ragged", 300, 3)
    c = _pack(w)
    out, lse = O.decode(c, w["q"], w["scale"])
    G = w["Hq"] // w["Hkv"]
    for b in range(w["B"]):
        for h in range(w["Hkv"]):
            kh, vh = [], []
            for pos, tau in kept_tokens(w, b, h):
                tb, sb = O.TIER_BITS[tau]
                r16, th, s, _ = O.encode(w["keys"][b, h, pos], tb, sb)
                kh.append(dequantize(r16[0], th[0], s[0], tb, sb))
                v = w["values"][b, h, pos]
                if O.VALUE_BITS[tau] == 8:
                    _, scb, cc = O.v8_encode(v)
                    vh.append(O.v8_decode(scb, cc))
                else:
                    vh.append(v.view(np.float16).astype(np.float64))
            kh, vh = np.array(kh).reshape(-1, 128), np.array(vh).reshape(-1, 128)
            for g in range(G):
                o_ref, l_ref = dense_attention(kh, vh, w["q"][b, h * G + g], w["scale"])
                if kh.shape[0] == 0:
                    assert lse[b, h * G + g] == -np.inf
                    continue
                assert np.max(np.abs(out[b, h * G + g] - o_ref)) <= 1e-12 * np.max(np.abs(o_ref))


def test_rdr_chains():
    assert O.rdr_steps(0b111000)[0] == O.OK                 # T8V8, T4V8, T2V8
    assert O.rdr_steps(0b111001)[0] == O.OK                 # ... and T8 on top
    assert O.rdr_steps(0b111111)[0] == O.EUNSUPPORTED       # T2 (298 B) is worse than T8V8 (262 B)
    assert O.rdr_steps(1 << 6)[0] == O.EINVAL
    st, tiers, dR, c = O.rdr_steps(0b111001)
    assert list(tiers) == [5, 4, 3, 0] and list(dR) == [174, 24, 64, 124]


@pytest.mark.parametrize("seed", range(4))
def test_rdr_v8_chain_brute_force(seed):
    rng = np.random.default_rng(200 + seed)
    n, mask = 6, 0b111001
    chain = [-1, 5, 4, 3, 0]
    rate = {t: (O.tier_rate(t) if t >= 0 else 0) for t in chain}
    dist = {-1: 1.0}
    for t in chain[1:]:
        tb, sb = O.TIER_BITS[t]
        dist[t] = 2.0 ** -(tb + sb) + (2.0 ** -14 if O.VALUE_BITS[t] == 8 else 0.0)
    util = np.exp(rng.standard_normal(n)).astype(np.float32)
    budget = int(rng.integers(0, 386 * n))
    st, tiers = O.rdr_assign(np.array([n], np.int32), util[None, None], np.array([budget]), tier_mask=mask)
    assert st == O.OK
    t = [int(x) for x in tiers[0, 0]]
    Rg = sum(rate[x] for x in t)
    Dg = sum(float(u) * dist[x] for u, x in zip(util, t))
    assert Rg <= budget
    for combo in itertools.product(chain, repeat=n):
        if sum(rate[x] for x in combo) <= Rg:
            assert sum(float(u) * dist[x] for u, x in zip(util, combo)) >= Dg - 1e-12 * max(1.0, Dg)


def test_repack_into_v8_chain():
    w = W.config("llama8b", ctx=256, batch=2)
    src = _pack(w)
    per_row, pages, units = upper_capacity(w, 386 * w["P"] // 16)
    dst = O.Cache(w["P"], w["Hq"], w["Hkv"], w["B"], per_row, pages, units)
    util = np.exp(np.random.default_rng(5).standard_normal((src.page_capacity, w["P"]))).astype(np.float32)
    cur = [sum(O.tier_rate(int(x)) for x in w["tiers"][b].ravel() if x >= 0) for b in range(w["B"])]
    budget = [int(0.5 * r) for r in cur]
    st, tv = O.repack(src, w["B"], util, budget, dst, tier_mask=0b111000)
    assert st == O.OK
    P = w["P"]
    for b in range(w["B"]):
        assert sum(O.tier_rate(int(x)) for x in tv[b].ravel() if x >= 0) <= budget[b]
    for row in range(w["B"] * w["Hkv"]):
        b, h = divmod(row, w["Hkv"])
        for t in np.nonzero(tv[b, h] >= 0)[0]:
            told = int(src.page_meta[src.page_table[row, t // P], 0])
            tnew = int(tv[b, h, t])
            assert tnew >= 3 and O.TIER_BITS[tnew][0] <= O.TIER_BITS[told][0]   # V8 values, keys no finer
    # the re-packed cache decodes like dense attention over transcoded keys and V8 values
    out, lse = O.decode(dst, w["q"], w["scale"])
    G = w["Hq"] // w["Hkv"]
    for b in range(w["B"]):
        for h in range(w["Hkv"]):
            row = b * w["Hkv"] + h
            keys, vals = [], []
            for tau in range(O.NUM_TIERS):
                for t in np.nonzero(tv[b, h] == tau)[0]:
                    page = src.page_table[row, t // P]
                    told = int(src.page_meta[page, 0])
                    r16, th, s, _ = O.read_token(src, page, t % P)
                    th_n, s_n = O.transcode(told, tau, th, s)
                    tb, sb = O.TIER_BITS[tau]
                    keys.append(dequantize(r16, th_n[0], s_n[0], tb, sb))
                    v16 = O.read_values(src, page, t % P).astype(np.float16).view(np.uint16)
                    _, scb, cc = O.v8_encode(v16)
                    vals.append(O.v8_decode(scb, cc))
            keys, vals = np.array(keys).reshape(-1, 128), np.array(vals).reshape(-1, 128)
            for g in range(G):
                o_ref, _ = dense_attention(keys, vals, w["q"][b, h * G + g], w["scale"])
                if keys.shape[0]:
                    assert np.max(np.abs(out[b, h * G + g] - o_ref)) <= 1e-12 * np.max(np.abs(o_ref))
    # V8 -> V8 with an unlimited budget reproduces the re-packed cache byte for byte
    dst2 = O.Cache(w["P"], w["Hq"], w["Hkv"], w["B"], per_row, pages, units)
    st, _ = O.repack(dst, w["B"], util, [1 << 40] * w["B"], dst2, tier_mask=0b111000)
    assert st == O.OK
    for k in ("page_table", "num_pages", "open_page", "page_meta", "arena", "alloc"):
        assert np.array_equal(getattr(dst, k), getattr(dst2, k)), k
