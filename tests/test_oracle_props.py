"""Property tests of the oracle (hypothesis): random small caches -- page
size, heads and grouping, ragged context lengths, tier mixes over all six
tiers, empty heads, both pair layouts -- must satisfy what the method fixes
whatever the draw:

* pack: every kept token sits in exactly one slot of a page of its tier, in
  (tier id, position) order, and unused slots are zero;
* append of the same tokens one at a time, in pack order, gives the same
  cache as pack;
* decode equals plain softmax attention over the dequantised keys and the
  decoded values (fp64, 1e-12), and heads without a kept token give o = 0,
  lse = -inf;
* utility sums to G over every row with kept tokens."""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import oracle as O
from tests.util import dense_attention, dequantize

SETTINGS = settings(max_examples=30, deadline=None, suppress_health_check=list(HealthCheck))


@st.composite
def caches(draw):
    P = draw(st.sampled_from([16, 32]))
    Hkv = draw(st.integers(1, 3))
    G = draw(st.sampled_from([1, 2, 4]))
    B = draw(st.integers(1, 3))
    stride = draw(st.integers(1, 80))
    seed = draw(st.integers(0, 2 ** 32 - 1))
    layout = draw(st.sampled_from([0, 1]))
    rng = np.random.default_rng(seed)
    ctx = rng.integers(0, stride + 1, B).astype(np.int32)
    p_drop = draw(st.floats(0.0, 1.0))
    tiers = rng.integers(0, 6, (B, Hkv, stride)).astype(np.int8)
    tiers[rng.random(tiers.shape) < p_drop] = -1
    if draw(st.booleans()):
        tiers[rng.integers(0, B), rng.integers(0, Hkv)] = -1            # an empty head
    keys = (rng.standard_normal((B, Hkv, stride, 128)) * np.exp(rng.standard_normal((B, Hkv, stride, 1)))).astype(
        np.float32)
    values = rng.standard_normal((B, Hkv, stride, 128)).astype(np.float16).view(np.uint16)
    q = rng.standard_normal((B, Hkv * G, 128)).astype(np.float32)
    return dict(P=P, Hkv=Hkv, G=G, B=B, stride=stride, ctx=ctx, tiers=tiers, keys=keys, values=values, q=q,
                layout=layout)


def _kept(c, b, h):
    t = c["tiers"][b, h, : c["ctx"][b]]
    return [(int(p), tau) for tau in range(6) for p in np.nonzero(t == tau)[0]]


def _empty(c):
    per_row = -(-c["stride"] // c["P"]) + 6
    pages = c["B"] * c["Hkv"] * per_row
    return O.Cache(c["P"], c["Hkv"] * c["G"], c["Hkv"], c["B"], per_row, pages, pages * 386 * c["P"] // 16,
                   pair_layout=c["layout"])


@SETTINGS
@given(caches())
def test_pack_places_every_kept_token(c):
    oc = _empty(c)
    assert O.pack(oc, c["ctx"], c["tiers"], c["keys"], c["values"], nthreads=2) == O.OK
    P = c["P"]
    for b in range(c["B"]):
        for h in range(c["Hkv"]):
            row = b * c["Hkv"] + h
            slots = []
            for i in range(oc.num_pages[row]):
                page = oc.page_table[row, i]
                tier, count, _ = oc.meta(page)
                assert 1 <= count <= P
                slots += [(page, s, tier) for s in range(count)]
                raw = O.value_part(oc, page).view(np.uint16)
                if O.VALUE_BITS[tier] == 16:   # fp16 slots past the count are zero
                    for s in range(count, P):
                        assert not raw[(s // 8) * 1024 + np.arange(128) * 8 + s % 8].any()
            kept = _kept(c, b, h)
            assert [t for _, _, t in slots] == [tau for _, tau in kept]
            for (page, s, tier), (pos, tau) in zip(slots, kept):
                tb, sb = O.TIER_BITS[tau]
                r16, th, sc, _ = O.read_token(oc, page, s)
                r_e, th_e, s_e, st_e = O.encode(c["keys"][b, h, pos], tb, sb, pair_layout=c["layout"])
                assert st_e == O.OK and r16 == r_e[0]
                assert np.array_equal(th, th_e[0]) and np.array_equal(sc, s_e[0])


@SETTINGS
@given(caches())
def test_append_one_by_one_equals_pack(c):
    packed = _empty(c)
    assert O.pack(packed, c["ctx"], c["tiers"], c["keys"], c["values"], nthreads=2) == O.OK
    appended = _empty(c)
    for b in range(c["B"]):
        for h in range(c["Hkv"]):
            for pos, tau in _kept(c, b, h):
                st_a = O.append(appended, [b], [h], [tau], c["keys"][b, h, pos][None], c["values"][b, h, pos][None])
                assert st_a == O.OK
    n = int(packed.alloc[0])
    for k in ("num_pages", "alloc"):
        assert np.array_equal(getattr(packed, k), getattr(appended, k)), k
    for row in range(c["B"] * c["Hkv"]):
        assert np.array_equal(packed.page_table[row, : packed.num_pages[row]],
                              appended.page_table[row, : appended.num_pages[row]])
    assert np.array_equal(packed.page_meta[:n], appended.page_meta[:n])
    u = int(packed.alloc[1]) * 16
    assert np.array_equal(packed.arena[:u], appended.arena[:u])


@SETTINGS
@given(caches())
def test_decode_is_softmax_attention_over_decoded_tokens(c):
    oc = _empty(c)
    assert O.pack(oc, c["ctx"], c["tiers"], c["keys"], c["values"], nthreads=2) == O.OK
    scale = 128 ** -0.5
    out, lse = O.decode(oc, c["q"], scale, nthreads=2)
    util = O.decode_utility(oc, c["q"], scale, nthreads=2)
    G = c["G"]
    for b in range(c["B"]):
        for h in range(c["Hkv"]):
            kh, vh = [], []
            for pos, tau in _kept(c, b, h):
                tb, sb = O.TIER_BITS[tau]
                r16, th, s, _ = O.encode(c["keys"][b, h, pos], tb, sb, pair_layout=c["layout"])
                kh.append(dequantize(r16[0], th[0], s[0], tb, sb, half_split=c["layout"] == 1))
                v = c["values"][b, h, pos]
                if O.VALUE_BITS[tau] == 8:
                    _, scb, cc = O.v8_encode(v)
                    vh.append(O.v8_decode(scb, cc))
                else:
                    vh.append(v.view(np.float16).astype(np.float64))
            kh, vh = np.array(kh).reshape(-1, 128), np.array(vh).reshape(-1, 128)
            row = b * c["Hkv"] + h
            pages = oc.page_table[row, : oc.num_pages[row]]
            for g in range(G):
                hq = h * G + g
                if kh.shape[0] == 0:
                    assert lse[b, hq] == -np.inf and not out[b, hq].any()
                    continue
                o_ref, l_ref = dense_attention(kh, vh, c["q"][b, hq], scale)
                assert np.max(np.abs(out[b, hq] - o_ref)) <= 1e-12 * max(1.0, np.max(np.abs(o_ref)))
                assert abs(lse[b, hq] - l_ref) <= 1e-12 * max(1.0, abs(l_ref))
            if kh.shape[0]:
                total = sum(np.nansum(util[p]) for p in pages)
                assert abs(total - G) <= 1e-12 * G
