"""Pins of the oracle's per-token utility (attention mass) of one decode step.

u_t = sum over the KV head's query heads of the token's softmax weight.  It
must equal the same sum computed by plain numpy softmax over the dequantised
keys, sum to G over every row with kept tokens (each head's weights sum to
one), equal G for a lone token, and leave every other entry of the output
untouched."""
import numpy as np

import workloads as W
from oracle import oracle as O
from tests.util import dequantize, kept_tokens, upper_capacity

BLOCK16_MAX = {16: 386, 32: 772}   # T8 key part + fp16 values, in 16-byte units


def _pack(w, tiers=None):
    per_row, pages, units = upper_capacity(w, BLOCK16_MAX[w["P"]])
    c = O.Cache(w["P"], w["Hq"], w["Hkv"], w["B"], per_row, pages, units)
    assert O.pack(c, w["ctx_len"], w["tiers"] if tiers is None else tiers, w["keys"], w["values"]) == O.OK
    return c


def _slots(c, w, b, h, tiers):
    """(page, slot) of each kept token of (b, h) in kept_tokens order."""
    row = b * w["Hkv"] + h
    by_tier = {0: [], 1: [], 2: []}
    for i in range(c.num_pages[row]):
        page = c.page_table[row, i]
        tier, count = int(c.page_meta[page, 0]), int(c.page_meta[page, 1])
        by_tier[tier].extend((page, s) for s in range(count))
    out = []
    for pos, tau in kept_tokens(dict(w, tiers=tiers), b, h):
        out.append(by_tier[tau].pop(0))
    return out


def test_utility_equals_numpy_softmax_mass():
    w = W.config("ragged", ctx=400, batch=3)
    c = _pack(w)
    u = O.decode_utility(c, w["q"], w["scale"])
    G = w["Hq"] // w["Hkv"]
    for b in range(w["B"]):
        for h in range(w["Hkv"]):
            toks = kept_tokens(w, b, h)
            if not toks:
                continue
            kh = []
            for pos, tau in toks:
                tb, sb = O.TIER_BITS[tau]
                r16, th, s, st = O.encode(w["keys"][b, h, pos], tb, sb)
                kh.append(dequantize(r16[0], th[0], s[0], tb, sb))
            kh = np.array(kh).reshape(-1, 128)
            mass = np.zeros(len(toks))
            for g in range(G):
                lg = w["scale"] * (kh @ w["q"][b, h * G + g].astype(np.float64))
                e = np.exp(lg - lg.max())
                mass += e / e.sum()
            got = np.array([u[p, s] for p, s in _slots(c, w, b, h, w["tiers"])])
            assert np.max(np.abs(got - mass)) <= 1e-12 * G, (b, h)


def test_utility_rows_sum_to_group_size():
    w = W.config("llama8b", ctx=300, batch=2)
    c = _pack(w)
    u = O.decode_utility(c, w["q"], w["scale"])
    G = w["Hq"] // w["Hkv"]
    for b in range(w["B"]):
        for h in range(w["Hkv"]):
            vals = [u[p, s] for p, s in _slots(c, w, b, h, w["tiers"])]
            assert abs(sum(vals) - G) <= 1e-12 * G


def test_utility_lone_token_and_untouched_entries():
    w = W.config("llama8b", ctx=200, batch=2)
    t = w["tiers"].copy()
    t[0, 3, :] = -1
    t[0, 3, 77] = 1                     # one kept token in row (0, 3)
    t[1, 5, :] = -1                     # an empty row
    c = _pack(w, tiers=t)
    u = O.decode_utility(c, w["q"], w["scale"])
    G = w["Hq"] // w["Hkv"]
    (p, s), = _slots(c, w, 0, 3, t)
    assert u[p, s] == G
    # exactly the slots holding kept tokens were written
    written = np.zeros(u.shape, bool)
    for b in range(w["B"]):
        for h in range(w["Hkv"]):
            for p, s in _slots(c, w, b, h, t):
                written[p, s] = True
    assert np.isfinite(u[written]).all() and np.isnan(u[~written]).all()
