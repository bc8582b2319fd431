"""Pins of the oracle's half-split pair layout: pair j = (k[j], k[j+64]),
the pairing of the rotate-half form of rotary position embeddings, as a
configuration alternative to adjacent pairs (k[2j], k[2j+1]).

A key whose only non-zero components are k[j0] and k[j0+64] must encode to
one full-magnitude pair j0 whose angle is the nearest grid point of
atan2(k[j0+64], k[j0]), every other pair being a zero pair; rotating every
half-split pair by a quarter turn must shift every angle code by 2^(tb-2)
and leave radius and magnitudes alone; the decode must equal dense
attention over keys dequantised in that layout, and unquantised
angle-domain logits must equal q . k."""
import numpy as np
import pytest

import workloads as W
from oracle import oracle as O
from tests.util import dense_attention, dequantize, kept_tokens, upper_capacity

HALF = O.PAIRS_HALF


@pytest.mark.parametrize("tier", [0, 1, 2])
def test_single_pair_closed_form(tier):
    tb, sb = O.TIER_BITS[tier]
    N, L = 1 << tb, (1 << sb) - 1
    rng = np.random.default_rng(tier)
    for j0 in (0, 5, 37, 63):
        c0 = int(rng.integers(0, N))
        phi = -np.pi + (c0 + 0.25) * 2 * np.pi / N          # a quarter step off grid point c0
        rho = float(rng.uniform(0.5, 20.0))
        key = np.zeros(128, np.float32)
        key[j0], key[j0 + 64] = rho * np.cos(phi), rho * np.sin(phi)
        r16, th, s, st = O.encode(key, tb, sb, pair_layout=HALF)
        assert st == O.OK
        x, y = float(key[j0]), float(key[j0 + 64])
        assert r16[0] == np.float16(np.hypot(x, y)).view(np.uint16)
        want_s = np.zeros(64, np.uint16)
        want_s[j0] = L
        assert np.array_equal(s[0], want_s)
        want_th = np.full(64, N // 2, np.uint16)                # zero pairs
        want_th[j0] = c0
        assert np.array_equal(th[0], want_th)
        # the adjacent layout sees two half-filled pairs instead
        _, _, s_adj, _ = O.encode(key, tb, sb)
        assert set(np.nonzero(s_adj[0])[0]) == {j0 // 2, (j0 + 64) // 2}


@pytest.mark.parametrize("tier", [0, 1, 2])
def test_quarter_turn_shifts_angle_codes(tier):
    tb, sb = O.TIER_BITS[tier]
    N = 1 << tb
    keys = np.random.default_rng(10 + tier).standard_normal((200, 128)).astype(np.float32)
    rot = np.empty_like(keys)
    rot[:, :64] = -keys[:, 64:]                          # (x, y) -> (-y, x) on every pair (k[j], k[j+64])
    rot[:, 64:] = keys[:, :64]
    r1, th1, s1, st1 = O.encode(keys, tb, sb, pair_layout=HALF)
    r2, th2, s2, st2 = O.encode(rot, tb, sb, pair_layout=HALF)
    assert st1 == st2 == O.OK
    assert np.array_equal(r1, r2) and np.array_equal(s1, s2)
    assert np.array_equal(th2.astype(np.int64), (th1.astype(np.int64) + N // 4) % N)


def test_identity_logits_equal_dot_product():
    rng = np.random.default_rng(4)
    keys = rng.standard_normal((64, 128)).astype(np.float32)
    q = rng.standard_normal(128).astype(np.float32)
    lg = O.identity_logits(keys, q, pair_layout=HALF)
    ref = keys.astype(np.float64) @ q.astype(np.float64)
    assert np.max(np.abs(lg - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_decode_equals_dense_over_half_split_keys():
    w = W.config("ragged", ctx=300, batch=3)
    per_row, pages, units = upper_capacity(w, 386 * w["P"] // 16)
    c = O.Cache(w["P"], w["Hq"], w["Hkv"], w["B"], per_row, pages, units, pair_layout=HALF)
    assert O.pack(c, w["ctx_len"], w["tiers"], w["keys"], w["values"]) == O.OK
    out, lse = O.decode(c, w["q"], w["scale"])
    G = w["Hq"] // w["Hkv"]
    for b in range(w["B"]):
        for h in range(w["Hkv"]):
            toks = kept_tokens(w, b, h)
            kh, vh = [], []
            for pos, tau in toks:
                tb, sb = O.TIER_BITS[tau]
                r16, th, s, st = O.encode(w["keys"][b, h, pos], tb, sb, pair_layout=HALF)
                kh.append(dequantize(r16[0], th[0], s[0], tb, sb, half_split=True))
                vh.append(w["values"][b, h, pos].view(np.float16).astype(np.float64))
            kh, vh = np.array(kh).reshape(-1, 128), np.array(vh).reshape(-1, 128)
            for g in range(G):
                o_ref, l_ref = dense_attention(kh, vh, w["q"][b, h * G + g], w["scale"])
                if kh.shape[0] == 0:
                    assert lse[b, h * G + g] == -np.inf
                    continue
                assert np.max(np.abs(out[b, h * G + g] - o_ref)) <= 1e-12 * np.max(np.abs(o_ref))
                assert abs(lse[b, h * G + g] - l_ref) <= 1e-12 * max(1.0, abs(l_ref))
