"""Pins of the oracle's paged decode: it must equal plain softmax attention
(numpy, fp64) over the dequantised keys read from the same codes, and obey
the invariants of attention: weights sum to one, dropped tokens contribute
nothing, lossless angle-domain logits equal q.k, closed forms for one token /
zero query, linearity in V, and chunk merging.

Method followed: the abstract of "SPHERICAL KV" (arXiv 2605.18856, Abstract):
logits are computed from radius + angle codes without rebuilding dense keys,
on a paged decode path over tier-homogeneous pages."""
import numpy as np
import pytest

import workloads as W
from oracle import oracle as O
from tests.util import dense_attention, dequantize, kept_tokens, upper_capacity

BLOCK16_MAX = {16: 386, 32: 772}   # T8 key part + fp16 values, in 16-byte units


def _pack(w, tiers=None, keys=None, values=None):
    per_row, pages, units = upper_capacity(w, BLOCK16_MAX[w["P"]])
    c = O.Cache(w["P"], w["Hq"], w["Hkv"], w["B"], per_row, pages, units)
    st = O.pack(c, w["ctx_len"], w["tiers"] if tiers is None else tiers,
                w["keys"] if keys is None else keys, w["values"] if values is None else values)
    assert st == O.OK
    return c


def _small(name="llama8b", ctx=384, batch=2):
    return W.config(name, ctx=ctx, batch=batch)


@pytest.mark.parametrize("name,ctx,batch", [("llama8b", 384, 2), ("long256k", 200, 1),
                                            ("ragged", 300, 3), ("tiny", 100, 1)])
def test_decode_equals_dense_attention_on_dequantised_keys(name, ctx, batch):
    w = _small(name, ctx, batch)
    c = _pack(w)
    out, lse = O.decode(c, w["q"], w["scale"])
    G = w["Hq"] // w["Hkv"]
    # independent codes for every kept token (the encoder is pinned elsewhere)
    for b in range(w["B"]):
        for h in range(w["Hkv"]):
            toks = kept_tokens(w, b, h)
            kh, vh = [], []
            for pos, tau in toks:
                tb, sb = O.TIER_BITS[tau]
                r16, th, s, st = O.encode(w["keys"][b, h, pos], tb, sb)
                kh.append(dequantize(r16[0], th[0], s[0], tb, sb))
                vh.append(w["values"][b, h, pos].view(np.float16).astype(np.float64))
            kh = np.array(kh).reshape(-1, 128)
            vh = np.array(vh).reshape(-1, 128)
            for g in range(G):
                hq = h * G + g
                o_ref, lse_ref = dense_attention(kh, vh, w["q"][b, hq], w["scale"])
                if len(toks) == 0:
                    assert (out[b, hq] == 0).all() and lse[b, hq] == -np.inf
                    continue
                assert np.max(np.abs(out[b, hq] - o_ref)) <= 1e-12 * np.max(np.abs(o_ref))
                assert abs(lse[b, hq] - lse_ref) <= 1e-12 * max(1.0, abs(lse_ref))


def test_lossless_angle_domain_logits_equal_dot_product():
    rng = np.random.default_rng(5)
    keys = (rng.standard_normal((500, 128)) * np.exp(rng.standard_normal(128))).astype(np.float32)
    keys[0] = 0
    q = rng.standard_normal(128).astype(np.float32)
    got = O.identity_logits(keys, q)
    ref = keys.astype(np.float64) @ q.astype(np.float64)
    tol = 1e-12 * np.linalg.norm(keys.astype(np.float64), axis=1) * np.linalg.norm(q)
    assert (np.abs(got - ref) <= tol + 1e-300).all()


def test_weights_sum_to_one():
    w = _small()
    w["values"][:] = np.float16(1.0).view(np.uint16)
    out, _ = O.decode(_pack(w), w["q"], w["scale"])
    assert np.max(np.abs(out - 1.0)) <= 1e-14


def test_dropped_tokens_contribute_nothing():
    w = _small()
    c1 = _pack(w)
    keys = w["keys"].copy()
    vals = w["values"].copy()
    drop = w["tiers"] < 0
    keys[drop] = np.nan
    vals[drop] = np.float16(np.nan).view(np.uint16)
    c2 = _pack(w, keys=keys, values=vals)
    o1, l1 = O.decode(c1, w["q"], w["scale"])
    o2, l2 = O.decode(c2, w["q"], w["scale"])
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.isfinite(o1).all()


def test_single_token_and_zero_query_closed_forms():
    w = W.config("tiny", ctx=64)
    tiers = np.full_like(w["tiers"], -1)
    tiers[0, 0, 17] = 1
    c = _pack(w, tiers=tiers)
    out, lse = O.decode(c, w["q"], w["scale"])
    v = w["values"][0, 0, 17].view(np.float16).astype(np.float64)
    assert np.array_equal(out[0, 0], v)                 # one token: weight exactly 1
    r16, th, s, _ = O.encode(w["keys"][0, 0, 17], 4, 4)
    lg = w["scale"] * dequantize(r16[0], th[0], s[0], 4, 4) @ w["q"][0, 0].astype(np.float64)
    assert abs(lse[0, 0] - lg) <= 1e-12 * max(1, abs(lg))
    # zero query: every logit is 0, output is the plain mean of the kept values
    w2 = _small()
    c2 = _pack(w2)
    out0, lse0 = O.decode(c2, np.zeros_like(w2["q"]), w2["scale"])
    G = w2["Hq"] // w2["Hkv"]
    for b in range(w2["B"]):
        for h in range(w2["Hkv"]):
            pos = [p for p, _ in kept_tokens(w2, b, h)]
            mean = w2["values"][b, h, pos].view(np.float16).astype(np.float64).mean(0)
            for g in range(G):
                assert np.max(np.abs(out0[b, h * G + g] - mean)) <= 1e-14
                assert abs(lse0[b, h * G + g] - np.log(len(pos))) <= 1e-12


def test_no_kept_tokens():
    w = W.config("tiny", ctx=32)
    c = _pack(w, tiers=np.full_like(w["tiers"], -1))
    out, lse = O.decode(c, w["q"], w["scale"])
    assert (out == 0).all() and lse[0, 0] == -np.inf


def test_linear_in_values():
    w = _small()
    o1, _ = O.decode(_pack(w), w["q"], w["scale"])
    v2 = (w["values"].view(np.float16).astype(np.float32) * 2).astype(np.float16).view(np.uint16)
    o2, _ = O.decode(_pack(w, values=v2), w["q"], w["scale"])
    assert np.max(np.abs(o2 - 2 * o1)) <= 1e-14 * np.max(np.abs(o1))


def test_chunked_merge_equals_whole():
    """Split each (b, h)'s kept tokens into chunks, decode each chunk on its
    own, merge with m* = max m_c, l* = sum l_c e^(m_c - m*),
    o = sum o_c l_c e^(m_c - m*) / l*; the result equals the unsplit decode."""
    w = _small(batch=1)
    o_full, lse_full = O.decode(_pack(w), w["q"], w["scale"])
    t = w["tiers"]
    ctx = int(w["ctx_len"][0])
    cuts = [0, 37, 200, ctx]
    parts = []
    for a, z in zip(cuts[:-1], cuts[1:]):
        tp = np.full_like(t, -1)
        tp[:, :, a:z] = t[:, :, a:z]
        parts.append(O.decode(_pack(w, tiers=tp), w["q"], w["scale"]))
    m = np.max([p[1] for p in parts], axis=0)
    lsum = sum(np.exp(p[1] - m) for p in parts)
    o = sum(p[0] * np.exp(p[1] - m)[..., None] for p in parts) / lsum[..., None]
    assert np.max(np.abs(o - o_full)) <= 1e-13 * np.max(np.abs(o_full))
    assert np.max(np.abs(m + np.log(lsum) - lse_full)) <= 1e-13 * np.max(np.abs(lse_full))


def test_logit_error_falls_with_bits():
    rng = np.random.default_rng(8)
    keys = (rng.standard_normal((400, 128)) * np.exp(0.5 * rng.standard_normal(128))).astype(np.float32)
    q = rng.standard_normal(128)
    exact = keys.astype(np.float64) @ q
    errs = []
    for tb, sb in [(2, 3), (4, 4), (8, 8), (12, 12), (16, 16)]:
        r16, th, s, st = O.encode(keys, tb, sb)
        assert st == O.OK
        # radius stays fp16, so compare directions: normalise by the fp16 radius
        kh = dequantize(r16, th, s, tb, sb)
        rh = np.asarray(r16).view(np.float16).astype(np.float64)
        r = np.linalg.norm(keys.astype(np.float64), axis=1)
        errs.append(np.mean(np.abs(kh @ q / rh - exact / r)))
    assert all(a > b for a, b in zip(errs, errs[1:])), errs
