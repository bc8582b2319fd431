"""Pins of the oracle's RDR re-pack: code-space transcoding, RDR with
per-item caps (downgrade only), and the re-packed cache.

Transcoding must equal re-encoding the exactly dequantised angle / magnitude
(angles: the encoder on the grid direction, half up on exact ties;
magnitudes: exact fractions, which never tie for these tiers).  Capped RDR
must be optimal at its own rate among assignments within the caps (brute
force) and reduce to plain RDR without caps.  A re-pack with an unlimited
budget must reproduce the source pack byte for byte; any re-pack must keep
to its budget, only downgrade, and decode like dense attention over the
transcoded keys."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import workloads as W
from oracle import oracle as O
from tests.util import dense_attention, dequantize, upper_capacity

RATE = {-1: 0, 2: 298, 1: 322, 0: 386}
DIST = {-1: 1.0, 2: 2.0 ** -5, 1: 2.0 ** -8, 0: 2.0 ** -16}
LEVEL = {-1: 0, 2: 1, 1: 2, 0: 3}
PAIRS = [(0, 1), (0, 2), (1, 2)]


@pytest.mark.parametrize("t_old,t_new", PAIRS)
def test_transcode_angle_is_reencoding(t_old, t_new):
    tb_o, sb_o = O.TIER_BITS[t_old]
    tb_n, sb_n = O.TIER_BITS[t_new]
    d = tb_o - tb_n
    codes = np.arange(1 << tb_o, dtype=np.uint16)
    th = np.zeros((codes.size, 64), np.uint16)
    th[:, 0] = codes
    th_n, _ = O.transcode(t_old, t_new, th, np.zeros_like(th))
    for c in codes:
        got = int(th_n[c, 0])
        if c % (1 << d) == (1 << (d - 1)):            # exact tie between two new grid points
            assert got == (((int(c) >> d) + 1) % (1 << tb_n))
            continue
        ang = -np.pi + float(c) * 2 * np.pi / (1 << tb_o)
        key = np.zeros(128, np.float32)
        key[0], key[1] = np.cos(ang), np.sin(ang)
        _, th_e, _, st = O.encode(key, tb_n, sb_n)
        assert st == O.OK and got == int(th_e[0][0]), (c, got, int(th_e[0][0]))


@pytest.mark.parametrize("t_old,t_new", PAIRS)
def test_transcode_magnitude_exact(t_old, t_new):
    L_o = (1 << O.TIER_BITS[t_old][1]) - 1
    L_n = (1 << O.TIER_BITS[t_new][1]) - 1
    s = np.zeros((L_o + 1, 64), np.uint16)
    s[:, 5] = np.arange(L_o + 1)
    _, s_n = O.transcode(t_old, t_new, np.zeros_like(s), s)
    for c in range(L_o + 1):
        x = Fraction(c * L_n, L_o)
        assert x - int(x) != Fraction(1, 2)             # never a tie
        assert int(s_n[c, 5]) == int(x + Fraction(1, 2)), c


def test_transcode_same_tier_is_identity():
    rng = np.random.default_rng(0)
    for t in range(3):
        tb, sb = O.TIER_BITS[t]
        th = rng.integers(0, 1 << tb, (4, 64)).astype(np.uint16)
        s = rng.integers(0, 1 << sb, (4, 64)).astype(np.uint16)
        th_n, s_n = O.transcode(t, t, th, s)
        assert np.array_equal(th, th_n) and np.array_equal(s, s_n)


@pytest.mark.parametrize("seed", range(6))
def test_capped_rdr_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    n = 6
    util = np.exp(rng.standard_normal(n)).astype(np.float32)
    cap = rng.integers(0, 4, n).astype(np.int8)         # steps allowed per item
    budget = int(rng.integers(0, 386 * n + 50))
    st, tiers = O.rdr_assign(np.array([n], np.int32), util[None, None], np.array([budget]), cap_level=cap[None, None])
    assert st == O.OK
    t = tiers[0, 0]
    assert all(LEVEL[int(x)] <= int(k) for x, k in zip(t, cap))
    Rg = sum(RATE[int(x)] for x in t)
    Dg = sum(float(u) * DIST[int(x)] for u, x in zip(util, t))
    assert Rg <= budget
    choices = [[x for x in (-1, 2, 1, 0) if LEVEL[x] <= k] for k in cap]
    for combo in itertools.product(*choices):
        if sum(RATE[x] for x in combo) <= Rg:
            assert sum(float(u) * DIST[x] for u, x in zip(util, combo)) >= Dg - 1e-12 * max(1.0, Dg)


def test_capped_rdr_without_binding_caps_is_rdr():
    rng = np.random.default_rng(3)
    util = np.exp(rng.standard_normal((2, 3, 200))).astype(np.float32)
    ctx, budget = np.array([200, 150], np.int32), np.array([90000, 40000])
    st1, t1 = O.rdr_assign(ctx, util, budget)
    st2, t2 = O.rdr_assign(ctx, util, budget, cap_level=np.full(util.shape, 3, np.int8))
    assert st1 == st2 == O.OK and np.array_equal(t1, t2)


def _packed(w):
    per_row, pages, units = upper_capacity(w, 386 * w["P"] // 16)
    src = O.Cache(w["P"], w["Hq"], w["Hkv"], w["B"], per_row, pages, units)
    assert O.pack(src, w["ctx_len"], w["tiers"], w["keys"], w["values"]) == O.OK
    dst = O.Cache(w["P"], w["Hq"], w["Hkv"], w["B"], per_row, pages, units)
    return src, dst


def test_repack_unlimited_budget_reproduces_pack():
    w = W.config("ragged", ctx=500, batch=3)
    src, dst = _packed(w)
    util = np.exp(np.random.default_rng(1).standard_normal((src.page_capacity, w["P"]))).astype(np.float32)
    st, tv = O.repack(src, w["B"], util, np.full(w["B"], 1 << 40), dst)
    assert st == O.OK
    for k in ("page_table", "num_pages", "open_page", "page_meta", "arena", "alloc"):
        assert np.array_equal(getattr(src, k), getattr(dst, k)), k


def test_repack_budget_downgrade_and_decode():
    w = W.config("llama8b", ctx=320, batch=2)
    src, dst = _packed(w)
    util = np.exp(np.random.default_rng(2).standard_normal((src.page_capacity, w["P"]))).astype(np.float32)
    cur_rate = [sum(RATE[int(x)] for x in w["tiers"][b].ravel()) for b in range(w["B"])]
    budget = np.array([int(0.45 * r) for r in cur_rate])
    st, tv = O.repack(src, w["B"], util, budget, dst)
    assert st == O.OK
    P = w["P"]
    for b in range(w["B"]):
        assert sum(RATE[int(x)] for x in tv[b].ravel()) <= budget[b]
    q = w["q"]
    out, lse = O.decode(dst, q, w["scale"])
    G = w["Hq"] // w["Hkv"]
    for b in range(w["B"]):
        for h in range(w["Hkv"]):
            row = b * w["Hkv"] + h
            keys, vals = [], []
            for tau in (0, 1, 2):                         # the destination's page order
                for t in np.nonzero(tv[b, h] == tau)[0]:
                    page = src.page_table[row, t // P]
                    told = int(src.page_meta[page, 0])
                    assert LEVEL[tau] <= LEVEL[told]       # downgrade only
                    r16, th, s, _ = O.read_token(src, page, t % P)
                    th_n, s_n = O.transcode(told, tau, th, s)
                    tb, sb = O.TIER_BITS[tau]
                    keys.append(dequantize(r16, th_n[0], s_n[0], tb, sb))
                    sl = int(t % P)
                    vals.append(O.value_part(src, page).view(np.uint16)[(sl // 8) * 1024 + np.arange(128) * 8 + sl % 8]
                                .view(np.float16).astype(np.float64))
            keys, vals = np.array(keys).reshape(-1, 128), np.array(vals).reshape(-1, 128)
            for g in range(G):
                o_ref, l_ref = dense_attention(keys, vals, q[b, h * G + g], w["scale"])
                if keys.shape[0] == 0:
                    assert lse[b, h * G + g] == -np.inf
                    continue
                assert np.max(np.abs(out[b, h * G + g] - o_ref)) <= 1e-12 * np.max(np.abs(o_ref))
