"""GPU parity of the HIP library against the CPU oracle, through the C ABI.

Bit-exact: code arena, page metadata, page tables, page counts, open pages,
allocation counters and RDR tier maps.  Outputs: per (sequence, query head)
row, max |o_gpu - o_ref| <= 2e-3 max |o_ref| and |lse_gpu - lse_ref| <= 2e-3.
Sizes here span many pages and work-groups with ragged tails; the full
workload sizes are in test_gpu_fullsize.py."""
import numpy as np
import pytest
import torch

import compressed_kv_cache_ada_amd as ada
import workloads as W
from oracle import oracle as O
from tests.gpu_util import (TOL, check_outputs, compare_caches, gpu_cache, gpu_pack, log, oracle_cache,
                            to_dev)
from tests.util import near_boundary_pairs

pytestmark = pytest.mark.gpu

SMALL = [("tiny", 4096, 1), ("llama8b", 1536, 2), ("long256k", 3000, 1), ("ragged", 2500, 5)]


def _oracle_pack(w, tiers=None):
    oc = oracle_cache(w)
    st = O.pack(oc, w["ctx_len"], w["tiers"] if tiers is None else tiers, w["keys"], w["values"])
    assert st == O.OK
    return oc


def test_lut_matches_oracle():
    w = W.config("llama8b", ctx=16, batch=2)
    cfg = ada.make_config(16, w["Hq"], w["Hkv"])
    lut = ada.build_lut(cfg, torch.from_numpy(w["q"]).cuda()).cpu().numpy()
    for b in range(w["B"]):
        for hq in range(w["Hq"]):
            q = w["q"][b, hq]
            ref = np.concatenate([O.lut(q, 8).ravel(), O.lut(q, 4).ravel(), O.lut(q, 2).ravel()])
            err = np.max(np.abs(lut[b, hq] - ref)) / np.max(np.abs(ref))
            assert err <= 1e-6, (b, hq, err)


@pytest.mark.parametrize("name,ctx,batch", SMALL)
def test_pack_bit_exact(name, ctx, batch):
    log(f"pack {name} ctx={ctx} batch={batch}")
    w = W.config(name, ctx=ctx, batch=batch)
    gc, _ = gpu_pack(w)
    compare_caches(gc, _oracle_pack(w), w["P"])


@pytest.mark.parametrize("name,ctx,batch", SMALL)
def test_decode_parity(name, ctx, batch):
    log(f"decode {name} ctx={ctx} batch={batch}")
    w = W.config(name, ctx=ctx, batch=batch)
    gc, dev = gpu_pack(w)
    out, lse = ada.decode(gc, dev["q"], w["scale"])
    o_ref, lse_ref = O.decode(_oracle_pack(w), w["q"], w["scale"])
    worst = check_outputs(out.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref)
    log(f"  worst row rel err {worst:.2e}")


@pytest.mark.parametrize("chunk_pages", [1, 4, 7, 1000])
def test_decode_chunking_invariance(chunk_pages):
    """Split-K merge: any chunk length gives the oracle's result."""
    w = W.config("llama8b", ctx=1024, batch=1)
    cfg = ada.make_config(16, w["Hq"], w["Hkv"], decode_chunk_pages=chunk_pages)
    dev = to_dev(w)
    gc = gpu_cache(w, cfg=cfg)
    ada.pack(gc, w["ctx_len"], torch.from_numpy(w["tiers"]).cuda(), dev["keys"], dev["values"])
    assert ada.read_status(gc.status) == ada.OK
    out, lse = ada.decode(gc, dev["q"], w["scale"])
    o_ref, lse_ref = O.decode(_oracle_pack(w), w["q"], w["scale"])
    check_outputs(out.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref)


def test_decode_deterministic_and_partials_api():
    w = W.config("ragged", ctx=2000, batch=3)
    gc, dev = gpu_pack(w)
    o1, l1 = ada.decode(gc, dev["q"], w["scale"])
    ws = ada.decode_workspace(gc, w["B"])
    ada.decode_partials(gc, dev["q"], w["scale"], ws)
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    ada.decode_reduce(gc, w["B"], o2, l2, ws)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_edge_rows_empty_single_partial():
    w = W.config("llama8b", ctx=300, batch=2)
    t = w["tiers"].copy()
    t[0, 0, :] = -1                  # empty row
    t[0, 1, :] = -1
    t[0, 1, 123] = 2                 # a single T2 token
    t[1, 2, :] = -1
    t[1, 2, :17] = 1                 # one full page + one token
    gc, dev = gpu_pack(w, tiers=t)
    out, lse = ada.decode(gc, dev["q"], w["scale"])
    o_ref, lse_ref = O.decode(_oracle_pack(w, tiers=t), w["q"], w["scale"])
    check_outputs(out.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref)
    G = w["Hq"] // w["Hkv"]
    assert torch.all(out[0, :G] == 0) and torch.all(torch.isinf(lse[0, :G]))


def test_permuted_page_pool_gives_identical_output():
    w = W.config("ragged", ctx=1500, batch=4)
    gc, dev = gpu_pack(w)
    o1, l1 = ada.decode(gc, dev["q"], w["scale"])
    n = int(gc.alloc[0].item())
    perm = torch.from_numpy(W.page_permutation(w["perm_rng"], n)).cuda().long()
    meta = gc.page_meta[:n].clone()
    gc.page_meta[perm] = meta
    pt = gc.page_table.long()
    mask = torch.arange(pt.shape[1], device=pt.device)[None, :] < gc.num_pages[:, None]
    gc.page_table.copy_(torch.where(mask, perm[pt.clamp(0, n - 1)], pt).int())
    o2, l2 = ada.decode(gc, dev["q"], w["scale"])
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_zero_query_gives_mean():
    w = W.config("long256k", ctx=700, batch=1)
    gc, dev = gpu_pack(w)
    out, _ = ada.decode(gc, torch.zeros_like(dev["q"]), w["scale"])
    G = w["Hq"] // w["Hkv"]
    for h in range(w["Hkv"]):
        kept = w["tiers"][0, h] >= 0
        mean = w["values"][0, h][kept].view(np.float16).astype(np.float64).mean(0)
        got = out[0, h * G:(h + 1) * G].cpu().numpy()
        assert np.max(np.abs(got - mean[None])) <= TOL * np.max(np.abs(mean))


# ------------------------------------------------------------------ RDR
def _gpu_rdr(w, budget=None, mask=0):
    cfg = ada.make_config(w["P"], w["Hq"], w["Hkv"], rdr_tier_mask=mask)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    t = ada.rdr_assign(cfg, w["ctx_len"], torch.from_numpy(w["utility"]).cuda(),
                       w["budget"] if budget is None else budget, status)
    st = ada.read_status(status)
    return st, t.cpu().numpy()


def test_rdr_bit_exact():
    w = W.config("rdr128k", ctx=3000, batch=3)
    st, t = _gpu_rdr(w)
    assert st == ada.OK
    st_o, t_o = O.rdr_assign(w["ctx_len"], w["utility"], w["budget"])
    assert st_o == O.OK and np.array_equal(t, t_o)


@pytest.mark.parametrize("case", ["ties", "zeros", "budget0", "huge", "t4only", "neg_zero", "ragged"])
def test_rdr_edge_cases(case):
    w = W.config("rdr128k", ctx=600, batch=2)
    budget = w["budget"]
    mask = 0
    if case == "ties":
        w["utility"][:] = 1.5
    elif case == "zeros":
        w["utility"][0, :, ::3] = 0.0
        w["utility"][1] = 0.0
    elif case == "budget0":
        budget = np.zeros(2, np.int64)
    elif case == "huge":
        budget = np.full(2, 10 ** 12, np.int64)
    elif case == "t4only":
        mask = 0b010
    elif case == "neg_zero":
        w["utility"][:, :, ::2] = -0.0
    elif case == "ragged":
        w["ctx_len"] = np.array([600, 211], np.int32)
    st, t = _gpu_rdr(w, budget, mask)
    assert st == ada.OK
    st_o, t_o = O.rdr_assign(w["ctx_len"], w["utility"], budget, mask or 0b111)
    assert st_o == O.OK and np.array_equal(t, t_o)


def test_rdr_invalid_utility_sets_status():
    w = W.config("rdr128k", ctx=100, batch=1)
    w["utility"][0, 3, 7] = np.nan
    st, _ = _gpu_rdr(w)
    assert st == ada.EINVAL


# ---------------------------------------------------------------- append
def _append_both(w, gc, oc, seq, head, tier, keys, values):
    ada.encode_append(gc, torch.from_numpy(np.asarray(seq, np.int32)).cuda(),
                      torch.from_numpy(np.asarray(head, np.int32)).cuda(),
                      torch.from_numpy(np.asarray(tier, np.uint8)).cuda(),
                      torch.from_numpy(np.ascontiguousarray(keys, np.float32)).cuda(),
                      torch.from_numpy(np.ascontiguousarray(values).view(np.int16)).cuda())
    st = ada.read_status(gc.status)
    st_o = O.append(oc, seq, head, tier, keys, values)
    return st, st_o


def test_append_sequences_bit_exact():
    w = W.config("ragged", ctx=400, batch=3)
    gc = gpu_cache(w)
    oc = oracle_cache(w)
    rng = np.random.default_rng(5)
    flat_k = w["keys"].reshape(-1, 128)
    flat_v = w["values"].reshape(-1, 128)
    for n in [1, 37, 1500, 2100, 64]:   # several calls, one spanning tiles of 1024
        seq = rng.integers(0, w["B"], n)
        head = rng.integers(0, w["Hkv"], n)
        tier = rng.integers(0, 3, n)
        idx = rng.integers(0, flat_k.shape[0], n)
        st, st_o = _append_both(w, gc, oc, seq, head, tier, flat_k[idx], flat_v[idx])
        assert st == ada.OK and st_o == O.OK
        compare_caches(gc, oc, w["P"])
    # decode over appended (tier-interleaved) pages
    dev = to_dev(w)
    out, lse = ada.decode(gc, dev["q"], w["scale"])
    o_ref, lse_ref = O.decode(oc, w["q"], w["scale"])
    check_outputs(out.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref)


def test_append_after_pack_bit_exact():
    w = W.config("llama8b", ctx=500, batch=2)
    gc, dev = gpu_pack(w)
    oc = _oracle_pack(w)
    rng = np.random.default_rng(9)
    n = 300
    keys = rng.standard_normal((n, 128)).astype(np.float32) * 3
    vals = rng.standard_normal((n, 128)).astype(np.float16).view(np.uint16)
    st, st_o = _append_both(w, gc, oc, rng.integers(0, 2, n), rng.integers(0, 8, n), rng.integers(0, 3, n),
                            keys, vals)
    assert st == ada.OK and st_o == O.OK
    compare_caches(gc, oc, w["P"])


def test_append_errors_write_nothing():
    w = W.config("tiny", ctx=64)
    small = (2, 2, 2 * 386)   # two pages of the largest fp16 block
    gc = gpu_cache(w, dims_override=small)
    before = gc.host()
    keys = w["keys"][0, 0, :40]
    vals = w["values"][0, 0, :40]
    # 40 T4 tokens need 3 pages of 16 but only 2 fit
    ada.encode_append(gc, torch.zeros(40, dtype=torch.int32, device="cuda"),
                      torch.zeros(40, dtype=torch.int32, device="cuda"),
                      torch.ones(40, dtype=torch.uint8, device="cuda"),
                      torch.from_numpy(keys).cuda(), torch.from_numpy(vals.view(np.int16)).cuda())
    assert ada.read_status(gc.status) == ada.ENOSPC
    after = gc.host()
    for k in before:
        assert np.array_equal(before[k], after[k]), k
    bad = keys.copy()
    bad[3, 5] = np.inf
    ada.encode_append(gc, torch.zeros(4, dtype=torch.int32, device="cuda"),
                      torch.zeros(4, dtype=torch.int32, device="cuda"),
                      torch.ones(4, dtype=torch.uint8, device="cuda"),
                      torch.from_numpy(bad[:4]).cuda(), torch.from_numpy(vals[:4].view(np.int16)).cuda())
    assert ada.read_status(gc.status) == ada.EINVAL
    after = gc.host()
    for k in before:
        assert np.array_equal(before[k], after[k]), k


def test_pack_errors_write_nothing():
    w = W.config("llama8b", ctx=256, batch=1)
    gc = gpu_cache(w, dims_override=(200, 5, 5000))
    before = gc.host()
    dev = to_dev(w)
    ada.pack(gc, w["ctx_len"], torch.from_numpy(w["tiers"]).cuda(), dev["keys"], dev["values"])
    assert ada.read_status(gc.status) == ada.ENOSPC
    after = gc.host()
    for k in before:
        assert np.array_equal(before[k], after[k]), k
    bad = w["tiers"].copy()
    bad[0, 1, 9] = 5
    gc2 = gpu_cache(w)
    before = gc2.host()
    ada.pack(gc2, w["ctx_len"], torch.from_numpy(bad).cuda(), dev["keys"], dev["values"])
    assert ada.read_status(gc2.status) == ada.EINVAL
    after = gc2.host()
    for k in before:
        assert np.array_equal(before[k], after[k]), k


# -------------------------------------------------------- codec stress
@pytest.mark.parametrize("tier", [0, 1, 2])
def test_adversarial_codec_bit_exact(tier):
    """Keys with angles a hair from rounding boundaries, exact ties, zero
    pairs, zero keys, huge and subnormal values: pages must be byte-equal."""
    tb, sb = O.TIER_BITS[tier]
    keys = []
    pairs = near_boundary_pairs(max(tb, 3)) if tb > 2 else []
    for start in range(0, len(pairs), 64):
        chunk = pairs[start:start + 64] + [(0.0, 0.0)] * (64 - len(pairs[start:start + 64]))
        k = np.zeros(128, np.float32)
        for j, (x, y) in enumerate(chunk):
            k[2 * j], k[2 * j + 1] = x, y
        keys.append(k)
    diag = np.zeros(128, np.float32)
    diag[0::2] = [1, -1, -1, 1] * 16
    diag[1::2] = [1, 1, -1, -1] * 16
    keys.append(diag)                                   # 2-bit diagonal ties
    tie = np.zeros(128, np.float32)
    tie[[0, 2, 4, 6]] = 1.0
    keys.append(tie)                                    # magnitude ties
    keys.append(np.zeros(128, np.float32))              # zero key
    keys.append(np.full(128, 3e38, np.float32))         # radius saturates
    keys.append(np.full(128, 1e-42, np.float32))        # subnormal inputs
    rng = np.random.default_rng(tier)
    keys.extend((rng.standard_normal((200, 128)) * np.exp(2 * rng.standard_normal((200, 128)))).astype(np.float32))
    keys = np.array(keys, np.float32)
    n = keys.shape[0]
    vals = rng.standard_normal((n, 128)).astype(np.float16).view(np.uint16)
    w = W.config("tiny", ctx=max(n, 16))
    gc = gpu_cache(w)
    oc = oracle_cache(w)
    st, st_o = _append_both(w, gc, oc, np.zeros(n), np.zeros(n), np.full(n, tier), keys, vals)
    assert st == ada.OK and st_o == O.OK
    compare_caches(gc, oc, w["P"])


@pytest.mark.parametrize("name,chunk_pages", [("long256k", 0), ("long256k", 1000), ("llama8b", 1000)])
def test_decode_late_logit_spikes(name, chunk_pages):
    """Keys planted late in each row along one query head's direction, each
    larger than the last, so that a wavefront's running maximum has to move
    by far more than 2^8 (base 2) in the middle of its groups: the rescale
    path of the online softmax after groups weighted against an older
    maximum (eight query heads per KV head), and the per-group maximum
    (four).  A chunk length of 1000 pages puts one chunk on each row, so
    every wavefront walks several groups."""
    w = W.config(name, ctx=2600, batch=1)
    G = w["Hq"] // w["Hkv"]
    keys, tiers = w["keys"].copy(), w["tiers"].copy()
    for h in range(w["Hkv"]):
        for k, pos in enumerate((1500, 1900, 2300, 2550)):
            g = h * G + (pos + h) % G
            keys[0, h, pos] = (1.0 + k) * w["q"][0, g]   # logit about 11 (1 + k) |q|^2 / 128 for head g
            tiers[0, h, pos] = 1                          # kept, T4
    w = dict(w, keys=keys, tiers=tiers)
    log(f"late spikes {name} chunk_pages={chunk_pages}")
    cfg = ada.make_config(w["P"], w["Hq"], w["Hkv"], decode_chunk_pages=chunk_pages)
    dev = to_dev(w)
    gc = gpu_cache(w, cfg=cfg)
    ada.pack(gc, w["ctx_len"], torch.from_numpy(tiers).cuda(), dev["keys"], dev["values"])
    assert ada.read_status(gc.status) == ada.OK
    out, lse = ada.decode(gc, dev["q"], w["scale"])
    o_ref, lse_ref = O.decode(_oracle_pack(w), w["q"], w["scale"])
    # the spikes dominate their heads: the largest lse is far above the rest
    assert np.max(lse_ref) > np.median(lse_ref) + 20
    worst = check_outputs(out.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref)
    log(f"  worst row rel err {worst:.2e}")
