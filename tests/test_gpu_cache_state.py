"""Cache state on the device: the page-list check (ada_validate_cache) and a
checkpoint round trip, and the cache's row order (a dispatch hint).

The check must accept packed caches and flag, through the status word, a
page count past the row's table, a page id outside the pool, malformed
page metadata and a row order that is not a permutation of the rows.  The decode is never launched on a corrupted table (it does
not range-check page ids).  The round trip copies every caller-owned buffer
of a packed cache to the host, restores it into a fresh cache and checks
that decode and append then behave bit for bit as on the original."""
import numpy as np
import pytest
import torch

import compressed_kv_cache_ada_amd as ada
import workloads as W
from tests.gpu_util import dims, gpu_pack, log

pytestmark = pytest.mark.gpu


def _status_after(cache, B):
    ada.validate_cache(cache, B)
    return ada.read_status(cache.status)


def test_validate_accepts_packed_and_flags_corruption():
    w = W.config("ragged", ctx=1200, batch=3)
    log("validate ragged ctx 1200 batch 3")
    gc, _ = gpu_pack(w)
    B = w["B"]
    assert _status_after(gc, B) == ada.OK
    cap = gc.desc.page_capacity
    r, k = 4, 1
    # a page id outside the pool
    good = int(gc.page_table[r, k])
    gc.page_table[r, k] = cap + 5
    assert _status_after(gc, B) == ada.EINVAL
    gc.page_table[r, k] = -3
    assert _status_after(gc, B) == ada.EINVAL
    gc.page_table[r, k] = good
    assert _status_after(gc, B) == ada.OK
    # a page count past the row's table, and a negative one
    n = int(gc.num_pages[r])
    gc.num_pages[r] = gc.desc.max_pages_per_head + 1
    assert _status_after(gc, B) == ada.EINVAL
    gc.num_pages[r] = -1
    assert _status_after(gc, B) == ada.EINVAL
    gc.num_pages[r] = n
    # malformed metadata of a listed page: count 0, tier 7, non-zero reserved
    # field, code block past the arena
    meta = gc.page_meta[good].clone()
    for byte, value in ((1, 0), (0, 7), (2, 1)):
        gc.page_meta[good, byte] = value
        assert _status_after(gc, B) == ada.EINVAL, (byte, value)
        gc.page_meta[good].copy_(meta)
    off = np.frombuffer(meta.cpu().numpy().tobytes(), dtype=np.uint32)[1]
    bad = np.array([gc.desc.arena_capacity16], dtype=np.uint32).view(np.uint8)
    gc.page_meta[good, 4:8] = torch.from_numpy(bad.copy()).cuda()
    assert _status_after(gc, B) == ada.EINVAL
    gc.page_meta[good].copy_(meta)
    assert off < gc.desc.arena_capacity16 and _status_after(gc, B) == ada.OK
    # rows of sequences past B are not looked at
    last = B * w["Hkv"] - 1
    n_last = int(gc.num_pages[last])
    gc.num_pages[last] = -7
    assert _status_after(gc, B - 1) == ada.OK
    assert _status_after(gc, B) == ada.EINVAL
    gc.num_pages[last] = n_last
    # the row order: an entry out of range, negative, or repeated
    order = gc.row_order.clone()
    rows = order.numel()
    for i, v in ((2, rows), (0, -1), (1, int(order[3]))):
        gc.row_order[i] = v
        assert _status_after(gc, B) == ada.EINVAL, (i, v)
        gc.row_order.copy_(order)
    assert _status_after(gc, B) == ada.OK


def test_checkpoint_round_trip():
    w = W.config("llama8b", ctx=1300, batch=2)
    log("checkpoint llama8b ctx 1300 batch 2")
    src, dev = gpu_pack(w)
    saved = {k: t.cpu().clone() for k, t in (("page_table", src.page_table), ("num_pages", src.num_pages),
                                              ("open_page", src.open_page), ("page_meta", src.page_meta),
                                              ("code_arena", src.code_arena), ("alloc", src.alloc),
                                              ("status", src.status), ("row_order", src.row_order))}
    dst = ada.Cache(src.cfg, src.desc.num_seqs, src.desc.max_pages_per_head, src.desc.page_capacity,
                    src.desc.arena_capacity16)
    for k, t in saved.items():
        getattr(dst, k).copy_(t)
    assert _status_after(dst, w["B"]) == ada.OK
    o1, l1 = ada.decode(src, dev["q"], w["scale"])
    o2, l2 = ada.decode(dst, dev["q"], w["scale"])
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # the restored cache keeps growing exactly like the original
    rng = np.random.default_rng(9)
    n = 40
    req = [torch.from_numpy(x).cuda() for x in (rng.integers(0, w["B"], n).astype(np.int32),
                                                  rng.integers(0, w["Hkv"], n).astype(np.int32),
                                                  rng.integers(0, 3, n).astype(np.uint8),
                                                  rng.standard_normal((n, 128), dtype=np.float32),
                                                  rng.standard_normal((n, 128)).astype(np.float16).view(np.int16))]
    for c in (src, dst):
        ada.encode_append(c, *req)
        assert ada.read_status(c.status) == ada.OK
    hs, hd = src.host(), dst.host()
    for k in hs:
        assert np.array_equal(hs[k], hd[k]), k
    o1, l1 = ada.decode(src, dev["q"], w["scale"])
    o2, l2 = ada.decode(dst, dev["q"], w["scale"])
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _longest_first(num_pages):
    return np.argsort(-num_pages.astype(np.int64), kind="stable").astype(np.int32)


def test_row_order_sorts_rows_and_changes_no_result():
    """ada_cache_init writes the identity; pack and re-pack leave the rows
    sorted by decreasing page count (ties in row order); the decode's result
    does not depend on the order (every output bit equal under the identity
    and under a reversed order)."""
    w = W.config("ragged", ctx=2400, batch=6)
    log("row order ragged ctx 2400 batch 6")
    c = ada.Cache(ada.make_config(w["P"], w["Hq"], w["Hkv"]), w["B"], *dims(w))
    ada.cache_init(c)
    assert np.array_equal(c.row_order.cpu().numpy(), np.arange(w["B"] * w["Hkv"]))
    dev = {"keys": torch.from_numpy(w["keys"]).cuda(), "values": torch.from_numpy(w["values"].view(np.int16)).cuda(),
           "q": torch.from_numpy(w["q"]).cuda()}
    ada.pack(c, w["ctx_len"], torch.from_numpy(w["tiers"]).cuda(), dev["keys"], dev["values"])
    assert ada.read_status(c.status) == ada.OK
    npg = c.num_pages.cpu().numpy()
    assert np.array_equal(c.row_order.cpu().numpy(), _longest_first(npg))
    assert len(set(npg.tolist())) > 1   # the rows differ in length
    o1, l1 = ada.decode(c, dev["q"], w["scale"])
    sorted_order = c.row_order.clone()
    for order in (torch.arange(npg.size, dtype=torch.int32, device="cuda"),
                  torch.flip(sorted_order, [0]).contiguous()):
        c.row_order.copy_(order)
        o2, l2 = ada.decode(c, dev["q"], w["scale"])
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # re-pack: the destination's order follows its own page counts
    c.row_order.copy_(sorted_order)
    util = torch.rand((c.desc.page_capacity, w["P"]), device="cuda")
    dst = ada.Cache(c.cfg, w["B"], c.desc.max_pages_per_head, c.desc.page_capacity, c.desc.arena_capacity16)
    ada.cache_init(dst)
    budget = [int(x) for x in np.full(w["B"], 300_000)]
    ada.repack(c, w["B"], util, budget, dst)
    assert ada.read_status(dst.status) == ada.OK
    assert np.array_equal(dst.row_order.cpu().numpy(), _longest_first(dst.num_pages.cpu().numpy()))
