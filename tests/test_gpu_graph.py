"""The decode step under HIP graph capture.

ada_decode and ada_decode_append allocate nothing, copy nothing and set no
memory from the host, so a serving loop can capture one step in a graph and
replay it.  Each test captures the step through torch's graph API (the
binding passes torch's current stream, the capture stream), then replays it
several times with eager work and synchronisation in between, changing the
query (and, for the fused step, the new tokens) in place before each replay,
and compares every replay bit for bit with the same step run eagerly."""
import numpy as np
import pytest
import torch

import compressed_kv_cache_ada_amd as ada
import workloads as W
from oracle import oracle as O
from tests.gpu_util import check_outputs, gpu_pack, log

pytestmark = pytest.mark.gpu


def _eager_noise():
    # unrelated eager work between replays
    x = torch.randn(1 << 20, device="cuda")
    return float((x * 2).sum().item())


def test_decode_graph_replays_match_eager():
    w = W.config("llama8b", ctx=1500, batch=2)
    log("graph decode llama8b ctx 1500 batch 2")
    cache, dev = gpu_pack(w)
    B, Hq = w["B"], w["Hq"]
    q = dev["q"].clone()
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws = ada.decode_workspace(cache, B)
    ada.decode(cache, q, w["scale"], out, lse, ws)   # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ada.decode(cache, q, w["scale"], out, lse, ws)
    rng = np.random.default_rng(31)
    for rep in range(4):
        qn = rng.standard_normal((B, Hq, 128), dtype=np.float32)
        q.copy_(torch.from_numpy(qn))
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        _eager_noise()
        ref_o, ref_l = ada.decode(cache, torch.from_numpy(qn).cuda(), w["scale"])
        torch.cuda.synchronize()
        assert torch.equal(got_o, ref_o) and torch.equal(got_l, ref_l), rep
    # the last replay also against the oracle
    oc = O.Cache(w["P"], w["Hq"], w["Hkv"], B, cache.desc.max_pages_per_head, cache.desc.page_capacity,
                 cache.desc.arena_capacity16)
    assert O.pack(oc, w["ctx_len"], w["tiers"], w["keys"], w["values"]) == O.OK
    o_ref, l_ref = O.decode(oc, qn, w["scale"])
    check_outputs(got_o.cpu().numpy(), got_l.cpu().numpy(), o_ref, l_ref)


def test_fused_append_decode_graph_matches_eager_steps():
    w = W.config("llama8b", ctx=1000, batch=2)
    log("graph decode_append llama8b ctx 1000 batch 2, 5 steps")
    B, Hq, Hkv = w["B"], w["Hq"], w["Hkv"]
    cg, dev = gpu_pack(w)      # replayed through the graph
    ce, _ = gpu_pack(w, dev=dev)   # stepped eagerly
    q = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
    nk = torch.empty((B, Hkv, 128), dtype=torch.float32, device="cuda")
    nv = torch.empty((B, Hkv, 128), dtype=torch.int16, device="cuda")
    nt = torch.empty((B, Hkv), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    wsg = ada.decode_append_workspace(cg, B)
    wse = ada.decode_append_workspace(ce, B)
    rng = np.random.default_rng(32)

    def inputs():
        return (rng.standard_normal((B, Hq, 128), dtype=np.float32),
                rng.standard_normal((B, Hkv, 128), dtype=np.float32),
                rng.standard_normal((B, Hkv, 128)).astype(np.float16).view(np.int16),
                rng.integers(0, 3, (B, Hkv)).astype(np.uint8))

    # step 0 eagerly on both caches (also warms up), then capture step 1 on cg
    steps = [inputs() for _ in range(6)]
    for c, ws in ((cg, wsg), (ce, wse)):
        a = steps[0]
        ada.decode_append(c, torch.from_numpy(a[0]).cuda(), w["scale"], torch.from_numpy(a[1]).cuda(),
                          torch.from_numpy(a[2]).cuda(), torch.from_numpy(a[3]).cuda(), ws=ws)
    torch.cuda.synchronize()
    for t, x in zip((q, nk, nv, nt), steps[1]):
        t.copy_(torch.from_numpy(x))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):   # capturing records the step; it does not run it
        ada.decode_append(cg, q, w["scale"], nk, nv, nt, out, lse, wsg)
    for i in range(1, 6):
        for t, x in zip((q, nk, nv, nt), steps[i]):
            t.copy_(torch.from_numpy(x))
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        _eager_noise()
        ref_o, ref_l = ada.decode_append(ce, *[torch.from_numpy(x).cuda() for x in steps[i][:1]], w["scale"],
                                         *[torch.from_numpy(x).cuda() for x in steps[i][1:]], ws=wse)
        torch.cuda.synchronize()
        assert ada.read_status(cg.status) == ada.OK and ada.read_status(ce.status) == ada.OK
        assert torch.equal(got_o, ref_o) and torch.equal(got_l, ref_l), i
    hg, he = cg.host(), ce.host()
    for k in hg:
        assert np.array_equal(hg[k], he[k]), k
