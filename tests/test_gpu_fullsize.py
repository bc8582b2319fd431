"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (automatic split-K chunking): bit-exact pages and RDR tier
maps against the oracle, and decode outputs within 2e-3 per row."""
import numpy as np
import pytest
import torch

import compressed_kv_cache_ada_amd as ada
import workloads as W
from oracle import oracle as O
from tests.gpu_util import check_outputs, compare_caches, gpu_cache, gpu_pack, log, oracle_cache, to_dev
from tests.util import dense_attention
from workloads import dense_pages

pytestmark = pytest.mark.gpu


def _oracle_pack(w, tiers=None):
    oc = oracle_cache(w)
    assert O.pack(oc, w["ctx_len"], w["tiers"] if tiers is None else tiers, w["keys"], w["values"]) == O.OK
    return oc


@pytest.mark.parametrize("name", ["llama8b", "long256k", "ragged"])
def test_fullsize_pack_and_decode(name):
    log(f"full {name}: generate")
    w = W.config(name)
    log("  gpu pack")
    gc, dev = gpu_pack(w)
    log("  oracle pack")
    oc = _oracle_pack(w)
    log("  compare pages")
    compare_caches(gc, oc, w["P"])
    if name == "ragged":   # shared pool: physical page ids permuted after packing
        n = int(gc.alloc[0].item())
        perm = torch.from_numpy(W.page_permutation(w["perm_rng"], n)).cuda().long()
        gc.page_meta[perm] = gc.page_meta[:n].clone()
        pt = gc.page_table.long()
        mask = torch.arange(pt.shape[1], device=pt.device)[None, :] < gc.num_pages[:, None]
        gc.page_table.copy_(torch.where(mask, perm[pt.clamp(0, n - 1)], pt).int())
    log("  decode")
    out, lse = ada.decode(gc, dev["q"], w["scale"])
    o_ref, lse_ref = O.decode(oc, w["q"], w["scale"])
    worst = check_outputs(out.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref)
    log(f"  worst row rel err {worst:.2e}")


def test_fullsize_rdr_pack_decode():
    log("full rdr128k: generate")
    w = W.config("rdr128k")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    cfg = ada.make_config(w["P"], w["Hq"], w["Hkv"])
    util = torch.from_numpy(w["utility"]).cuda()
    log("  gpu rdr")
    t_gpu = ada.rdr_assign(cfg, w["ctx_len"], util, w["budget"], status)
    assert ada.read_status(status) == ada.OK
    log("  oracle rdr")
    st, t_ref = O.rdr_assign(w["ctx_len"], w["utility"], w["budget"])
    assert st == O.OK
    t_np = t_gpu.cpu().numpy()
    assert np.array_equal(t_np, t_ref)
    fr = {k: float((t_np == k).mean()) for k in (-1, 0, 1, 2)}
    log(f"  tier fractions drop/T8/T4/T2 = {fr[-1]:.4f}/{fr[0]:.5f}/{fr[1]:.4f}/{fr[2]:.4f}")
    w["tiers"] = t_ref
    log("  gpu pack")
    gc, dev = gpu_pack(w)
    log("  oracle pack")
    oc = _oracle_pack(w)
    compare_caches(gc, oc, w["P"])
    log("  decode")
    out, lse = ada.decode(gc, dev["q"], w["scale"])
    o_ref, lse_ref = O.decode(oc, w["q"], w["scale"])
    check_outputs(out.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref)


@pytest.mark.parametrize("name,ctx,batch", [("long256k", 1000, 1), ("long256k", 262144, 1), ("llama8b", 1500, 2),
                                            ("ragged", 900, 3), ("tiny", 700, 2)])
def test_dense_reference_parity(name, ctx, batch):
    """The dense fp16 reference decode (eight heads per KV head: logits on
    the matrix cores; fewer: fp32 FMAs) against fp64 softmax attention over
    the same fp16 keys and values, every query head of every sequence."""
    w = W.config(name, ctx=ctx, batch=batch)
    log(f"dense reference {name} ctx {ctx} batch {batch}")
    k16 = w["keys"].astype(np.float16).view(np.uint16)
    kp, vp, pt = dense_pages(k16, w["values"], w["P"])
    cfg = ada.make_config(w["P"], w["Hq"], w["Hkv"])
    out, lse = ada.dense_decode(cfg, torch.from_numpy(pt).cuda(),
                                torch.from_numpy(w["ctx_len"]).cuda(),
                                torch.from_numpy(kp.view(np.int16)).cuda(), torch.from_numpy(vp.view(np.int16)).cuda(),
                                torch.from_numpy(w["q"]).cuda(), w["scale"])
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    G = w["Hq"] // w["Hkv"]
    for b in range(w["B"]):
        n = int(w["ctx_len"][b])
        for h in range(w["Hkv"]):   # the KV head's keys and values converted once
            kf = k16[b, h, :n].view(np.float16).astype(np.float64)
            vf = w["values"][b, h, :n].view(np.float16).astype(np.float64)
            for hq in range(h * G, (h + 1) * G):
                o_ref, l_ref = dense_attention(kf, vf, w["q"][b, hq], w["scale"])
                err = np.max(np.abs(out[b, hq] - o_ref)) / np.max(np.abs(o_ref))
                assert err <= 2e-3 and abs(lse[b, hq] - l_ref) <= 2e-3, (b, hq, err)
            del kf, vf


RATE = {-1: 0, 0: 386, 1: 322, 2: 298}


def test_fullsize_repack_and_fused_append():
    """The full llama8b layer through the two measured steps beside the
    decode: an RDR re-pack to half of each sequence's bytes (seeded
    utilities) and one fused append + decode step on the re-packed cache,
    each against the oracle: caches byte for byte, outputs within 2e-3."""
    w = W.config("llama8b")
    log("full llama8b: pack both")
    gsrc, dev = gpu_pack(w)
    osrc = _oracle_pack(w)
    util = np.exp(np.random.default_rng(12).standard_normal((osrc.page_capacity, w["P"]))).astype(np.float32)
    budget = [int(0.5 * sum(RATE[int(x)] for x in w["tiers"][b].ravel())) for b in range(w["B"])]
    log("  re-pack")
    gdst = gpu_cache(w)
    ada.repack(gsrc, w["B"], torch.from_numpy(util).cuda(), budget, gdst)
    assert ada.read_status(gdst.status) == ada.OK
    odst = oracle_cache(w)
    st, _ = O.repack(osrc, w["B"], util, budget, odst)
    assert st == O.OK
    compare_caches(gdst, odst, w["P"])
    del gsrc, osrc
    log("  fused append + decode")
    rng = np.random.default_rng(13)
    B, Hkv = w["B"], w["Hkv"]
    keys = (rng.standard_normal((B, Hkv, 128)) * 2).astype(np.float32)
    vals = rng.standard_normal((B, Hkv, 128)).astype(np.float16).view(np.uint16)
    tiers = rng.integers(0, 3, (B, Hkv)).astype(np.uint8)
    out, lse = ada.decode_append(gdst, dev["q"], w["scale"], torch.from_numpy(keys).cuda(),
                                 torch.from_numpy(vals.view(np.int16)).cuda(), torch.from_numpy(tiers).cuda())
    assert ada.read_status(gdst.status) == ada.OK
    seq, head = np.repeat(np.arange(B), Hkv), np.tile(np.arange(Hkv), B)
    assert O.append(odst, seq, head, tiers.ravel(), keys.reshape(-1, 128), vals.reshape(-1, 128)) == O.OK
    compare_caches(gdst, odst, w["P"])
    o_ref, l_ref = O.decode(odst, w["q"], w["scale"])
    worst = check_outputs(out.cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref)
    log(f"  worst row rel err {worst:.2e}")
