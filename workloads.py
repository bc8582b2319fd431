"""Seeded synthetic inputs for ADA paged decode.

This module only draws random numbers and makes the workload's structural
choices (which tokens are dropped, which kept tokens go to which tier, how
physical pages are permuted).  It holds none of the method's arithmetic, and
both the CPU oracle and the HIP path consume exactly the arrays it returns.

Workloads (names used by the tests and the benchmark):

* ``tiny``      1 sequence, 1 query head / 1 KV head, head dim 128, context
                4096, page size 16, every token in the 4-bit tier, no drops.
* ``llama8b``   Llama-3-8B-like layer: batch 8, 32 query / 8 KV heads, context
                32768, page size 16; per (sequence, KV head) exactly 25% of
                tokens dropped at random; kept tokens assigned to tiers by a
                random permutation so that 307 / 768 / 461 full pages go to
                T8 / T4 / T2.
* ``rdr128k``   batch 4, 32 / 8 heads, context 131072, page size 16; utility
                lognormal(0,1) per (sequence, head, token); byte budget 35% of
                the dense fp16 KV of each sequence; tiers come from the RDR
                packer.
* ``ragged``    64 sequences, contexts uniform in [1024, 16384], 32 / 8 heads,
                page size 16; per sequence a drop rate uniform in [0, 0.5) and
                tier fractions Dirichlet(1,1,1); physical pages permuted over
                the shared pool after packing.
* ``long256k``  70B-like: batch 1, 64 / 8 heads, context 262144, page size 32,
                every kept token in T4, 40% of tokens dropped per head.

Distributions shared by all workloads: keys are fp32, N(0,1) per channel times
a per-channel scale exp(0.5 z) (lognormal(0, 0.5)) drawn per KV head, with 4
distinct channels per KV head multiplied by 8; values N(0,1) rounded to fp16;
queries N(0,1) fp32; softmax scale 1/sqrt(128).

The public evaluation suites the paper's area uses (long-context QA and
retrieval benchmarks) are not available here; these synthetic shapes stand in
for them and no benchmark item is reproduced.
"""
import numpy as np

D = 128
SEED_BASE = 1000
WORKLOADS = ("tiny", "llama8b", "rdr128k", "ragged", "long256k")
# index of each workload in the seed scheme (seed = 1000 + index)
_INDEX = {name: i for i, name in enumerate(WORKLOADS)}
T8, T4, T2, DROP = 0, 1, 2, -1


def _streams(name, salt=0):
    ss = np.random.SeedSequence(SEED_BASE + _INDEX[name] + 7919 * salt)
    kids = ss.spawn(8)
    names = ("key_scale", "keys", "values", "query", "drop", "tier", "utility", "perm")
    return {n: np.random.default_rng(k) for n, k in zip(names, kids)}


def key_scales(rng, Hkv):
    """Per-KV-head channel scales: lognormal(0, 0.5) with 4 outlier channels x8."""
    sig = np.exp(0.5 * rng.standard_normal((Hkv, D)))
    for h in range(Hkv):
        ch = rng.choice(D, size=4, replace=False)
        sig[h, ch] *= 8.0
    return sig


def draw_keys(rng_scale, rng_keys, B, Hkv, stride):
    sig = key_scales(rng_scale, Hkv).astype(np.float32)
    k = rng_keys.standard_normal((B, Hkv, stride, D), dtype=np.float32)
    k *= sig[None, :, None, :]
    return k


def draw_values(rng, B, Hkv, stride):
    v = rng.standard_normal((B, Hkv, stride, D), dtype=np.float32).astype(np.float16)
    return v.view(np.uint16)


def draw_queries(rng, B, Hq):
    return rng.standard_normal((B, Hq, D), dtype=np.float32)


def config(name, ctx=None, batch=None, salt=0):
    """Build a workload.  `ctx` / `batch` override the context length / batch
    (for reduced-size tests); the structure and distributions stay the same.

    Returns a dict with: name, P, Hq, Hkv, B, ctx_len (int32 [B]), stride,
    keys (fp32 [B][Hkv][stride][128]), values (fp16 bits, same shape),
    q (fp32 [B][Hq][128]), scale, and either `tiers` (int8 [B][Hkv][stride],
    -1 = drop) or, for ``rdr128k``, `utility` (fp32) and `budget` (int64 [B]).
    ``ragged`` also carries `perm_rng` for the physical page permutation."""
    R = _streams(name, salt)
    w = {"name": name, "scale": 1.0 / np.sqrt(D)}
    if name == "tiny":
        B, Hq, Hkv, P, c = 1, 1, 1, 16, 4096
        B = batch or B
        c = ctx or c
        ctx_len = np.full(B, c, np.int32)
        tiers = np.full((B, Hkv, c), T4, np.int8)
    elif name == "llama8b":
        B, Hq, Hkv, P, c = 8, 32, 8, 16, 32768
        B = batch or B
        c = ctx or c
        ctx_len = np.full(B, c, np.int32)
        tiers = np.full((B, Hkv, c), DROP, np.int8)
        n_drop = c // 4
        kept = c - n_drop
        n_pages = kept // P
        p8 = int(round(0.2 * n_pages))
        p4 = int(round(0.5 * n_pages))
        for b in range(B):
            for h in range(Hkv):
                order = R["drop"].permutation(c)
                kept_idx = np.sort(order[n_drop:])
                perm = R["tier"].permutation(kept)
                tier_of = np.full(kept, T2, np.int8)
                tier_of[perm[: p8 * P]] = T8
                tier_of[perm[p8 * P: (p8 + p4) * P]] = T4
                tiers[b, h, kept_idx] = tier_of
    elif name == "long256k":
        B, Hq, Hkv, P, c = 1, 64, 8, 32, 262144
        B = batch or B
        c = ctx or c
        ctx_len = np.full(B, c, np.int32)
        tiers = np.full((B, Hkv, c), T4, np.int8)
        n_drop = int(round(0.4 * c))
        for b in range(B):
            for h in range(Hkv):
                drop = R["drop"].choice(c, size=n_drop, replace=False)
                tiers[b, h, drop] = DROP
    elif name == "ragged":
        B, Hq, Hkv, P = 64, 32, 8, 16
        B = batch or B
        lo, hi = 1024, 16384
        if ctx:
            lo, hi = max(1, ctx // 16), ctx
        ctx_len = R["drop"].integers(lo, hi + 1, size=B).astype(np.int32)
        c = int(ctx_len.max())
        tiers = np.full((B, Hkv, c), DROP, np.int8)
        for b in range(B):
            L = int(ctx_len[b])
            rate = R["drop"].uniform(0.0, 0.5)
            f8, f4, _ = R["tier"].dirichlet((1.0, 1.0, 1.0))
            for h in range(Hkv):
                n_drop = int(round(rate * L))
                order = R["drop"].permutation(L)
                kept_idx = np.sort(order[n_drop:])
                k = kept_idx.size
                n8 = int(round(f8 * k))
                n4 = min(int(round(f4 * k)), k - n8)
                perm = R["tier"].permutation(k)
                tier_of = np.full(k, T2, np.int8)
                tier_of[perm[:n8]] = T8
                tier_of[perm[n8:n8 + n4]] = T4
                tiers[b, h, kept_idx] = tier_of
        w["perm_rng"] = R["perm"]
    elif name == "rdr128k":
        B, Hq, Hkv, P, c = 4, 32, 8, 16, 131072
        B = batch or B
        c = ctx or c
        ctx_len = np.full(B, c, np.int32)
        tiers = None
        util = np.exp(R["utility"].standard_normal((B, Hkv, c))).astype(np.float32)
        w["utility"] = util
        w["budget"] = np.array([(35 * int(L) * Hkv * 512) // 100 for L in ctx_len], np.int64)
    else:
        raise ValueError(name)
    stride = int(c)
    w.update(P=P, Hq=Hq, Hkv=Hkv, B=B, ctx_len=ctx_len, stride=stride)
    w["keys"] = draw_keys(R["key_scale"], R["keys"], B, Hkv, stride)
    w["values"] = draw_values(R["values"], B, Hkv, stride)
    w["q"] = draw_queries(R["query"], B, Hq)
    # positions past a sequence's context are padding: never kept
    if tiers is not None:
        for b in range(B):
            tiers[b, :, int(ctx_len[b]):] = DROP
    w["tiers"] = tiers
    return w


def page_permutation(rng, n_pages):
    """Seeded permutation of physical page ids (new id = perm[old id])."""
    return rng.permutation(n_pages).astype(np.int32)



def dense_pages(keys16, values16, P):
    """Dense fp16 reference layout (a measurement companion, not the
    method): lay out un-dropped fp16 keys / values [B][Hkv][ctx][128] (uint16 bits)
    as dense pages: key page [16 dim blocks][P][8], value page [P/8][128][8];
    row (b, h) owns pages row*npr .. row*npr + npr - 1.  Returns
    (k_pool [pages][P*128], v_pool [pages][P*128], page_table [rows][npr])."""
    B, H, ctx, _ = keys16.shape
    npr = -(-ctx // P)
    pad = npr * P - ctx
    k = np.pad(keys16, ((0, 0), (0, 0), (0, pad), (0, 0)))
    v = np.pad(values16, ((0, 0), (0, 0), (0, pad), (0, 0)))
    k = k.reshape(B * H * npr, P, 16, 8).transpose(0, 2, 1, 3).reshape(B * H * npr, P * 128)
    v = v.reshape(B * H * npr, P // 8, 8, 128).transpose(0, 1, 3, 2).reshape(B * H * npr, P * 128)
    pt = np.arange(B * H * npr, dtype=np.int32).reshape(B * H, npr)
    return np.ascontiguousarray(k), np.ascontiguousarray(v), pt
