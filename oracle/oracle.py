"""ctypes binding of the CPU oracle in ``ada_oracle.c``.

Test infrastructure only: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.
Every function here only marshals numpy arrays into the C oracle and back.
The method follows the abstract of "SPHERICAL KV: Angle-Domain Attention and
Rate-Distortion Retention for Efficient Long-Context Inference"
(arXiv 2605.18856, Abstract); the byte layout and rounding rules it leaves
open are fixed by this library's specification (see ``ada_oracle.c``).
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ada_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

OK, EINVAL, ENOSPC, EUNSUPPORTED, EUNDECIDABLE = 0, 1, 2, 3, 99
PAIRS_ADJACENT, PAIRS_HALF = 0, 1   # pair j = (k[2j], k[2j+1]) or (k[j], k[j+64])
TIER_BITS = {0: (8, 8), 1: (4, 4), 2: (2, 3), 3: (8, 8), 4: (4, 4), 5: (2, 3)}   # tier id -> (angle, magnitude bits)
VALUE_BITS = {0: 16, 1: 16, 2: 16, 3: 8, 4: 8, 5: 8}   # tier id -> value format (fp16 or V8)
NUM_TIERS = 6
D = 128
NP_PAIRS = 64


def build():
    """Compile the oracle with gcc (plain C, fp64, no FP contraction)."""
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-o", LIB, SRC,
                           "-lquadmath", "-lm", "-lpthread"])


_lib = None


def lib():
    """The oracle library; ORACLE_LIB names another build of ada_oracle.c
    (the sanitizer test loads an instrumented one)."""
    global _lib
    if _lib is None:
        alt = os.environ.get("ORACLE_LIB")
        if alt:
            _lib = ctypes.CDLL(alt)
            _declare(_lib)
            return _lib
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _lib = ctypes.CDLL(LIB)
        _declare(_lib)
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _declare(L):
    vp, i32, i64, u32, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_double
    L.orc_f64_to_f16.restype = ctypes.c_uint16
    L.orc_f64_to_f16.argtypes = [dbl]
    L.orc_f64_to_f16_many.argtypes = [vp, i64, vp]
    L.orc_f16_to_f64.restype = dbl
    L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
    L.orc_encode_key.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, ctypes.c_int]
    L.orc_encode_many.argtypes = [vp, i64, ctypes.c_int, ctypes.c_int, vp, vp, vp, ctypes.c_int]
    L.orc_bits_put.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int]
    L.orc_bits_get.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int]
    L.orc_block_bytes.restype = i64
    L.orc_block_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
    L.orc_key_bytes.restype = i64
    L.orc_key_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
    L.orc_pack.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, i64, vp, vp, vp,
                           i32, i64, i64, vp, vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int]
    L.orc_append.argtypes = [ctypes.c_int, ctypes.c_int, i32, i32, i64, i64, ctypes.c_int,
                             vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int]
    L.orc_rdr_steps.argtypes = [u32, vp, vp, vp, vp]
    L.orc_rdr_assign.argtypes = [ctypes.c_int, ctypes.c_int, vp, i64, vp, vp, u32, vp, vp]
    L.orc_transcode.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp]
    L.orc_repack.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, i32, vp, vp, vp, vp, vp, vp, u32,
                             i32, i64, i64, vp, vp, vp, vp, vp, vp, vp]
    L.orc_lut.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int]
    L.orc_decode.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, i32,
                             vp, vp, vp, vp, vp, dbl, vp, vp, ctypes.c_int, ctypes.c_int]
    L.orc_decode_utility.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, i32,
                                     vp, vp, vp, vp, vp, dbl, vp, ctypes.c_int, ctypes.c_int]
    L.orc_identity_logits.argtypes = [vp, i64, vp, vp, ctypes.c_int]
    L.orc_read_token.argtypes = [vp, vp, ctypes.c_int, i64, ctypes.c_int, vp, vp, vp, vp]
    L.orc_tier_rate.restype = i64
    L.orc_tier_rate.argtypes = [ctypes.c_int]
    L.orc_v8_encode.argtypes = [vp, vp, vp]
    L.orc_v8_decode.argtypes = [vp, vp, vp]
    L.orc_read_values.argtypes = [vp, vp, ctypes.c_int, i64, ctypes.c_int, vp]
    L.orc_value_index.restype = i64
    L.orc_value_index.argtypes = [ctypes.c_int, ctypes.c_int]


def f64_to_f16(x):
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f64_to_f16_many(_p(x), x.size, _p(out))
    return out


def f16_to_f64(h):
    return lib().orc_f16_to_f64(int(h))


def encode(keys, tb, sb, pair_layout=PAIRS_ADJACENT):
    """keys [n,128] fp32 -> (r16 [n] u16 fp16 bits, theta [n,64] u16, s [n,64] u16, status)."""
    keys = np.ascontiguousarray(keys, dtype=np.float32).reshape(-1, D)
    n = keys.shape[0]
    r16 = np.zeros(n, np.uint16)
    th = np.zeros((n, NP_PAIRS), np.uint16)
    s = np.zeros((n, NP_PAIRS), np.uint16)
    st = lib().orc_encode_many(_p(keys), n, tb, sb, _p(r16), _p(th), _p(s), pair_layout)
    return r16, th, s, st


def bits_put(codes, b):
    codes = np.ascontiguousarray(codes, dtype=np.uint16)
    out = np.zeros((codes.size * b + 7) // 8, np.uint8)
    lib().orc_bits_put(_p(out), b, _p(codes), codes.size)
    return out


def bits_get(buf, b, n):
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    out = np.zeros(n, np.uint16)
    lib().orc_bits_get(_p(buf), b, _p(out), n)
    return out


def block_bytes(tier, P):
    return lib().orc_block_bytes(tier, P)


class Cache:
    """Host copy of a paged ADA cache (the same buffers the library keeps on
    the device): page table, page counts, open pages, page metadata, code
    arena (each page's block: its key codes, then its values) and the two
    allocation counters.  pair_layout says
    which key and query components form the 64 pairs."""

    def __init__(self, P, Hq, Hkv, num_seqs, max_pages_per_head, page_capacity, arena_capacity16,
                 pair_layout=PAIRS_ADJACENT):
        self.P, self.Hq, self.Hkv = P, Hq, Hkv
        self.pair_layout = pair_layout
        self.num_seqs = num_seqs
        self.max_pages_per_head = max_pages_per_head
        self.page_capacity = page_capacity
        self.arena_capacity16 = arena_capacity16
        rows = num_seqs * Hkv
        self.page_table = np.zeros((rows, max_pages_per_head), np.int32)
        self.num_pages = np.zeros(rows, np.int32)
        self.open_page = np.full((rows, NUM_TIERS), -1, np.int32)
        self.page_meta = np.zeros((page_capacity, 8), np.uint8)
        self.arena = np.zeros(arena_capacity16 * 16, np.uint8)
        self.alloc = np.zeros(2, np.int64)

    def copy(self):
        c = Cache.__new__(Cache)
        c.__dict__.update({k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in self.__dict__.items()})
        return c

    def meta(self, page):
        m = self.page_meta[page]
        return int(m[0]), int(m[1]), int(m[4]) | (int(m[5]) << 8) | (int(m[6]) << 16) | (int(m[7]) << 24)


def pack(cache, ctx_len, tiers, keys, values, nthreads=None):
    """Bulk pack sequences 0..B-1 into `cache` (in place). Returns status."""
    ctx_len = np.ascontiguousarray(ctx_len, dtype=np.int32)
    tiers = np.ascontiguousarray(tiers, dtype=np.int8)
    keys = np.ascontiguousarray(keys, dtype=np.float32)
    values = np.ascontiguousarray(values, dtype=np.uint16)
    B, Hkv, stride = tiers.shape
    assert Hkv == cache.Hkv and keys.shape == (B, Hkv, stride, D) and values.shape == keys.shape
    nthreads = nthreads or max(1, len(os.sched_getaffinity(0)))
    return lib().orc_pack(cache.P, cache.Hkv, B, _p(ctx_len), stride, _p(tiers), _p(keys), _p(values),
                          cache.max_pages_per_head, cache.page_capacity, cache.arena_capacity16,
                          _p(cache.page_table), _p(cache.num_pages), _p(cache.open_page),
                          _p(cache.page_meta), _p(cache.arena), _p(cache.alloc),
                          nthreads, cache.pair_layout)


def append(cache, seq, head, tier, keys, values):
    seq = np.ascontiguousarray(seq, dtype=np.int32)
    head = np.ascontiguousarray(head, dtype=np.int32)
    tier = np.ascontiguousarray(tier, dtype=np.uint8)
    keys = np.ascontiguousarray(keys, dtype=np.float32).reshape(-1, D)
    values = np.ascontiguousarray(values, dtype=np.uint16).reshape(-1, D)
    n = seq.size
    return lib().orc_append(cache.P, cache.Hkv, cache.num_seqs, cache.max_pages_per_head,
                            cache.page_capacity, cache.arena_capacity16, n,
                            _p(seq), _p(head), _p(tier), _p(keys), _p(values),
                            _p(cache.page_table), _p(cache.num_pages), _p(cache.open_page),
                            _p(cache.page_meta), _p(cache.arena), _p(cache.alloc),
                            cache.pair_layout)


def rdr_steps(tier_mask):
    n = ctypes.c_int(0)
    st_tier = np.zeros(NUM_TIERS, np.int32)
    dR = np.zeros(NUM_TIERS, np.int64)
    c = np.zeros(NUM_TIERS, np.float64)
    st = lib().orc_rdr_steps(tier_mask, ctypes.byref(n), _p(st_tier), _p(dR), _p(c))
    return st, st_tier[:n.value], dR[:n.value], c[:n.value]


def rdr_assign(ctx_len, utility, budget, tier_mask=0b111, cap_level=None):
    """utility fp32 [B][Hkv][stride] -> (status, tiers int8 same shape).
    cap_level (optional int8, same shape): steps an item may take."""
    ctx_len = np.ascontiguousarray(ctx_len, dtype=np.int32)
    utility = np.ascontiguousarray(utility, dtype=np.float32)
    budget = np.ascontiguousarray(budget, dtype=np.int64)
    B, Hkv, stride = utility.shape
    out = np.full(utility.shape, -1, np.int8)
    cap = None if cap_level is None else np.ascontiguousarray(cap_level, dtype=np.int8)
    st = lib().orc_rdr_assign(Hkv, B, _p(ctx_len), stride, _p(utility), _p(budget), tier_mask,
                              None if cap is None else _p(cap), _p(out))
    return st, out


def transcode(tier_old, tier_new, theta, s):
    """codes [..., 64] of tier_old -> codes of tier_new (code-space rounding)."""
    theta = np.ascontiguousarray(theta, dtype=np.uint16).reshape(-1, NP_PAIRS)
    s = np.ascontiguousarray(s, dtype=np.uint16).reshape(-1, NP_PAIRS)
    th_n, s_n = np.zeros_like(theta), np.zeros_like(s)
    for i in range(theta.shape[0]):
        lib().orc_transcode(tier_old, tier_new, _p(theta[i]), _p(s[i]), _p(th_n[i:i + 1]), _p(s_n[i:i + 1]))
    return th_n, s_n


def repack(src, B, util, budget, dst, tier_mask=0):
    """RDR re-pack of sequences 0..B-1 of `src` into the empty cache `dst`
    from per-slot utilities util fp32 [page_capacity][P]; returns
    (status, tier map int8 [B][Hkv][src.max_pages_per_head * P])."""
    util = np.ascontiguousarray(util, dtype=np.float32)
    budget = np.ascontiguousarray(budget, dtype=np.int64)
    tv = np.full((B, src.Hkv, src.max_pages_per_head * src.P), -1, np.int8)
    st = lib().orc_repack(src.P, src.Hkv, B, src.max_pages_per_head, _p(src.page_table), _p(src.num_pages),
                          _p(src.page_meta), _p(src.arena), _p(util), _p(budget), tier_mask,
                          dst.max_pages_per_head, dst.page_capacity, dst.arena_capacity16, _p(dst.page_table),
                          _p(dst.num_pages), _p(dst.open_page), _p(dst.page_meta), _p(dst.arena),
                          _p(dst.alloc), _p(tv))
    return st, tv


def lut(q, tb, pair_layout=PAIRS_ADJACENT):
    q = np.ascontiguousarray(q, dtype=np.float32).reshape(D)
    out = np.zeros((NP_PAIRS, 1 << tb), np.float64)
    lib().orc_lut(_p(q), tb, _p(out), pair_layout)
    return out


def decode(cache, q, scale, nthreads=None):
    """q fp32 [B][Hq][128] -> (out fp64 [B][Hq][128], lse fp64 [B][Hq])."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    B, Hq, _ = q.shape
    assert Hq == cache.Hq
    out = np.zeros((B, Hq, D), np.float64)
    lse = np.zeros((B, Hq), np.float64)
    nthreads = nthreads or max(1, len(os.sched_getaffinity(0)))
    st = lib().orc_decode(cache.P, cache.Hq, cache.Hkv, B, cache.max_pages_per_head,
                          _p(cache.page_table), _p(cache.num_pages), _p(cache.page_meta),
                          _p(cache.arena), _p(q), float(scale),
                          _p(out), _p(lse), nthreads, cache.pair_layout)
    assert st == OK, st
    return out, lse


def decode_utility(cache, q, scale, util=None, nthreads=None):
    """Attention mass of every kept token for q fp32 [B][Hq][128]: returns
    util fp64 [page_capacity][P], util[page][slot] = sum over the KV head's
    query heads of the token's softmax weight; entries of slots holding no
    kept token of sequences 0..B-1 keep their input value (NaN by default)."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    B, Hq, _ = q.shape
    assert Hq == cache.Hq
    if util is None:
        util = np.full((cache.page_capacity, cache.P), np.nan, np.float64)
    nthreads = nthreads or max(1, len(os.sched_getaffinity(0)))
    st = lib().orc_decode_utility(cache.P, cache.Hq, cache.Hkv, B, cache.max_pages_per_head,
                                  _p(cache.page_table), _p(cache.num_pages), _p(cache.page_meta),
                                  _p(cache.arena), _p(q), float(scale), _p(util), nthreads, cache.pair_layout)
    assert st == OK, st
    return util


def identity_logits(keys, q, pair_layout=PAIRS_ADJACENT):
    keys = np.ascontiguousarray(keys, dtype=np.float32).reshape(-1, D)
    q = np.ascontiguousarray(q, dtype=np.float32).reshape(D)
    out = np.zeros(keys.shape[0], np.float64)
    lib().orc_identity_logits(_p(keys), keys.shape[0], _p(q), _p(out), pair_layout)
    return out


def read_token(cache, page, slot):
    r16 = np.zeros(1, np.uint16)
    th = np.zeros(NP_PAIRS, np.uint16)
    s = np.zeros(NP_PAIRS, np.uint16)
    tier = ctypes.c_int(0)
    lib().orc_read_token(_p(cache.arena), _p(cache.page_meta), cache.P, page, slot,
                         _p(r16), _p(th), _p(s), ctypes.byref(tier))
    return int(r16[0]), th, s, tier.value


def tier_rate(tier):
    return lib().orc_tier_rate(tier)


def v8_encode(values):
    """fp16 bits [128] -> (status, scale bytes [4] u8, codes [128] int8)."""
    v = np.ascontiguousarray(values, dtype=np.uint16).reshape(D)
    sb = np.zeros(4, np.uint8)
    c = np.zeros(D, np.int8)
    st = lib().orc_v8_encode(_p(v), _p(sb), _p(c))
    return st, sb, c


def v8_decode(scale_bytes, codes):
    sb = np.ascontiguousarray(scale_bytes, dtype=np.uint8).reshape(4)
    c = np.ascontiguousarray(codes, dtype=np.int8).reshape(D)
    out = np.zeros(D, np.float64)
    lib().orc_v8_decode(_p(sb), _p(c), _p(out))
    return out


def read_values(cache, page, slot):
    """decoded values (fp64 [128]) of a cached token, in its page's format"""
    out = np.zeros(D, np.float64)
    lib().orc_read_values(_p(cache.arena), _p(cache.page_meta), cache.P, page, slot, _p(out))
    return out


def value_index(slot, d):
    """u16 index of fp16 value (slot, d) inside an fp16 page's value part"""
    return lib().orc_value_index(slot, d)


def key_bytes(tier, P):
    """bytes of a page's key part (radius and codes); its value part follows"""
    return lib().orc_key_bytes(tier, P)


def value_part(cache, page):
    """the value part of a page's block, as bytes (a view into the arena)"""
    tier, _, off16 = cache.meta(page)
    start = off16 * 16 + key_bytes(tier, cache.P)
    return cache.arena[start: off16 * 16 + block_bytes(tier, cache.P)]
