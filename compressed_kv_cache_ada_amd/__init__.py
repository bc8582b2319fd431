"""Python binding of ``libada.so``, the MI355X (gfx950) ADA paged-decode library.

Argument marshalling only: every step of the method runs in the HIP kernels
behind the C ABI of ``include/ada.h``.  PyTorch supplies device memory and the
current HIP stream.  The functions keep the C names without the ``ada_``
prefix (``ada_decode`` -> ``decode``) and raise ``AdaError`` on any non-OK
status.  There is no CPU fallback: if the library is not built, importing
works but every call raises.

Method: "SPHERICAL KV: Angle-Domain Attention and Rate-Distortion Retention
for Efficient Long-Context Inference" (arXiv 2605.18856), Abstract.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libada.so")

OK, EINVAL, ENOSPC, EUNSUPPORTED, EHIP, EINTERNAL = 0, 1, 2, 3, 4, 5
T8, T4, T2 = 0, 1, 2
TIER_BITS = {T8: (8, 8), T4: (4, 4), T2: (2, 3)}
D = 128


class AdaError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__(f"{what}: {status_str(status) if _lib is not None else status}")


class Config(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("rdr_tier_mask", ctypes.c_uint32), ("decode_chunk_pages", ctypes.c_int32),
                ("pair_layout", ctypes.c_int32), ("value_tiers", ctypes.c_int32)]


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("max_pages_per_head", ctypes.c_int32),
                ("page_capacity", ctypes.c_int64), ("arena_capacity16", ctypes.c_int64),
                ("page_table", ctypes.c_void_p), ("num_pages", ctypes.c_void_p),
                ("open_page", ctypes.c_void_p), ("page_meta", ctypes.c_void_p),
                ("code_arena", ctypes.c_void_p), ("alloc", ctypes.c_void_p), ("status", ctypes.c_void_p),
                ("row_order", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libada.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with compressed_kv_cache_ada_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        _declare(L)
        _lib = L
    return _lib


def _declare(L):
    vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    cfgp, cachep = ctypes.POINTER(Config), ctypes.POINTER(CacheDesc)
    st = ctypes.c_int
    sig = {
        "ada_status_str": (ctypes.c_char_p, [st]),
        "ada_block_bytes": (i64, [i32, i32]),
        "ada_lut_floats": (sz, [cfgp]),
        "ada_cache_init": (st, [cfgp, cachep, vp]),
        "ada_validate_cache": (st, [cfgp, cachep, i32, vp]),
        "ada_build_lut": (st, [cfgp, vp, i32, vp, vp]),
        "ada_decode_workspace": (st, [cfgp, cachep, i32, ctypes.POINTER(sz)]),
        "ada_decode": (st, [cfgp, cachep, vp, i32, f32, vp, vp, vp, sz, vp]),
        "ada_decode_noalloc": (st, [cfgp, cachep, vp, i32, f32, vp, vp, vp]),
        "ada_decode_partials": (st, [cfgp, cachep, vp, i32, f32, vp, sz, vp]),
        "ada_decode_reduce": (st, [cfgp, cachep, i32, vp, vp, vp, sz, vp]),
        "ada_decode_multi_workspace": (st, [cfgp, cachep, i32, i32, ctypes.POINTER(sz)]),
        "ada_decode_multi": (st, [cfgp, cachep, vp, i32, i32, f32, vp, vp, vp, sz, vp]),
        "ada_decode_utility_workspace": (st, [cfgp, cachep, i32, ctypes.POINTER(sz)]),
        "ada_decode_utility": (st, [cfgp, cachep, vp, i32, f32, vp, vp, vp, vp, sz, vp]),
        "ada_repack_workspace": (st, [cfgp, cachep, i32, ctypes.POINTER(sz)]),
        "ada_repack": (st, [cfgp, cachep, i32, vp, vp, cachep, vp, sz, vp]),
        "ada_decode_append_workspace": (st, [cfgp, cachep, i32, ctypes.POINTER(sz)]),
        "ada_decode_append": (st, [cfgp, cachep, vp, i32, f32, vp, vp, vp, vp, vp, vp, sz, vp]),
        "ada_append_workspace": (st, [cfgp, cachep, i32, ctypes.POINTER(sz)]),
        "ada_encode_append": (st, [cfgp, cachep, i32, vp, vp, vp, vp, vp, vp, sz, vp]),
        "ada_rdr_workspace": (st, [cfgp, i32, i64, ctypes.POINTER(sz)]),
        "ada_rdr_assign": (st, [cfgp, i32, vp, i64, vp, vp, vp, vp, vp, sz, vp]),
        "ada_pack_workspace": (st, [cfgp, cachep, i32, i64, ctypes.POINTER(sz)]),
        "ada_pack": (st, [cfgp, cachep, i32, vp, i64, vp, vp, vp, vp, sz, vp]),
        "ada_read_status": (st, [vp, vp]),
        "ada_dense_workspace": (st, [cfgp, i32, i32, ctypes.POINTER(sz)]),
        "ada_dense_decode": (st, [cfgp, i32, i32, vp, vp, vp, vp, vp, f32, vp, vp, vp, sz, vp]),
        "ada_probe_copy": (st, [vp, vp, sz, vp]),
        "ada_probe_read": (st, [vp, sz, i32, vp, vp]),
        "ada_host_f64_to_f16": (ctypes.c_uint16, [ctypes.c_double]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args


ABI_SYMBOLS = ("ada_status_str", "ada_block_bytes", "ada_lut_floats", "ada_cache_init", "ada_validate_cache",
               "ada_build_lut",
               "ada_decode_workspace", "ada_decode", "ada_decode_noalloc", "ada_decode_partials", "ada_decode_reduce",
               "ada_decode_multi_workspace", "ada_decode_multi", "ada_decode_append_workspace",
               "ada_decode_append", "ada_decode_utility_workspace", "ada_decode_utility", "ada_repack_workspace",
               "ada_repack",
               "ada_append_workspace", "ada_encode_append", "ada_rdr_workspace", "ada_rdr_assign",
               "ada_pack_workspace", "ada_pack", "ada_read_status", "ada_dense_workspace",
               "ada_dense_decode", "ada_probe_copy", "ada_probe_read", "ada_host_f64_to_f16")


def status_str(s):
    return lib().ada_status_str(int(s)).decode()


def _check(status, what):
    if status != OK:
        raise AdaError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, dtype, name):
    if t is None:
        return None
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name}: need a contiguous {dtype} tensor on the GPU, got {t.dtype} {t.device}")
    return t


def block_bytes(tier, page_size):
    return int(lib().ada_block_bytes(tier, page_size))


NUM_TIERS = 6   # T8, T4, T2 (fp16 values), T8V8, T4V8, T2V8 (V8 values)
PAIRS_ADJACENT, PAIRS_HALF_SPLIT = 0, 1   # pair j = (x[2j], x[2j+1]) or (x[j], x[j+64])


def make_config(page_size, num_q_heads, num_kv_heads, rdr_tier_mask=0, decode_chunk_pages=0,
                pair_layout=PAIRS_ADJACENT, value_tiers=False):
    return Config(D, page_size, num_q_heads, num_kv_heads, rdr_tier_mask, decode_chunk_pages, pair_layout,
                  int(bool(value_tiers)))


class Cache:
    """Device buffers of one layer's ADA cache (torch tensors) and the C
    descriptor that points at them."""

    def __init__(self, cfg, num_seqs, max_pages_per_head, page_capacity, arena_capacity16, device="cuda"):
        self.cfg = cfg
        rows = num_seqs * cfg.num_kv_heads
        self.page_table = torch.zeros((rows, max_pages_per_head), dtype=torch.int32, device=device)
        self.num_pages = torch.zeros(rows, dtype=torch.int32, device=device)
        self.open_page = torch.full((rows, NUM_TIERS), -1, dtype=torch.int32, device=device)
        self.page_meta = torch.zeros((page_capacity, 8), dtype=torch.uint8, device=device)
        self.code_arena = torch.zeros(arena_capacity16 * 16, dtype=torch.uint8, device=device)
        self.alloc = torch.zeros(2, dtype=torch.int64, device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)
        self.row_order = torch.arange(rows, dtype=torch.int32, device=device)
        self.desc = CacheDesc(num_seqs, max_pages_per_head, page_capacity, arena_capacity16,
                              self.page_table.data_ptr(), self.num_pages.data_ptr(), self.open_page.data_ptr(),
                              self.page_meta.data_ptr(), self.code_arena.data_ptr(), self.alloc.data_ptr(),
                              self.status.data_ptr(), self.row_order.data_ptr())

    def host(self):
        """numpy copies of every buffer (for comparisons)."""
        import numpy as np
        return {"page_table": self.page_table.cpu().numpy(), "num_pages": self.num_pages.cpu().numpy(),
                "open_page": self.open_page.cpu().numpy(), "page_meta": self.page_meta.cpu().numpy(),
                "arena": self.code_arena.cpu().numpy(), "alloc": self.alloc.cpu().numpy()}


def cache_init(cache):
    _check(lib().ada_cache_init(ctypes.byref(cache.cfg), ctypes.byref(cache.desc), _stream()), "ada_cache_init")


def validate_cache(cache, B):
    """Range-check the page lists of sequences 0..B-1 on the device; the
    verdict lands in cache.status (read it with read_status)."""
    _check(lib().ada_validate_cache(ctypes.byref(cache.cfg), ctypes.byref(cache.desc), B, _stream()),
           "ada_validate_cache")


def lut_floats(cfg):
    return int(lib().ada_lut_floats(ctypes.byref(cfg)))


def build_lut(cfg, q, lut=None):
    q = _dev(q, torch.float32, "q")
    B = q.shape[0]
    if lut is None:
        lut = torch.empty((B, cfg.num_q_heads, lut_floats(cfg)), dtype=torch.float32, device=q.device)
    _check(lib().ada_build_lut(ctypes.byref(cfg), _ptr(q), B, _ptr(lut), _stream()), "ada_build_lut")
    return lut


def decode_workspace(cache, B):
    n = ctypes.c_size_t(0)
    _check(lib().ada_decode_workspace(ctypes.byref(cache.cfg), ctypes.byref(cache.desc), B, ctypes.byref(n)),
           "ada_decode_workspace")
    return torch.empty(max(1, n.value), dtype=torch.uint8, device=cache.page_table.device)


def decode(cache, q, scale, out=None, lse=None, ws=None):
    q = _dev(q, torch.float32, "q")
    B = q.shape[0]
    if out is None:
        out = torch.empty((B, cache.cfg.num_q_heads, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, cache.cfg.num_q_heads), dtype=torch.float32, device=q.device)
    ws = decode_workspace(cache, B) if ws is None else ws
    _check(lib().ada_decode(ctypes.byref(cache.cfg), ctypes.byref(cache.desc), _ptr(q), B, float(scale),
                            _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream()), "ada_decode")
    return out, lse


def decode_noalloc(cache, q, scale, out=None, lse=None):
    """ada_decode with the library's own per-GPU partials array (no workspace)."""
    q = _dev(q, torch.float32, "q")
    B = q.shape[0]
    if out is None:
        out = torch.empty((B, cache.cfg.num_q_heads, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, cache.cfg.num_q_heads), dtype=torch.float32, device=q.device)
    _check(lib().ada_decode_noalloc(ctypes.byref(cache.cfg), ctypes.byref(cache.desc), _ptr(q), B, float(scale),
                                    _ptr(out), _ptr(lse), _stream()), "ada_decode_noalloc")
    return out, lse


def decode_multi_workspace(cache, B, Q):
    n = ctypes.c_size_t(0)
    _check(lib().ada_decode_multi_workspace(ctypes.byref(cache.cfg), ctypes.byref(cache.desc), B, Q,
                                            ctypes.byref(n)), "ada_decode_multi_workspace")
    return torch.empty(max(1, n.value), dtype=torch.uint8, device=cache.page_table.device)


def decode_multi(cache, q, scale, out=None, lse=None, ws=None):
    """q: fp32 [B][Q][Hq][128] -> out [B][Q][Hq][128], lse [B][Q][Hq]."""
    q = _dev(q, torch.float32, "q")
    B, Q = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty((B, Q, cache.cfg.num_q_heads, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Q, cache.cfg.num_q_heads), dtype=torch.float32, device=q.device)
    ws = decode_multi_workspace(cache, B, Q) if ws is None else ws
    _check(lib().ada_decode_multi(ctypes.byref(cache.cfg), ctypes.byref(cache.desc), _ptr(q), B, Q, float(scale),
                                  _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream()), "ada_decode_multi")
    return out, lse


def decode_partials(cache, q, scale, ws):
    q = _dev(q, torch.float32, "q")
    _check(lib().ada_decode_partials(ctypes.byref(cache.cfg), ctypes.byref(cache.desc), _ptr(q), q.shape[0],
                                     float(scale), _ptr(ws), ws.numel(), _stream()), "ada_decode_partials")


def decode_reduce(cache, B, out, lse, ws):
    _check(lib().ada_decode_reduce(ctypes.byref(cache.cfg), ctypes.byref(cache.desc), B, _ptr(out), _ptr(lse),
                                   _ptr(ws), ws.numel(), _stream()), "ada_decode_reduce")


def append_workspace_bytes(cache, n):
    sz = ctypes.c_size_t(0)
    _check(lib().ada_append_workspace(ctypes.byref(cache.cfg), ctypes.byref(cache.desc), n, ctypes.byref(sz)),
           "ada_append_workspace")
    return sz.value


def encode_append(cache, seq, kv_head, tier, keys, values, ws=None):
    seq = _dev(seq, torch.int32, "seq")
    kv_head = _dev(kv_head, torch.int32, "kv_head")
    tier = _dev(tier, torch.uint8, "tier")
    keys = _dev(keys, torch.float32, "keys")
    values = _dev(values, torch.int16, "values")
    n = seq.numel()
    if ws is None:
        sz = ctypes.c_size_t(0)
        _check(lib().ada_append_workspace(ctypes.byref(cache.cfg), ctypes.byref(cache.desc), n, ctypes.byref(sz)),
               "ada_append_workspace")
        ws = torch.empty(max(1, sz.value), dtype=torch.uint8, device=keys.device)
    _check(lib().ada_encode_append(ctypes.byref(cache.cfg), ctypes.byref(cache.desc), n, _ptr(seq), _ptr(kv_head),
                                   _ptr(tier), _ptr(keys), _ptr(values), _ptr(ws), ws.numel(), _stream()),
           "ada_encode_append")


def decode_utility_workspace(cache, B):
    n = ctypes.c_size_t(0)
    _check(lib().ada_decode_utility_workspace(ctypes.byref(cache.cfg), ctypes.byref(cache.desc), B,
                                              ctypes.byref(n)), "ada_decode_utility_workspace")
    return torch.empty(max(1, n.value), dtype=torch.uint8, device=cache.page_table.device)


def decode_utility(cache, q, scale, util=None, out=None, lse=None, ws=None):
    """Decode q ([B][Hq][128]) and write every kept token's attention mass
    into util (fp32 [page_capacity][P]; a new NaN-filled tensor if None)."""
    q = _dev(q, torch.float32, "q")
    B = q.shape[0]
    if util is None:
        util = torch.full((cache.desc.page_capacity, cache.cfg.page_size), float("nan"), dtype=torch.float32,
                          device=q.device)
    if out is None:
        out = torch.empty((B, cache.cfg.num_q_heads, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, cache.cfg.num_q_heads), dtype=torch.float32, device=q.device)
    ws = decode_utility_workspace(cache, B) if ws is None else ws
    _check(lib().ada_decode_utility(ctypes.byref(cache.cfg), ctypes.byref(cache.desc), _ptr(q), B, float(scale),
                                    _ptr(out), _ptr(lse), _ptr(util), _ptr(ws), ws.numel(), _stream()),
           "ada_decode_utility")
    return out, lse, util


def repack_workspace(src, B):
    n = ctypes.c_size_t(0)
    _check(lib().ada_repack_workspace(ctypes.byref(src.cfg), ctypes.byref(src.desc), B, ctypes.byref(n)),
           "ada_repack_workspace")
    return torch.empty(max(1, n.value), dtype=torch.uint8, device=src.page_table.device)


def repack(src, B, util, budget, dst, ws=None):
    """RDR re-pack of sequences 0..B-1 of `src` into `dst` from per-slot
    utilities util (device fp32 [page_capacity][P]) under budget (host
    sequence of B byte counts).  Device errors land in dst.status."""
    util = _dev(util, torch.float32, "util")
    bud = (ctypes.c_int64 * B)(*[int(x) for x in budget])
    ws = repack_workspace(src, B) if ws is None else ws
    _check(lib().ada_repack(ctypes.byref(src.cfg), ctypes.byref(src.desc), B, _ptr(util), bud,
                            ctypes.byref(dst.desc), _ptr(ws), ws.numel(), _stream()), "ada_repack")


def decode_append_workspace(cache, B):
    n = ctypes.c_size_t(0)
    _check(lib().ada_decode_append_workspace(ctypes.byref(cache.cfg), ctypes.byref(cache.desc), B, ctypes.byref(n)),
           "ada_decode_append_workspace")
    return torch.empty(max(1, n.value), dtype=torch.uint8, device=cache.page_table.device)


def decode_append(cache, q, scale, new_keys, new_values, new_tier, out=None, lse=None, ws=None):
    """One decode step: append new_keys / new_values ([B][Hkv][128]) at
    new_tier ([B][Hkv]) and decode q ([B][Hq][128]) over the cache including
    them.  Device errors land in cache.status (read with read_status)."""
    q = _dev(q, torch.float32, "q")
    new_keys = _dev(new_keys, torch.float32, "new_keys")
    new_values = _dev(new_values, torch.int16, "new_values")
    new_tier = _dev(new_tier, torch.uint8, "new_tier")
    B = q.shape[0]
    if out is None:
        out = torch.empty((B, cache.cfg.num_q_heads, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, cache.cfg.num_q_heads), dtype=torch.float32, device=q.device)
    ws = decode_append_workspace(cache, B) if ws is None else ws
    _check(lib().ada_decode_append(ctypes.byref(cache.cfg), ctypes.byref(cache.desc), _ptr(q), B, float(scale),
                                   _ptr(new_keys), _ptr(new_values), _ptr(new_tier), _ptr(out), _ptr(lse),
                                   _ptr(ws), ws.numel(), _stream()), "ada_decode_append")
    return out, lse


def rdr_assign(cfg, ctx_len, utility, budget, status, tier_out=None):
    """ctx_len / budget: host sequences; utility: device fp32 [B][Hkv][stride]."""
    utility = _dev(utility, torch.float32, "utility")
    B, Hkv, stride = utility.shape
    ctx = (ctypes.c_int32 * B)(*[int(x) for x in ctx_len])
    bud = (ctypes.c_int64 * B)(*[int(x) for x in budget])
    if tier_out is None:
        tier_out = torch.empty((B, Hkv, stride), dtype=torch.int8, device=utility.device)
    sz = ctypes.c_size_t(0)
    _check(lib().ada_rdr_workspace(ctypes.byref(cfg), B, stride, ctypes.byref(sz)), "ada_rdr_workspace")
    ws = torch.empty(max(1, sz.value), dtype=torch.uint8, device=utility.device)
    _check(lib().ada_rdr_assign(ctypes.byref(cfg), B, ctx, stride, _ptr(utility), bud, _ptr(tier_out),
                                _ptr(status), _ptr(ws), ws.numel(), _stream()), "ada_rdr_assign")
    return tier_out


def pack(cache, ctx_len, tiers, keys, values):
    """ctx_len: host sequence; tiers int8 / keys fp32 / values int16(fp16 bits) on the device."""
    tiers = _dev(tiers, torch.int8, "tiers")
    keys = _dev(keys, torch.float32, "keys")
    values = _dev(values, torch.int16, "values")
    B, Hkv, stride = tiers.shape
    ctx = (ctypes.c_int32 * B)(*[int(x) for x in ctx_len])
    sz = ctypes.c_size_t(0)
    _check(lib().ada_pack_workspace(ctypes.byref(cache.cfg), ctypes.byref(cache.desc), B, stride, ctypes.byref(sz)),
           "ada_pack_workspace")
    ws = torch.empty(max(1, sz.value), dtype=torch.uint8, device=keys.device)
    _check(lib().ada_pack(ctypes.byref(cache.cfg), ctypes.byref(cache.desc), B, ctx, stride, _ptr(tiers),
                          _ptr(keys), _ptr(values), _ptr(ws), ws.numel(), _stream()), "ada_pack")
    return ws


def read_status(status):
    """Synchronise, return and clear a device status word (int)."""
    return int(lib().ada_read_status(_ptr(status), _stream()))


def dense_workspace(cfg, B, max_pages_per_head, device="cuda"):
    sz = ctypes.c_size_t(0)
    _check(lib().ada_dense_workspace(ctypes.byref(cfg), B, max_pages_per_head, ctypes.byref(sz)),
           "ada_dense_workspace")
    return torch.empty(max(1, sz.value), dtype=torch.uint8, device=device)


def dense_decode(cfg, page_table, ctx_len, k_pool, v_pool, q, scale, out=None, lse=None, ws=None):
    q = _dev(q, torch.float32, "q")
    B = q.shape[0]
    maxp = page_table.shape[1]
    if out is None:
        out = torch.empty((B, cfg.num_q_heads, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, cfg.num_q_heads), dtype=torch.float32, device=q.device)
    ws = dense_workspace(cfg, B, maxp, q.device) if ws is None else ws
    _check(lib().ada_dense_decode(ctypes.byref(cfg), B, maxp, _ptr(page_table), _ptr(ctx_len), _ptr(k_pool),
                                  _ptr(v_pool), _ptr(q), float(scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                  _stream()), "ada_dense_decode")
    return out, lse


def probe_copy(src, dst, nbytes):
    _check(lib().ada_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream()), "ada_probe_copy")


def probe_read(src, nbytes, variant, out):
    _check(lib().ada_probe_read(_ptr(src), nbytes, variant, _ptr(out), _stream()), "ada_probe_read")


def host_f64_to_f16(x):
    return int(lib().ada_host_f64_to_f16(float(x)))
