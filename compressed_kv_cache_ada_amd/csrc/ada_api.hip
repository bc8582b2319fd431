// ada_api.hip -- host side of the C ABI declared in include/ada.h:
// argument validation, workspace layout and kernel launches.  No memory is
// allocated here; nothing throws across the boundary.
#include <string.h>

#include <algorithm>
#include <mutex>

#include "ada_internal.h"

using namespace ada;

namespace {

inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

// Multi-query decode: at most this many virtual heads (Q * Hq / Hkv) per KV head.
constexpr int kMaxVirtualHeads = 64;

// Workspaces larger than this are refused (ADA_EUNSUPPORTED), so no size
// computed here can wrap around.
constexpr size_t kMaxWorkspace = size_t(1) << 48;

// a * b, saturating at SIZE_MAX
inline size_t smul(size_t a, size_t b) {
    size_t r;
    return __builtin_mul_overflow(a, b, &r) ? SIZE_MAX : r;
}
inline size_t smul(size_t a, size_t b, size_t c) { return smul(smul(a, b), c); }
inline size_t smul(size_t a, size_t b, size_t c, size_t d) { return smul(smul(a, b, c), d); }

// carve typed arrays out of a workspace; once the running size passes
// kMaxWorkspace it sticks at SIZE_MAX and the pointers are null
struct Carver {
    char *base;
    size_t off = 0;
    explicit Carver(void *p) : base(static_cast<char *>(p)) {}
    template <typename T>
    T *take(size_t n) {
        const size_t bytes = smul(n, sizeof(T));
        if (off > kMaxWorkspace || bytes > kMaxWorkspace - off) {
            off = SIZE_MAX;
            return nullptr;
        }
        T *p = reinterpret_cast<T *>(base ? base + off : nullptr);
        off = align_up(off + bytes);
        return p;
    }
};

// a + b for workspace sizes, saturating like the carver
inline size_t ws_add(size_t a, size_t b) { return (a > kMaxWorkspace || b > kMaxWorkspace) ? SIZE_MAX : a + b; }

// report a workspace size, or refuse one past kMaxWorkspace
inline ada_status_t ws_out(size_t n, size_t *bytes) {
    if (n > kMaxWorkspace) return ADA_EUNSUPPORTED;
    *bytes = n;
    return ADA_OK;
}

ada_status_t check_cfg(const ada_config_t *cfg) {
    if (!cfg) return ADA_EINVAL;
    if (cfg->num_q_heads <= 0 || cfg->num_kv_heads <= 0 || cfg->num_q_heads % cfg->num_kv_heads != 0)
        return ADA_EINVAL;
    if (cfg->head_dim != kD) return ADA_EUNSUPPORTED;
    if (cfg->page_size != 16 && cfg->page_size != 32) return ADA_EUNSUPPORTED;
    const int G = cfg->num_q_heads / cfg->num_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8) return ADA_EUNSUPPORTED;
    if (cfg->decode_chunk_pages < 0) return ADA_EINVAL;
    if (cfg->rdr_tier_mask >> kNumTiers) return ADA_EINVAL;
    if (cfg->pair_layout != ADA_PAIRS_ADJACENT && cfg->pair_layout != ADA_PAIRS_HALF_SPLIT) return ADA_EINVAL;
    if (cfg->value_tiers != 0 && cfg->value_tiers != 1) return ADA_EINVAL;
    if (!cfg->value_tiers && (cfg->rdr_tier_mask >> 3)) return ADA_EINVAL;   // V8 tiers need value_tiers
    return ADA_OK;
}

// Batch and row shapes the kernels index with 32-bit integers: query-head
// rows B * Hq and token positions max_pages_per_head * P.
ada_status_t check_dims(const ada_config_t *cfg, int64_t B, int64_t maxp) {
    if ((int64_t)B * cfg->num_q_heads > INT32_MAX || maxp * cfg->page_size > INT32_MAX) return ADA_EUNSUPPORTED;
    return ADA_OK;
}

ada_status_t check_cache(const ada_config_t *cfg, const ada_cache_t *c) {
    if (!c) return ADA_EINVAL;
    if (c->num_seqs <= 0 || c->max_pages_per_head <= 0 || c->page_capacity <= 0 || c->arena_capacity16 <= 0)
        return ADA_EINVAL;
    if (c->page_capacity > INT32_MAX || c->arena_capacity16 > (int64_t)UINT32_MAX) return ADA_EUNSUPPORTED;
    if (check_dims(cfg, c->num_seqs, c->max_pages_per_head)) return ADA_EUNSUPPORTED;
    if (!c->page_table || !c->num_pages || !c->open_page || !c->page_meta || !c->code_arena || !c->alloc ||
        !c->status)
        return ADA_EINVAL;
    if (((uintptr_t)c->code_arena & 15) || ((uintptr_t)c->page_meta & 7))
        return ADA_EINVAL;
    return ADA_OK;
}

inline ada_status_t hip_status(hipError_t e) { return e == hipSuccess ? ADA_OK : ADA_EHIP; }

// Split-K chunk length in pages.  Automatic choice: about one round of
// resident work-groups over the whole cache (B * Hkv rows of up to maxp
// pages), so no partial last round idles compute units and each work-group
// builds its LUTs once for as much work as possible.
int decode_chunk_pages(const ada_config_t *cfg, int32_t B, int32_t maxp, int gv) {
    const int tpg = 64 / cfg->page_size;
    int cp = cfg->decode_chunk_pages;
    if (cp <= 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;   // MI355X
        // work-groups resident at once, per slice of the virtual heads
        const size_t slots = std::max<size_t>(1, (size_t)cus * decode_waves_per_simd(slice_heads(gv)) / slices(gv));
        const size_t units = smul((size_t)B, (size_t)cfg->num_kv_heads, (size_t)maxp);
        cp = (int)std::min<size_t>(units / slots + (units % slots != 0), 1 << 20);
    }
    cp = std::min(cp, kMaxChunkPages);
    cp = (cp + tpg - 1) / tpg * tpg;
    if (cp < tpg) cp = tpg;
    if (cp > kMaxChunkPages) cp = kMaxChunkPages;   // page list of a work-group lives in LDS
    return cp;
}

struct DecodeWs {
    float *pm, *pl, *pacc;
    size_t bytes;
    int S, cp;
};

// Q queries per sequence; partial rows are (sequence, query, query head)
DecodeWs decode_layout(const ada_config_t *cfg, int32_t B, int32_t Q, int32_t maxp, void *ws) {
    DecodeWs d;
    d.cp = decode_chunk_pages(cfg, B, maxp, Q * (cfg->num_q_heads / cfg->num_kv_heads));
    d.S = (int)(((int64_t)maxp + d.cp - 1) / d.cp);
    const size_t rows = smul((size_t)B, (size_t)Q, (size_t)cfg->num_q_heads, (size_t)d.S);
    Carver c(ws);
    d.pm = c.take<float>(rows);
    d.pl = c.take<float>(rows);
    d.pacc = c.take<float>(smul(rows, kD));
    d.bytes = c.off;
    return d;
}

DecodeLaunch make_decode(const ada_config_t *cfg, const ada_cache_t *cache, const float *q, int32_t B, int32_t Q,
                         float scale, float *out, float *lse, const DecodeWs &w) {
    DecodeLaunch a;
    a.Q = Q;
    a.page_table = cache->page_table;
    a.num_pages = cache->num_pages;
    a.page_meta = cache->page_meta;
    a.arena = cache->code_arena;
    a.q = q;
    a.pm = w.pm;
    a.pl = w.pl;
    a.pacc = w.pacc;
    a.out = out;
    a.lse = lse;
    a.B = B;
    a.Hq = cfg->num_q_heads;
    a.Hkv = cfg->num_kv_heads;
    a.P = cfg->page_size;
    a.maxp = cache->max_pages_per_head;
    a.chunk_pages = w.cp;
    a.S = w.S;
    a.scale = scale;
    a.app_page = nullptr;
    a.app_slot = nullptr;
    a.app_keys = nullptr;
    a.app_values = nullptr;
    a.arena_w = nullptr;
    a.status = cache->status;
    a.logit_buf = nullptr;
    a.util = nullptr;
    a.half_pairs = cfg->pair_layout == ADA_PAIRS_HALF_SPLIT;
    a.value_tiers = cfg->value_tiers;
    a.nslice = slices(Q * (cfg->num_q_heads / cfg->num_kv_heads));
    // the cache's row order covers all its rows: usable when all are decoded
    a.row_order = B == cache->num_seqs ? cache->row_order : nullptr;
    return a;
}

struct AppendWs {
    int32_t *key_cnt, *key_c0, *key_done, *key_page_and_off;
    int64_t *totals;
    int32_t *dest_page, *dest_slot, *new_pages, *n_new;
    size_t bytes;
};

AppendWs append_layout(const ada_config_t *cfg, const ada_cache_t *cache, int32_t n, void *ws) {
    AppendWs w;
    const size_t nkeys = smul((size_t)cache->num_seqs, (size_t)cfg->num_kv_heads, kNumTiers);
    Carver c(ws);
    w.key_cnt = c.take<int32_t>(nkeys);
    w.key_c0 = c.take<int32_t>(nkeys);
    w.key_done = c.take<int32_t>(nkeys);
    w.key_page_and_off = c.take<int32_t>(smul(2, nkeys));
    w.totals = c.take<int64_t>(2);
    w.dest_page = c.take<int32_t>(n > 0 ? n : 1);
    w.dest_slot = c.take<int32_t>(n > 0 ? n : 1);
    w.new_pages = c.take<int32_t>(n > 0 ? n : 1);
    w.n_new = c.take<int32_t>(2);
    w.bytes = c.off;
    return w;
}

AppendLaunch make_append(const ada_config_t *cfg, const ada_cache_t *cache, int32_t n, const int32_t *seq,
                         const int32_t *kv_head, const uint8_t *tier, const float *keys, const uint16_t *values,
                         const AppendWs &w) {
    AppendLaunch a;
    a.n = n;
    a.Hkv = cfg->num_kv_heads;
    a.P = cfg->page_size;
    a.num_seqs = cache->num_seqs;
    a.maxp = cache->max_pages_per_head;
    a.page_capacity = cache->page_capacity;
    a.arena_capacity16 = cache->arena_capacity16;
    a.seq = seq;
    a.head = kv_head;
    a.tier = tier;
    a.keys = keys;
    a.values = values;
    a.page_table = cache->page_table;
    a.num_pages = cache->num_pages;
    a.open_page = cache->open_page;
    a.page_meta = cache->page_meta;
    a.arena = cache->code_arena;
    a.alloc = cache->alloc;
    a.status = cache->status;
    a.key_cnt = w.key_cnt;
    a.key_c0 = w.key_c0;
    a.key_done = w.key_done;
    a.key_page = w.key_page_and_off;
    a.totals = w.totals;
    a.dest_page = w.dest_page;
    a.dest_slot = w.dest_slot;
    a.new_pages = w.new_pages;
    a.n_new = w.n_new;
    a.half_pairs = cfg->pair_layout == ADA_PAIRS_HALF_SPLIT;
    a.n_tiers = cfg->value_tiers ? kNumTiers : 3;
    return a;
}

struct PackWs {
    int32_t *tile_counts, *row_counts, *row_base, *dest_page, *dest_slot, *range, *ctx;
    int64_t *row_unit, *item_of_slot;
    int64_t item_slot_pages;
    int n_tiles;
    size_t bytes;
};

PackWs pack_layout(const ada_config_t *cfg, int32_t B, int64_t stride, void *ws) {
    PackWs w;
    const size_t rows = smul((size_t)B, (size_t)cfg->num_kv_heads);
    const int64_t tiles = stride / 1024 + (stride % 1024 != 0);
    w.n_tiles = (int)std::min<int64_t>(tiles, INT32_MAX);
    Carver c(ws);
    w.tile_counts = c.take<int32_t>(smul(rows, (size_t)tiles, kNumTiers));
    w.row_counts = c.take<int32_t>(smul(rows, kNumTiers));
    w.row_base = c.take<int32_t>(smul(rows, kNumTiers));
    w.row_unit = c.take<int64_t>(smul(rows, kNumTiers));
    w.dest_page = c.take<int32_t>(smul(rows, (size_t)stride));
    w.dest_slot = c.take<int32_t>(smul(rows, (size_t)stride));
    w.range = c.take<int32_t>(2);
    w.ctx = c.take<int32_t>(B);
    // new pages of a pack: at most ceil(stride / P) per row, plus one
    // partial page per tier
    const size_t pages = smul(rows, (size_t)(stride / cfg->page_size + 1 + kNumTiers));
    w.item_slot_pages = (int64_t)std::min<size_t>(pages, INT64_MAX);
    w.item_of_slot = c.take<int64_t>(smul(pages, (size_t)cfg->page_size));
    w.bytes = c.off;
    return w;
}

struct RdrWs {
    unsigned long long *hist, *prefix;
    long long *above;
    int32_t *all_fit, *ctx;
    int64_t *budget;
    uint8_t *tie_sel;
    long long *tie_tile;
    size_t bytes;
};

RdrWs rdr_layout(const ada_config_t *cfg, int32_t B, int64_t stride, void *ws) {
    RdrWs w;
    Carver c(ws);
    w.hist = c.take<unsigned long long>(smul((size_t)B, 256 * kRdrPasses));
    w.prefix = c.take<unsigned long long>(smul((size_t)B, kRdrPasses + 1));
    w.above = c.take<long long>(smul((size_t)B, kRdrPasses + 1));
    w.all_fit = c.take<int32_t>(smul((size_t)B, kRdrPasses + 1));
    w.ctx = c.take<int32_t>(B);
    w.budget = c.take<int64_t>(B);
    const size_t row_items = smul((size_t)cfg->num_kv_heads, (size_t)stride);
    w.tie_sel = c.take<uint8_t>(smul((size_t)B, row_items));
    w.tie_tile = c.take<long long>(smul((size_t)B, row_items / kRdrTieTile + (row_items % kRdrTieTile != 0)));
    w.bytes = c.off;
    return w;
}

// RDR upgrade steps of the enabled tiers (rate order); EUNSUPPORTED when the
// savings per byte do not strictly decrease.  Distortion of a tier:
// 2^-(tb + sb), plus 2^-14 for V8 values.
ada_status_t rdr_steps(uint32_t mask, int *n_steps, int32_t *step_tier, int64_t *dR, double *c) {
    int ids[kNumTiers], n = 0;
    for (int t = 0; t < kNumTiers; ++t)
        if (mask & (1u << t)) ids[n++] = t;
    auto rate = [](int t) { return tier_rate(t); };
    for (int i = 1; i < n; ++i)   // insertion sort by rate
        for (int j = i; j > 0 && rate(ids[j]) < rate(ids[j - 1]); --j) {
            const int tmp = ids[j];
            ids[j] = ids[j - 1];
            ids[j - 1] = tmp;
        }
    int64_t prevR = 0;
    double prevD = 1.0;
    for (int i = 0; i < n; ++i) {
        const int t = ids[i];
        const int64_t R = rate(t);
        const double D = ldexp(1.0, -(tier_tb(t) + tier_sb(t))) + (tier_v8(t) ? ldexp(1.0, -14) : 0.0);
        if (R <= prevR || D >= prevD) return ADA_EUNSUPPORTED;
        dR[i] = R - prevR;
        c[i] = (prevD - D) / (double)dR[i];
        if (i > 0 && !(c[i] < c[i - 1])) return ADA_EUNSUPPORTED;
        step_tier[i] = t;
        prevR = R;
        prevD = D;
    }
    *n_steps = n;
    return n ? ADA_OK : ADA_EINVAL;
}

}  // namespace

// ---- decode without a caller workspace ----------------------------------
// The split-K partials of ada_decode_noalloc live in this file-scope device
// array (one copy per GPU, held until the process ends).  Host code never
// passes the array's name to a kernel: its device address is looked up once
// per device with hipGetSymbolAddress and kept in noalloc_ptr[].
constexpr size_t kNoallocScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

static std::mutex noalloc_mu;
static void *noalloc_ptr[kMaxDevices];

// the current device's address of `scratch`, or nullptr if it cannot be had
static void *noalloc_scratch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(noalloc_mu);
    if (!noalloc_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        noalloc_ptr[dev] = p;
    }
    return noalloc_ptr[dev];
}

extern "C" {

const char *ada_status_str(ada_status_t s) {
    // a C caller may pass any int; read its bits without an enum load
    static_assert(sizeof(ada_status_t) == sizeof(int32_t), "status is an int");
    int32_t v;
    memcpy(&v, &s, sizeof(v));
    switch (v) {
        case ADA_OK: return "ADA_OK";
        case ADA_EINVAL: return "ADA_EINVAL: invalid argument or input";
        case ADA_ENOSPC: return "ADA_ENOSPC: cache capacity exceeded";
        case ADA_EUNSUPPORTED: return "ADA_EUNSUPPORTED: unsupported shape";
        case ADA_EHIP: return "ADA_EHIP: HIP runtime error";
        case ADA_EINTERNAL: return "ADA_EINTERNAL: undecidable code";
        default: return "ADA_UNKNOWN";
    }
}

int64_t ada_block_bytes(int32_t tier, int32_t page_size) {
    if (tier < 0 || tier >= kNumTiers || (page_size != 16 && page_size != 32)) return -1;
    return (int64_t)block16(tier, page_size) * 16;
}

size_t ada_lut_floats(const ada_config_t *cfg) {
    (void)cfg;
    return 64 * (256 + 16 + 4);
}

ada_status_t ada_cache_init(const ada_config_t *cfg, const ada_cache_t *cache, void *stream) {
    ada_status_t st = check_cfg(cfg);
    if (st) return st;
    if ((st = check_cache(cfg, cache))) return st;
    return hip_status(launch_cache_init(cache->num_seqs * cfg->num_kv_heads, cache->num_pages, cache->open_page,
                                        cache->alloc, cache->status, cache->row_order, (hipStream_t)stream));
}

ada_status_t ada_validate_cache(const ada_config_t *cfg, const ada_cache_t *cache, int32_t B, void *stream) {
    ada_status_t st = check_cfg(cfg);
    if (st) return st;
    if ((st = check_cache(cfg, cache))) return st;
    if (B < 0 || B > cache->num_seqs) return ADA_EINVAL;
    if (B == 0) return ADA_OK;
    return hip_status(launch_validate(B * cfg->num_kv_heads, cache->max_pages_per_head, cache->page_capacity,
                                      cache->arena_capacity16, cfg->page_size, cfg->value_tiers ? kNumTiers : 3,
                                      cache->num_pages, cache->page_table, cache->page_meta, cache->row_order,
                                      cache->num_seqs * cfg->num_kv_heads, cache->status, (hipStream_t)stream));
}

ada_status_t ada_build_lut(const ada_config_t *cfg, const float *q, int32_t B, float *lut, void *stream) {
    ada_status_t st = check_cfg(cfg);
    if (st) return st;
    if (B < 0 || (B > 0 && (!q || !lut))) return ADA_EINVAL;
    if ((st = check_dims(cfg, B, 0))) return st;
    if (B == 0) return ADA_OK;
    return hip_status(launch_build_lut(q, B * cfg->num_q_heads, lut, cfg->pair_layout == ADA_PAIRS_HALF_SPLIT,
                                       (hipStream_t)stream));
}

// queries per sequence: a power of two with Q * (Hq / Hkv) <= 8
static ada_status_t check_queries(const ada_config_t *cfg, int32_t Q) {
    if (Q < 1) return ADA_EINVAL;
    const int gv = Q * (cfg->num_q_heads / cfg->num_kv_heads);
    if ((Q & (Q - 1)) || gv > kMaxVirtualHeads) return ADA_EUNSUPPORTED;
    return ADA_OK;
}

ada_status_t ada_decode_multi_workspace(const ada_config_t *cfg, const ada_cache_t *cache, int32_t B, int32_t Q,
                                        size_t *bytes) {
    ada_status_t st = check_cfg(cfg);
    if (st) return st;
    if ((st = check_queries(cfg, Q))) return st;
    if (!cache || !bytes || B < 0 || cache->max_pages_per_head <= 0) return ADA_EINVAL;
    if ((st = check_dims(cfg, B, cache->max_pages_per_head))) return st;
    return ws_out(decode_layout(cfg, B, Q, cache->max_pages_per_head, nullptr).bytes, bytes);
}

ada_status_t ada_decode_workspace(const ada_config_t *cfg, const ada_cache_t *cache, int32_t B, size_t *bytes) {
    return ada_decode_multi_workspace(cfg, cache, B, 1, bytes);
}

static ada_status_t decode_common(const ada_config_t *cfg, const ada_cache_t *cache, int32_t B, int32_t Q, void *ws,
                                  size_t ws_bytes, DecodeWs *w) {
    ada_status_t st = check_cfg(cfg);
    if (st) return st;
    if ((st = check_queries(cfg, Q))) return st;
    if ((st = check_cache(cfg, cache))) return st;
    if (B < 0 || B > cache->num_seqs) return ADA_EINVAL;
    *w = decode_layout(cfg, B, Q, cache->max_pages_per_head, ws);
    if (w->bytes > kMaxWorkspace) return ADA_EUNSUPPORTED;
    if (B > 0 && (!ws || ws_bytes < w->bytes)) return ADA_EINVAL;
    return ADA_OK;
}

ada_status_t ada_decode_partials(const ada_config_t *cfg, const ada_cache_t *cache, const float *q, int32_t B,
                                 float scale, void *ws, size_t ws_bytes, void *stream) {
    DecodeWs w;
    ada_status_t st = decode_common(cfg, cache, B, 1, ws, ws_bytes, &w);
    if (st) return st;
    if (B == 0) return ADA_OK;
    if (!q) return ADA_EINVAL;
    DecodeLaunch a = make_decode(cfg, cache, q, B, 1, scale, nullptr, nullptr, w);
    return hip_status(launch_decode_partials(a, (hipStream_t)stream));
}

ada_status_t ada_decode_reduce(const ada_config_t *cfg, const ada_cache_t *cache, int32_t B, float *out, float *lse,
                               void *ws, size_t ws_bytes, void *stream) {
    DecodeWs w;
    ada_status_t st = decode_common(cfg, cache, B, 1, ws, ws_bytes, &w);
    if (st) return st;
    if (B == 0) return ADA_OK;
    if (!out) return ADA_EINVAL;
    DecodeLaunch a = make_decode(cfg, cache, nullptr, B, 1, 0.f, out, lse, w);
    return hip_status(launch_decode_reduce(a, (hipStream_t)stream));
}

ada_status_t ada_decode_multi(const ada_config_t *cfg, const ada_cache_t *cache, const float *q, int32_t B,
                              int32_t Q, float scale, float *out, float *lse, void *ws, size_t ws_bytes, void *stream) {
    DecodeWs w;
    ada_status_t st = decode_common(cfg, cache, B, Q, ws, ws_bytes, &w);
    if (st) return st;
    if (B == 0) return ADA_OK;
    if (!q || !out) return ADA_EINVAL;
    DecodeLaunch a = make_decode(cfg, cache, q, B, Q, scale, out, lse, w);
    hipError_t e = launch_decode_partials(a, (hipStream_t)stream);
    if (e != hipSuccess) return ADA_EHIP;
    return hip_status(launch_decode_reduce(a, (hipStream_t)stream));
}

ada_status_t ada_decode(const ada_config_t *cfg, const ada_cache_t *cache, const float *q, int32_t B, float scale,
                        float *out, float *lse, void *ws, size_t ws_bytes, void *stream) {
    return ada_decode_multi(cfg, cache, q, B, 1, scale, out, lse, ws, ws_bytes, stream);
}

ada_status_t ada_decode_noalloc(const ada_config_t *cfg, const ada_cache_t *cache, const float *q, int32_t B,
                                float scale, float *out, float *lse, void *stream) {
    ada_status_t st = check_cfg(cfg);
    if (st) return st;
    if ((st = check_cache(cfg, cache))) return st;
    if (B < 0 || B > cache->num_seqs) return ADA_EINVAL;
    if (B == 0) return ADA_OK;
    if (!q || !out) return ADA_EINVAL;
    // sizes first (no device memory touched): the partials must fit the array
    if (decode_layout(cfg, B, 1, cache->max_pages_per_head, nullptr).bytes > kNoallocScratchBytes)
        return ADA_EUNSUPPORTED;
    void *ws = noalloc_scratch();
    if (!ws) return ADA_EHIP;
    // every partial the reduction reads is written by the split-K pass of the
    // same call, so nothing in the array needs clearing first
    const DecodeWs w = decode_layout(cfg, B, 1, cache->max_pages_per_head, ws);
    DecodeLaunch a = make_decode(cfg, cache, q, B, 1, scale, out, lse, w);
    hipError_t e = launch_decode_partials(a, (hipStream_t)stream);
    if (e != hipSuccess) return ADA_EHIP;
    return hip_status(launch_decode_reduce(a, (hipStream_t)stream));
}

ada_status_t ada_append_workspace(const ada_config_t *cfg, const ada_cache_t *cache, int32_t n, size_t *bytes) {
    ada_status_t st = check_cfg(cfg);
    if (st) return st;
    if (!cache || !bytes || n < 0 || cache->num_seqs <= 0) return ADA_EINVAL;
    return ws_out(append_layout(cfg, cache, n, nullptr).bytes, bytes);
}

ada_status_t ada_encode_append(const ada_config_t *cfg, const ada_cache_t *cache, int32_t n, const int32_t *seq,
                               const int32_t *kv_head, const uint8_t *tier, const float *keys, const uint16_t *values,
                               void *ws, size_t ws_bytes, void *stream) {
    ada_status_t st = check_cfg(cfg);
    if (st) return st;
    if ((st = check_cache(cfg, cache))) return st;
    if (n < 0) return ADA_EINVAL;
    if (n == 0) return ADA_OK;
    if (!seq || !kv_head || !tier || !keys || !values) return ADA_EINVAL;
    AppendWs w = append_layout(cfg, cache, n, ws);
    if (w.bytes > kMaxWorkspace) return ADA_EUNSUPPORTED;
    if (!ws || ws_bytes < w.bytes) return ADA_EINVAL;
    AppendLaunch a = make_append(cfg, cache, n, seq, kv_head, tier, keys, values, w);
    return hip_status(launch_append(a, true, (hipStream_t)stream));
}

// Fused append + decode: workspace = decode partials, then the append's
// booking arrays for B * Hkv requests.
static size_t decode_append_layout(const ada_config_t *cfg, const ada_cache_t *cache, int32_t B, void *ws,
                                   DecodeWs *dw, AppendWs *aw) {
    *dw = decode_layout(cfg, B, 1, cache->max_pages_per_head, ws);
    char *ab = ws ? static_cast<char *>(ws) + dw->bytes : nullptr;
    *aw = append_layout(cfg, cache, (int32_t)std::min<int64_t>((int64_t)B * cfg->num_kv_heads, INT32_MAX), ab);
    return ws_add(dw->bytes, aw->bytes);
}

ada_status_t ada_decode_append_workspace(const ada_config_t *cfg, const ada_cache_t *cache, int32_t B,
                                         size_t *bytes) {
    ada_status_t st = check_cfg(cfg);
    if (st) return st;
    if (!cache || !bytes || B < 0 || cache->max_pages_per_head <= 0 || cache->num_seqs <= 0) return ADA_EINVAL;
    if ((st = check_dims(cfg, B, cache->max_pages_per_head))) return st;
    DecodeWs dw;
    AppendWs aw;
    return ws_out(decode_append_layout(cfg, cache, B, nullptr, &dw, &aw), bytes);
}

ada_status_t ada_decode_append(const ada_config_t *cfg, const ada_cache_t *cache, const float *q, int32_t B,
                               float scale, const float *new_keys, const uint16_t *new_values,
                               const uint8_t *new_tier, float *out, float *lse, void *ws, size_t ws_bytes,
                               void *stream) {
    ada_status_t st = check_cfg(cfg);
    if (st) return st;
    if ((st = check_cache(cfg, cache))) return st;
    if (B < 0 || B > cache->num_seqs) return ADA_EINVAL;
    if (B == 0) return ADA_OK;
    if (!q || !out || !new_keys || !new_values || !new_tier || !ws) return ADA_EINVAL;
    DecodeWs dw;
    AppendWs aw;
    const size_t need = decode_append_layout(cfg, cache, B, ws, &dw, &aw);
    if (need > kMaxWorkspace) return ADA_EUNSUPPORTED;
    if (ws_bytes < need) return ADA_EINVAL;
    const int32_t n = B * cfg->num_kv_heads;
    // 1. book one request per row (row order) and update the metadata
    AppendLaunch ap = make_append(cfg, cache, n, nullptr, nullptr, new_tier, new_keys, new_values, aw);
    hipError_t e = launch_append_rows(ap, (hipStream_t)stream);
    if (e != hipSuccess) return ADA_EHIP;
    // 2. split-K pass; the owner of each booked slot encodes and writes it first
    DecodeLaunch a = make_decode(cfg, cache, q, B, 1, scale, out, lse, dw);
    a.app_page = aw.dest_page;
    a.app_slot = aw.dest_slot;
    a.app_keys = new_keys;
    a.app_values = new_values;
    a.arena_w = cache->code_arena;
    if ((e = launch_decode_partials(a, (hipStream_t)stream)) != hipSuccess) return ADA_EHIP;
    // 3. reduction over the chunks
    return hip_status(launch_decode_reduce(a, (hipStream_t)stream));
}

// Utility emission: workspace = decode partials, then the logit buffer
// [page_capacity * P][G], then an lse buffer [B][Hq] (used when lse is NULL).
// The split-K pass addresses the logit buffer with 32-bit offsets.
static ada_status_t check_logit_buf(const ada_config_t *cfg, const ada_cache_t *cache) {
    const int64_t G = cfg->num_q_heads / cfg->num_kv_heads;
    return cache->page_capacity > (int64_t)UINT32_MAX / (cfg->page_size * G) ? ADA_EUNSUPPORTED : ADA_OK;
}

static size_t decode_utility_layout(const ada_config_t *cfg, const ada_cache_t *cache, int32_t B, void *ws,
                                    DecodeWs *dw, float **logit_buf, float **lse_buf) {
    *dw = decode_layout(cfg, B, 1, cache->max_pages_per_head, ws);
    Carver c(ws ? static_cast<char *>(ws) + dw->bytes : nullptr);
    const int G = cfg->num_q_heads / cfg->num_kv_heads;
    *logit_buf = c.take<float>(smul((size_t)cache->page_capacity, (size_t)cfg->page_size, (size_t)G));
    *lse_buf = c.take<float>(smul((size_t)B, (size_t)cfg->num_q_heads));
    return ws_add(dw->bytes, c.off);
}

ada_status_t ada_decode_utility_workspace(const ada_config_t *cfg, const ada_cache_t *cache, int32_t B,
                                          size_t *bytes) {
    ada_status_t st = check_cfg(cfg);
    if (st) return st;
    if (!cache || !bytes || B < 0 || cache->max_pages_per_head <= 0 || cache->page_capacity <= 0) return ADA_EINVAL;
    if ((st = check_dims(cfg, B, cache->max_pages_per_head)) || (st = check_logit_buf(cfg, cache))) return st;
    DecodeWs dw;
    float *lb, *sb;
    return ws_out(decode_utility_layout(cfg, cache, B, nullptr, &dw, &lb, &sb), bytes);
}

ada_status_t ada_decode_utility(const ada_config_t *cfg, const ada_cache_t *cache, const float *q, int32_t B,
                                float scale, float *out, float *lse, float *util, void *ws, size_t ws_bytes,
                                void *stream) {
    ada_status_t st = check_cfg(cfg);
    if (st) return st;
    if ((st = check_cache(cfg, cache))) return st;
    if ((st = check_logit_buf(cfg, cache))) return st;
    if (B < 0 || B > cache->num_seqs) return ADA_EINVAL;
    if (B == 0) return ADA_OK;
    if (!q || !out || !util || !ws) return ADA_EINVAL;
    DecodeWs dw;
    float *logit_buf, *lse_buf;
    const size_t need = decode_utility_layout(cfg, cache, B, ws, &dw, &logit_buf, &lse_buf);
    if (need > kMaxWorkspace) return ADA_EUNSUPPORTED;
    if (ws_bytes < need) return ADA_EINVAL;
    DecodeLaunch a = make_decode(cfg, cache, q, B, 1, scale, out, lse ? lse : lse_buf, dw);
    a.logit_buf = logit_buf;
    a.util = util;
    hipError_t e = launch_decode_partials(a, (hipStream_t)stream);
    if (e == hipSuccess) e = launch_decode_reduce(a, (hipStream_t)stream);
    if (e == hipSuccess) e = launch_decode_utility(a, (hipStream_t)stream);
    return hip_status(e);
}

ada_status_t ada_rdr_workspace(const ada_config_t *cfg, int32_t B, int64_t ctx_stride, size_t *bytes) {
    ada_status_t st = check_cfg(cfg);
    if (st) return st;
    if (!bytes || B < 0 || ctx_stride < 0) return ADA_EINVAL;
    return ws_out(rdr_layout(cfg, B, ctx_stride, nullptr).bytes, bytes);
}

ada_status_t ada_rdr_assign(const ada_config_t *cfg, int32_t B, const int32_t *ctx_len, int64_t ctx_stride,
                            const float *utility, const int64_t *budget, int8_t *tier_out, int32_t *status, void *ws,
                            size_t ws_bytes, void *stream) {
    ada_status_t st = check_cfg(cfg);
    if (st) return st;
    if (B < 0 || ctx_stride <= 0) return ADA_EINVAL;
    if (B == 0) return ADA_OK;
    if (!ctx_len || !utility || !budget || !tier_out || !status) return ADA_EINVAL;
    if (ctx_stride > INT32_MAX / cfg->num_kv_heads) return ADA_EUNSUPPORTED;
    for (int b = 0; b < B; ++b)
        if (ctx_len[b] < 0 || ctx_len[b] > ctx_stride || budget[b] < 0) return ADA_EINVAL;
    RdrLaunch a;
    const uint32_t mask = cfg->rdr_tier_mask ? cfg->rdr_tier_mask : 7u;
    if ((st = rdr_steps(mask, &a.n_steps, a.step_tier, a.dR, a.c))) return st;
    if ((int64_t)B * cfg->num_kv_heads > INT32_MAX) return ADA_EUNSUPPORTED;
    RdrWs w = rdr_layout(cfg, B, ctx_stride, ws);
    if (w.bytes > kMaxWorkspace) return ADA_EUNSUPPORTED;
    if (!ws || ws_bytes < w.bytes) return ADA_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    if (hipMemcpyAsync(w.ctx, ctx_len, sizeof(int32_t) * B, hipMemcpyHostToDevice, s) != hipSuccess) return ADA_EHIP;
    if (hipMemcpyAsync(w.budget, budget, sizeof(int64_t) * B, hipMemcpyHostToDevice, s) != hipSuccess)
        return ADA_EHIP;
    a.B = B;
    a.Hkv = cfg->num_kv_heads;
    a.stride = ctx_stride;
    a.ctx_len_dev = w.ctx;
    a.budget_dev = w.budget;
    a.utility = utility;
    a.tier_out = tier_out;
    a.status = status;
    a.hist = w.hist;
    a.prefix = w.prefix;
    a.above = w.above;
    a.all_fit = w.all_fit;
    a.tie_sel = w.tie_sel;
    a.tie_tile = w.tie_tile;
    a.cap = nullptr;
    return hip_status(launch_rdr(a, s));
}

ada_status_t ada_pack_workspace(const ada_config_t *cfg, const ada_cache_t *cache, int32_t B, int64_t ctx_stride,
                                size_t *bytes) {
    ada_status_t st = check_cfg(cfg);
    if (st) return st;
    if (!cache || !bytes || B < 0 || ctx_stride < 0) return ADA_EINVAL;
    return ws_out(pack_layout(cfg, B, ctx_stride, nullptr).bytes, bytes);
}

ada_status_t ada_pack(const ada_config_t *cfg, const ada_cache_t *cache, int32_t B, const int32_t *ctx_len,
                      int64_t ctx_stride, const int8_t *tier, const float *keys, const uint16_t *values, void *ws,
                      size_t ws_bytes, void *stream) {
    ada_status_t st = check_cfg(cfg);
    if (st) return st;
    if ((st = check_cache(cfg, cache))) return st;
    if (B < 0 || B > cache->num_seqs || ctx_stride <= 0) return ADA_EINVAL;
    if (B == 0) return ADA_OK;
    if (!ctx_len || !tier || !keys || !values) return ADA_EINVAL;
    if (ctx_stride > INT32_MAX) return ADA_EUNSUPPORTED;
    for (int b = 0; b < B; ++b)
        if (ctx_len[b] < 0 || ctx_len[b] > ctx_stride) return ADA_EINVAL;
    PackWs w = pack_layout(cfg, B, ctx_stride, ws);
    if (w.bytes > kMaxWorkspace) return ADA_EUNSUPPORTED;
    if (!ws || ws_bytes < w.bytes) return ADA_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    if (hipMemcpyAsync(w.ctx, ctx_len, sizeof(int32_t) * B, hipMemcpyHostToDevice, s) != hipSuccess) return ADA_EHIP;
    PackLaunch a;
    a.B = B;
    a.Hkv = cfg->num_kv_heads;
    a.P = cfg->page_size;
    a.maxp = cache->max_pages_per_head;
    a.stride = ctx_stride;
    a.page_capacity = cache->page_capacity;
    a.arena_capacity16 = cache->arena_capacity16;
    a.ctx_len_dev = w.ctx;
    a.tier = tier;
    a.keys = keys;
    a.values = values;
    a.page_table = cache->page_table;
    a.num_pages = cache->num_pages;
    a.open_page = cache->open_page;
    a.page_meta = cache->page_meta;
    a.arena = cache->code_arena;
    a.alloc = cache->alloc;
    a.status = cache->status;
    a.tile_counts = w.tile_counts;
    a.row_counts = w.row_counts;
    a.row_base = w.row_base;
    a.row_unit = w.row_unit;
    a.dest_page = w.dest_page;
    a.dest_slot = w.dest_slot;
    a.new_pages = nullptr;
    a.n_new = w.range;
    a.n_tiles = w.n_tiles;
    a.src_page_table = nullptr;
    a.src_page_meta = nullptr;
    a.src_arena = nullptr;
    a.src_maxp = 0;
    a.src_of_slot = nullptr;
    a.src_of_slot_pages = 0;
    a.first_pos = nullptr;
    a.page_order = nullptr;
    a.item_of_slot = w.item_of_slot;
    a.item_slot_pages = w.item_slot_pages;
    a.row_order = cache->row_order;
    a.rows_total = cache->num_seqs * cfg->num_kv_heads;
    a.half_pairs = cfg->pair_layout == ADA_PAIRS_HALF_SPLIT;
    a.n_tiers = cfg->value_tiers ? kNumTiers : 3;
    return hip_status(launch_pack(a, s));
}

// Re-pack workspace: the virtual item arrays (utility, step cap, tier map)
// over B * Hkv rows of S = max_pages_per_head(src) * P positions, then the
// RDR and pack workspaces for that stride.
struct RepackWs {
    float *util_v;
    int8_t *cap_v, *tier_v;
    void *rdr, *pack;
    int4 *src_of_slot;
    int64_t src_of_slot_pages;
    int32_t *first_pos, *page_order;
    size_t bytes;
};

static RepackWs repack_layout(const ada_config_t *cfg, const ada_cache_t *src, int32_t B, void *ws) {
    RepackWs r;
    const int64_t S = (int64_t)src->max_pages_per_head * cfg->page_size;
    const size_t n = smul((size_t)B, (size_t)cfg->num_kv_heads, (size_t)S);
    Carver c(ws);
    r.util_v = c.take<float>(n);
    r.cap_v = c.take<int8_t>(n);
    r.tier_v = c.take<int8_t>(n);
    const size_t rb = rdr_layout(cfg, B, S, nullptr).bytes;
    r.rdr = c.take<char>(rb);
    const size_t pb = pack_layout(cfg, B, S, nullptr).bytes;
    r.pack = c.take<char>(pb);
    const size_t pages =
        smul((size_t)B, (size_t)cfg->num_kv_heads, (size_t)repack_pages_per_row(src->max_pages_per_head));
    r.src_of_slot_pages = (int64_t)std::min<size_t>(pages, INT64_MAX);
    r.src_of_slot = c.take<int4>(smul(pages, (size_t)cfg->page_size));
    r.first_pos = c.take<int32_t>(pages);
    r.page_order = c.take<int32_t>(pages);
    r.bytes = c.off;
    return r;
}

ada_status_t ada_repack_workspace(const ada_config_t *cfg, const ada_cache_t *src, int32_t B, size_t *bytes) {
    ada_status_t st = check_cfg(cfg);
    if (st) return st;
    if (!src || !bytes || B < 0 || src->max_pages_per_head <= 0) return ADA_EINVAL;
    if ((st = check_dims(cfg, B, src->max_pages_per_head))) return st;
    return ws_out(repack_layout(cfg, src, B, nullptr).bytes, bytes);
}

ada_status_t ada_repack(const ada_config_t *cfg, const ada_cache_t *src, int32_t B, const float *util,
                        const int64_t *budget, const ada_cache_t *dst, void *ws, size_t ws_bytes, void *stream) {
    ada_status_t st = check_cfg(cfg);
    if (st) return st;
    if ((st = check_cache(cfg, src)) || (st = check_cache(cfg, dst))) return st;
    if (B < 0 || B > src->num_seqs || B > dst->num_seqs) return ADA_EINVAL;
    if (B == 0) return ADA_OK;
    if (!util || !budget || !ws) return ADA_EINVAL;
    const int P = cfg->page_size;
    const int64_t S = (int64_t)src->max_pages_per_head * P;
    if (S > INT32_MAX / cfg->num_kv_heads) return ADA_EUNSUPPORTED;
    for (int b = 0; b < B; ++b)
        if (budget[b] < 0) return ADA_EINVAL;
    RepackWs r = repack_layout(cfg, src, B, ws);
    if (r.bytes > kMaxWorkspace) return ADA_EUNSUPPORTED;
    if (ws_bytes < r.bytes) return ADA_EINVAL;
    RdrLaunch ra;
    const uint32_t mask = cfg->rdr_tier_mask ? cfg->rdr_tier_mask : 7u;
    if ((st = rdr_steps(mask, &ra.n_steps, ra.step_tier, ra.dR, ra.c))) return st;
    hipStream_t s = (hipStream_t)stream;
    // 1. the source's kept tokens as RDR items with their step caps
    RepackItemsLaunch it;
    it.B = B;
    it.Hkv = cfg->num_kv_heads;
    it.P = P;
    it.src_maxp = src->max_pages_per_head;
    it.page_table = src->page_table;
    it.num_pages = src->num_pages;
    it.page_meta = src->page_meta;
    it.util = util;
    // the codes hold nothing finer than they are: each tier of the chain
    // must hold no fewer angle, magnitude and value bits than the one
    // before, and a token may take the chain's tiers holding no more bits
    // than its own (a prefix of the chain)
    auto within = [](int a, int b) {
        return tier_tb(a) <= tier_tb(b) && tier_sb(a) <= tier_sb(b) && tier_vb(a) <= tier_vb(b);
    };
    for (int k = 1; k < ra.n_steps; ++k)
        if (!within(ra.step_tier[k - 1], ra.step_tier[k])) return ADA_EUNSUPPORTED;
    for (int t = 0; t < kNumTiers; ++t) {
        int lv = 0;
        while (lv < ra.n_steps && within(ra.step_tier[lv], t)) ++lv;
        it.level_of_tier[t] = (int8_t)lv;
    }
    it.util_v = r.util_v;
    it.cap_v = r.cap_v;
    RdrWs rw = rdr_layout(cfg, B, S, r.rdr);
    it.ctx_v = rw.ctx;
    hipError_t e = launch_repack_items(it, s);
    if (e != hipSuccess) return ADA_EHIP;
    // 2. capped RDR over them (status word: the destination's)
    if (hipMemcpyAsync(rw.budget, budget, sizeof(int64_t) * B, hipMemcpyHostToDevice, s) != hipSuccess)
        return ADA_EHIP;
    ra.B = B;
    ra.Hkv = cfg->num_kv_heads;
    ra.stride = S;
    ra.ctx_len_dev = rw.ctx;
    ra.budget_dev = rw.budget;
    ra.utility = r.util_v;
    ra.tier_out = r.tier_v;
    ra.status = dst->status;
    ra.hist = rw.hist;
    ra.prefix = rw.prefix;
    ra.above = rw.above;
    ra.all_fit = rw.all_fit;
    ra.tie_sel = rw.tie_sel;
    ra.tie_tile = rw.tie_tile;
    ra.cap = r.cap_v;
    if ((e = launch_rdr(ra, s)) != hipSuccess) return ADA_EHIP;
    // 3. pack the tier map into dst, transcoding each kept token from src
    PackWs w = pack_layout(cfg, B, S, r.pack);
    if (hipMemcpyAsync(w.ctx, rw.ctx, sizeof(int32_t) * B, hipMemcpyDeviceToDevice, s) != hipSuccess)
        return ADA_EHIP;
    PackLaunch a;
    a.B = B;
    a.Hkv = cfg->num_kv_heads;
    a.P = P;
    a.maxp = dst->max_pages_per_head;
    a.stride = S;
    a.page_capacity = dst->page_capacity;
    a.arena_capacity16 = dst->arena_capacity16;
    a.ctx_len_dev = w.ctx;
    a.tier = r.tier_v;
    a.keys = nullptr;
    a.values = nullptr;
    a.page_table = dst->page_table;
    a.num_pages = dst->num_pages;
    a.open_page = dst->open_page;
    a.page_meta = dst->page_meta;
    a.arena = dst->code_arena;
    a.alloc = dst->alloc;
    a.status = dst->status;
    a.tile_counts = w.tile_counts;
    a.row_counts = w.row_counts;
    a.row_base = w.row_base;
    a.row_unit = w.row_unit;
    a.dest_page = w.dest_page;
    a.dest_slot = w.dest_slot;
    a.new_pages = nullptr;
    a.n_new = w.range;
    a.n_tiles = w.n_tiles;
    a.src_page_table = src->page_table;
    a.src_page_meta = src->page_meta;
    a.src_arena = src->code_arena;
    a.src_maxp = src->max_pages_per_head;
    a.src_of_slot = r.src_of_slot;
    a.src_of_slot_pages = r.src_of_slot_pages;
    a.first_pos = r.first_pos;
    a.page_order = r.page_order;
    a.item_of_slot = nullptr;
    a.item_slot_pages = 0;
    a.row_order = dst->row_order;
    a.rows_total = dst->num_seqs * cfg->num_kv_heads;
    a.half_pairs = 0;   // codes are transcoded, no key is read
    a.n_tiers = cfg->value_tiers ? kNumTiers : 3;
    return hip_status(launch_pack(a, s));
}

ada_status_t ada_read_status(const int32_t *status, void *stream) {
    if (!status) return ADA_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    if (hipStreamSynchronize(s) != hipSuccess) return ADA_EHIP;
    int32_t v = 0;
    if (hipMemcpy(&v, status, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return ADA_EHIP;
    const int32_t zero = 0;
    if (hipMemcpy(const_cast<int32_t *>(status), &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess)
        return ADA_EHIP;
    return (ada_status_t)v;
}

ada_status_t ada_dense_workspace(const ada_config_t *cfg, int32_t B, int32_t max_pages_per_head, size_t *bytes) {
    ada_status_t st = check_cfg(cfg);
    if (st) return st;
    if (!bytes || B < 0 || max_pages_per_head <= 0) return ADA_EINVAL;
    if ((st = check_dims(cfg, B, max_pages_per_head))) return st;
    return ws_out(decode_layout(cfg, B, 1, max_pages_per_head, nullptr).bytes, bytes);
}

ada_status_t ada_dense_decode(const ada_config_t *cfg, int32_t B, int32_t max_pages_per_head,
                              const int32_t *page_table, const int32_t *ctx_len, const uint16_t *k_pool,
                              const uint16_t *v_pool, const float *q, float scale, float *out, float *lse, void *ws,
                              size_t ws_bytes, void *stream) {
    ada_status_t st = check_cfg(cfg);
    if (st) return st;
    if (B < 0 || max_pages_per_head <= 0) return ADA_EINVAL;
    if ((st = check_dims(cfg, B, max_pages_per_head))) return st;
    if (B == 0) return ADA_OK;
    if (!page_table || !ctx_len || !k_pool || !v_pool || !q || !out) return ADA_EINVAL;
    DecodeWs w = decode_layout(cfg, B, 1, max_pages_per_head, ws);
    if (w.bytes > kMaxWorkspace) return ADA_EUNSUPPORTED;
    if (!ws || ws_bytes < w.bytes) return ADA_EINVAL;
    DenseLaunch a;
    a.page_table = page_table;
    a.ctx_len = ctx_len;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.q = q;
    a.pm = w.pm;
    a.pl = w.pl;
    a.pacc = w.pacc;
    a.out = out;
    a.lse = lse;
    a.B = B;
    a.Hq = cfg->num_q_heads;
    a.Hkv = cfg->num_kv_heads;
    a.P = cfg->page_size;
    a.maxp = max_pages_per_head;
    a.chunk_pages = w.cp;
    a.S = w.S;
    a.scale = scale;
    hipError_t e = launch_dense_partials(a, (hipStream_t)stream);
    if (e != hipSuccess) return ADA_EHIP;
    return hip_status(launch_dense_reduce(a, (hipStream_t)stream));
}

ada_status_t ada_probe_copy(const void *src, void *dst, size_t bytes, void *stream) {
    if (!src || !dst || (bytes & 15)) return ADA_EINVAL;
    if (bytes == 0) return ADA_OK;
    return hip_status(launch_probe_copy(src, dst, bytes, (hipStream_t)stream));
}

ada_status_t ada_probe_read(const void *src, size_t bytes, int32_t variant, uint32_t *out, void *stream) {
    if (!src || !out || (bytes & 15) || variant < 0 || variant > 5) return ADA_EINVAL;
    if (bytes == 0) return ADA_OK;
    return hip_status(launch_probe_read(src, bytes, variant, out, (hipStream_t)stream));
}

uint16_t ada_host_f64_to_f16(double x) { return host_f64_to_f16(x); }

}  // extern "C"
