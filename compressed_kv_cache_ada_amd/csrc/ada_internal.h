// ada_internal.h -- shared definitions of the HIP library (not installed).
// Layout rules follow include/ada.h; the method is the angle-domain key
// representation of "SPHERICAL KV" (arXiv 2605.18856, Abstract).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ada.h"

namespace ada {

constexpr int kD = 128;       // head dimension
constexpr int kPairs = 64;    // 2-D pairs per key
constexpr int kMaxChunkPages = 256;   // page list of a split-K work-group (in LDS)

// Tier table in id order: angle bits, magnitude bits, value format.  Ids
// 3-5 carry the keys of ids 0-2 with V8 values instead of fp16.
constexpr int kNumTiers = ADA_NUM_TIERS;
__host__ __device__ constexpr int key_tier(int t) { return t >= 3 ? t - 3 : t; }
__host__ __device__ constexpr int tier_tb(int t) { return key_tier(t) == 0 ? 8 : (key_tier(t) == 1 ? 4 : 2); }
__host__ __device__ constexpr int tier_sb(int t) { return key_tier(t) == 0 ? 8 : (key_tier(t) == 1 ? 4 : 3); }
__host__ __device__ constexpr bool tier_v8(int t) { return t >= 3; }
__host__ __device__ constexpr int tier_vb(int t) { return tier_v8(t) ? 8 : 16; }
// bytes per token and KV head: radius, codes, values (fp16, or V8: 4 scale
// bytes + 128 codes)
__host__ __device__ constexpr int64_t tier_rate(int t) {
    return 2 + 8 * (tier_tb(t) + tier_sb(t)) + (tier_v8(t) ? 132 : 256);
}
// A page's block in the arena: its key part (radius and codes), then its
// value part.  Sizes in 16-byte units:
//   key part   P * (2 + 8 tb + 8 sb) / 16
//   value part P * 256 / 16 (fp16) or P * 132 / 16 (V8)
__host__ __device__ constexpr int key16(int t, int P) { return P * (2 + 8 * tier_tb(t) + 8 * tier_sb(t)) / 16; }
__host__ __device__ constexpr int val16(int t, int P) { return P * (tier_v8(t) ? 132 : 256) / 16; }
__host__ __device__ constexpr int block16(int t, int P) { return key16(t, P) + val16(t, P); }
// fp16 value part: 8-token groups of 2048 bytes, [128 dims][8 tokens] fp16.
// V8 value part: 16-token groups of 2112 bytes, [16 tokens][4 dimension
// blocks] scale bytes (a token's four scales are one 4-byte word), then
// [128 dims][16 tokens] code bytes c + 128 (offset binary)
constexpr int kV8Group = 2112;
constexpr int kV8Codes = 64;   // offset of the codes inside a group

// a pair of fp16 values, both finite
__host__ __device__ inline bool values_finite(uint32_t two_halves) {
    return (two_halves & 0x7C00u) != 0x7C00u && (two_halves & 0x7C000000u) != 0x7C000000u;
}

// fp16 bits -> float
__device__ __forceinline__ float h2f(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// One angle-LUT entry: q-pair projected on the grid direction (cos, sin).
// Shared by the stand-alone LUT builder and the decode's on-chip staging so
// that both produce identical values.
__device__ __forceinline__ float lut_entry(float qx, float qy, float2 cs) {
    return fmaf(qx, cs.x, qy * cs.y);
}

// cos / sin of the 8-bit angle grid point c: th = -pi + c * 2pi / 256.
// The 4- and 2-bit grids are the sub-grids c = 16 c4 and c = 64 c2.
__device__ __forceinline__ float2 grid_dir(int c) {
    float s, co;
    sincospif(-1.0f + (float)c * (1.0f / 128.0f), &s, &co);
    return make_float2(co, s);
}

// Split-K decode work-groups are 4 wavefronts (one per SIMD); this many are
// resident per compute unit (the kernels' launch bounds ask for it).
__host__ __device__ constexpr int decode_waves_per_simd(int G) { return G >= 8 ? 2 : 3; }

// ---- launchers (defined in the .hip files; called by ada_api.cpp) ------
// Q queries per sequence (multi-query decode): q, out are [B][Q][Hq][128].
// The split-K pass treats the Q * G queries of a KV head as G' = Q * G
// "virtual heads" v = qi * G + g; its partials are indexed by the virtual
// row (b * Hkv + h) * G' + v.
struct DecodeLaunch {
    const int32_t *page_table;
    const int32_t *num_pages;
    const ada_page_meta_t *page_meta;
    const uint8_t *arena;
    const float *q;
    float *pm, *pl, *pacc;     // split-K partials
    float *out, *lse;
    int32_t B, Q, Hq, Hkv, P, maxp, chunk_pages, S;
    float scale;
    // fused append (app_page != nullptr): row r's new token, already booked
    // at (app_page[r], app_slot[r]), is encoded and written by the
    // work-group whose chunk holds that page; a booked slot 0 is a new page,
    // which that work-group zeroes first
    const int32_t *app_page, *app_slot;
    const float *app_keys;        // [B * Hkv][128] fp32
    const uint16_t *app_values;   // [B * Hkv][128] fp16 bits
    uint8_t *arena_w;
    int32_t *status;
    // utility emission (logit_buf != nullptr): the split-K pass stores every
    // kept token's base-2 logits at [page * P + slot][Hq / Hkv]; the utility
    // pass turns them into attention mass in util[page * P + slot]
    float *logit_buf;
    float *util;
    int32_t half_pairs;   // pair j = (x[j], x[j + 64]) instead of (x[2j], x[2j + 1])
    int32_t value_tiers;  // the cache may hold pages of tiers 3-5 (V8 values)
    // rows in the order their work-groups are dispatched (longest first), or
    // nullptr for the natural order; only the dispatch order changes
    const int32_t *row_order;
    // G' > 8 (several queries per sequence): the virtual heads are cut into
    // nslice slices of 8, each computed by its own work-group of the chunk
    int32_t nslice;
};
// virtual heads per work-group and slices per chunk for G' virtual heads
__host__ __device__ constexpr int slice_heads(int gv) { return gv < 8 ? gv : 8; }
__host__ __device__ constexpr int slices(int gv) { return gv <= 8 ? 1 : gv / 8; }
hipError_t launch_decode_partials(const DecodeLaunch &a, hipStream_t s);
hipError_t launch_decode_reduce(const DecodeLaunch &a, hipStream_t s);
hipError_t launch_build_lut(const float *q, int32_t rows, float *lut, bool half_pairs, hipStream_t s);
// after the reduction (needs lse): util[page * P + slot] for every kept token
hipError_t launch_decode_utility(const DecodeLaunch &a, hipStream_t s);

struct DenseLaunch {
    const int32_t *page_table;
    const int32_t *ctx_len;
    const uint16_t *k_pool, *v_pool;
    const float *q;
    float *pm, *pl, *pacc;
    float *out, *lse;
    int32_t B, Hq, Hkv, P, maxp, chunk_pages, S;
    float scale;
};
hipError_t launch_dense_partials(const DenseLaunch &a, hipStream_t s);
hipError_t launch_dense_reduce(const DenseLaunch &a, hipStream_t s);

// Encoder / page writer shared by pack and append.
struct EncodeLaunch {
    const float *keys;          // [n][128]
    const uint16_t *values;     // [n][128]
    int64_t n;
    const int32_t *dest_page;   // [n], -1 = skip
    const int32_t *dest_slot;   // [n]
    const ada_page_meta_t *page_meta;
    uint8_t *arena;
    int32_t P;
    int32_t *status;
    int32_t half_pairs;   // pair j = (k[j], k[j + 64]) instead of (k[2j], k[2j + 1])
};
hipError_t launch_encode_write(const EncodeLaunch &a, hipStream_t s);
// Zero the blocks of new pages listed as (page id) in pages[0..*n_pages),
// upper bound max_n.
hipError_t launch_zero_pages(const int32_t *pages, const int32_t *n_pages, int64_t max_n,
                             const ada_page_meta_t *page_meta, uint8_t *arena, int32_t P, const int32_t *status,
                             hipStream_t s);
// Host-callable copies of device helpers, for CPU tests of the library.
uint16_t host_f64_to_f16(double x);

struct PackLaunch {
    int32_t B, Hkv, P, maxp;
    int64_t stride, page_capacity, arena_capacity16;
    const int32_t *ctx_len_dev;     // [B]
    const int8_t *tier;             // [B][Hkv][stride]
    const float *keys;
    const uint16_t *values;
    int32_t *page_table, *num_pages, *open_page;
    ada_page_meta_t *page_meta;
    uint8_t *arena;
    int64_t *alloc;
    int32_t *status;
    // workspace
    int32_t *tile_counts;   // [rows][n_tiles][kNumTiers]
    int32_t *row_counts;    // [rows][kNumTiers]
    int32_t *row_base;      // [rows][kNumTiers] first page id of (row, tier)
    int64_t *row_unit;      // [rows][kNumTiers] first code unit of (row, tier)
    int32_t *dest_page, *dest_slot;   // [B*Hkv*stride]
    int32_t *new_pages;     // [page upper bound] list of allocated pages
    int32_t *n_new;         // [1]
    int32_t n_tiles;
    // re-pack (src_page_table != nullptr): item (row, t) is slot t % P of
    // page-list entry t / P of the source cache's row; its codes are
    // transcoded instead of encoding keys (keys / values unused)
    const int32_t *src_page_table;
    const ada_page_meta_t *src_page_meta;
    const uint8_t *src_arena;
    int32_t src_maxp;
    int4 *src_of_slot;              // [src_of_slot_pages][P] source {page, slot, tier, code_off16} per new slot
    int64_t src_of_slot_pages;
    // re-pack: the source position of each new page's first token, and the
    // order the transcoder writes the new pages in (per row, all tiers by
    // that position), both [src_of_slot_pages]
    int32_t *first_pos, *page_order;
    // pack from keys: the item (row * stride + position) of every new slot,
    // [item_slot_pages][P], for the page writer
    int64_t *item_of_slot;
    int64_t item_slot_pages;
    int32_t half_pairs;             // key pair layout (see EncodeLaunch)
    int32_t n_tiers;                // tier ids below this are accepted (3, or 6 with value tiers)
    // the cache's row order (see ada_cache_t), re-sorted over all rows_total
    // rows after the pages are placed; nullptr: none kept
    int32_t *row_order;
    int32_t rows_total;
};
hipError_t launch_pack(const PackLaunch &a, hipStream_t s);
// pages a re-pack may open per row: sum over three tiers of ceil(n_tau / P)
// with sum n_tau <= src_maxp * P
inline int64_t repack_pages_per_row(int32_t src_maxp) { return (int64_t)src_maxp + 2; }

struct AppendLaunch {
    int32_t n, Hkv, P, num_seqs, maxp;
    int64_t page_capacity, arena_capacity16;
    const int32_t *seq, *head;   // nullptr: request i is row i (sequence i / Hkv, head i % Hkv)
    const uint8_t *tier;
    const float *keys;
    const uint16_t *values;
    int32_t *page_table, *num_pages, *open_page;
    ada_page_meta_t *page_meta;
    uint8_t *arena;
    int64_t *alloc;
    int32_t *status;
    // workspace
    int32_t *key_cnt;    // [keys] requests per (row, tier)
    int32_t *key_c0;     // [keys] initial fill of the open page
    int32_t *key_done;   // [keys] requests already placed
    int32_t *key_page;   // [keys] current page
    int64_t *totals;     // [2] pages, units needed
    int32_t *dest_page, *dest_slot;   // [n]
    int32_t *new_pages;  // [n]
    int32_t *n_new;      // [1]
    int32_t half_pairs;  // key pair layout (see EncodeLaunch)
    int32_t n_tiers;     // tier ids below this are accepted (3, or 6 with value tiers)
};
// append: book destinations, update metadata, zero new pages, then (with
// encode) encode and write the keys; without encode the caller encodes
hipError_t launch_append(const AppendLaunch &a, bool encode, hipStream_t s);
// one request per row (request r = row r, seq / head unused): book, check
// and update metadata in one launch; dest_page / dest_slot get the slots,
// new pages (slot 0) are not zeroed and new_pages[r] holds their code offset
hipError_t launch_append_rows(const AppendLaunch &a, hipStream_t s);

struct RdrLaunch {
    int32_t B, Hkv, n_steps;
    int64_t stride;
    const int32_t *ctx_len_dev;
    const int64_t *budget_dev;
    const float *utility;
    int8_t *tier_out;
    int32_t *status;
    int32_t step_tier[kNumTiers];
    int64_t dR[kNumTiers];
    double c[kNumTiers];
    // workspace: the radix select's histograms, one per pass, and its state
    // (chosen key bytes, bytes above them, "everything fits") before each
    // pass v = 0 .. kRdrPasses - 1 and after the last (v = kRdrPasses)
    unsigned long long *hist;   // [kRdrPasses][B][256]
    unsigned long long *prefix; // [kRdrPasses + 1][B]
    long long *above;           // [kRdrPasses + 1][B]
    int32_t *all_fit;           // [kRdrPasses + 1][B]
    uint8_t *tie_sel;           // [B][Hkv][stride]
    long long *tie_tile;        // [B][rdr_tie_tiles(Hkv * stride)]: tie bytes per tile, then their prefix
    const int8_t *cap;          // optional [B][Hkv][stride]: steps an item may take
};
constexpr int kRdrPasses = 8;       // radix-select passes: one key byte each
constexpr int kRdrTieTile = 1024;   // items per tile of the tie scan
__host__ __device__ inline int64_t rdr_tie_tiles(int64_t items) { return (items + kRdrTieTile - 1) / kRdrTieTile; }
hipError_t launch_rdr(const RdrLaunch &a, hipStream_t s);

// Re-pack items of a source cache: for B * Hkv rows of S = src_maxp * P
// virtual positions, util_v / cap_v get the kept tokens' utilities and step
// caps (0 for empty positions), ctx_v[b] = S.
struct RepackItemsLaunch {
    int32_t B, Hkv, P, src_maxp;
    const int32_t *page_table, *num_pages;
    const ada_page_meta_t *page_meta;
    const float *util;          // [page_capacity][P]
    int8_t level_of_tier[kNumTiers];   // chain tiers holding no more bits than each tier
    float *util_v;
    int8_t *cap_v;
    int32_t *ctx_v;
};
hipError_t launch_repack_items(const RepackItemsLaunch &a, hipStream_t s);

hipError_t launch_cache_init(int32_t rows, int32_t *num_pages, int32_t *open_page, int64_t *alloc,
                             int32_t *status, int32_t *row_order, hipStream_t s);
// rows 0..rows-1 of a cache: page counts, page ids and their metadata in range
hipError_t launch_validate(int32_t rows, int32_t maxp, int64_t page_capacity, int64_t arena16, int32_t P,
                           int32_t n_tiers, const int32_t *num_pages, const int32_t *page_table,
                           const ada_page_meta_t *page_meta, const int32_t *row_order, int32_t order_rows,
                           int32_t *status, hipStream_t s);
hipError_t launch_probe_copy(const void *src, void *dst, size_t bytes, hipStream_t s);
hipError_t launch_probe_read(const void *src, size_t bytes, int variant, uint32_t *out, hipStream_t s);

}  // namespace ada
