/*
 * ada.h -- C ABI of the ADA (Angle-Domain Attention) paged-decode library
 * for AMD Instinct MI355X (gfx950).
 *
 * Method: "SPHERICAL KV: Angle-Domain Attention and Rate-Distortion
 * Retention for Efficient Long-Context Inference" (arXiv 2605.18856),
 * Abstract (newx.sg paper page; searcharxiv.org abstract page).  The
 * abstract states that keys are stored as a scalar radius plus compact angle
 * codes, that attention logits are computed straight from the codes on a
 * paged, block-local decode path, and that Rate-Distortion Retention (RDR)
 * gives every (token, KV head) a precision tier or a drop within a byte
 * budget, the result being pages of a single tier described by small
 * metadata records.  The abstract fixes no bit layout; this header fixes one:
 *
 *  Key codec (head dim 128 -> 64 pairs (k[2j], k[2j+1]); with the half-split
 *  pair layout of ada_config_t, (k[j], k[j+64]), and the query likewise):
 *   radius     r = |k| (fp64, correctly rounded), stored as fp16 (round to
 *              nearest even straight from fp64, saturating at 65504);
 *   magnitude  s_j = |pair j| / r, code = nearest integer to s_j (2^sb - 1),
 *              ties up, dequantised s = code / (2^sb - 1);
 *   angle      th_j = atan2(k[2j+1], k[2j]), code = nearest integer to
 *              (th_j + pi) / (2 pi / 2^tb), ties up, mod 2^tb; dequantised
 *              th = -pi + code * 2 pi / 2^tb; a zero pair gets code 2^(tb-1).
 *   The norm^2 is the fixed pairwise tree sum of the 64 pair energies
 *   (strides 32, 16, ..., 1); codes are decided exactly (not up to rounding).
 *  Tiers (fixed table, id order): ADA_TIER_T8 = (tb 8, sb 8),
 *   ADA_TIER_T4 = (4, 4), ADA_TIER_T2 = (2, 3), all with fp16 values;
 *   ADA_TIER_T8V8, ADA_TIER_T4V8, ADA_TIER_T2V8 = the same keys with V8
 *   values (the abstract's precision tiers per token and head are not
 *   restricted to keys; it names no value format, this one is the
 *   library's):
 *  V8 value codec, per token and head, blocks k of 32 dimensions:
 *     e = floor(log2 max |v_d|) over the block, at least -18 (-18 for an
 *     all-zero block); code c_d = round-half-even(v_d * 2^(6 - e)) clamped
 *     to [-127, 127]; decoded value c_d * 2^(e - 6), an exact fp16 number.
 *     (The pattern of the OCP Microscaling formats: a shared power-of-two
 *     scale per 32 values, 8-bit elements with 6 fraction bits.)  Values of
 *     a V8 token must be finite.
 *  Logit of a kept token t for query q (per query head):
 *     l_t = scale * r_t * sum_j s_j * LUT[j][theta_code_j],
 *     LUT[j][c] = q[2j] cos(th_c) + q[2j+1] sin(th_c),
 *   followed by softmax over the kept tokens of the (sequence, KV head) and
 *   a weighted sum of their values (fp16, or V8 decoded to fp16).
 *
 *  Page layout (page size P in {16, 32}, head dim 128): a page is one block
 *   of the arena, 16-byte aligned at code_arena + 16 * code_off16: its key
 *   part, then its value part (so a page's footprint is exactly its tier's
 *   bytes per token times P).
 *   key part: [radius: P x u16][angle component][magnitude component]; a
 *     component of Bc = 8*b bytes per token is cut into floor(Bc/16) units
 *     of 16 bytes plus one 8-byte unit when Bc mod 16 == 8; unit u of all P
 *     tokens is stored contiguously (token-minor), units in order; code j of
 *     width b occupies bits [j*b, (j+1)*b) of the token's little-endian bit
 *     string.  Key part bytes: T8 130 P, T4 66 P, T2 42 P.
 *   value part, fp16 tiers (256 P bytes): u16 element (slot, d) at
 *     (slot/8)*1024 + d*8 + slot%8 (8-token groups, dimension-major).
 *   value part, V8 tiers (132 P bytes): per 16-token group g, at byte
 *     2112 g, [16 tokens][4 blocks] scale bytes e + 127, then at
 *     2112 g + 64, [128 dims][16 tokens] code bytes c + 128 (offset binary).
 *   Unused slots of a page (slot >= count) are zero in codes and values.
 *
 * Conventions for every call:
 *  - Pointers documented "device" point to HIP device memory owned by the
 *    caller; pointers documented "host" point to host memory read before
 *    the call returns.  The library never allocates or frees memory and
 *    keeps no global state (one exception: ada_decode_noalloc's per-GPU
 *    device array, below); scratch comes from a caller workspace whose size
 *    the matching *_workspace call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream).  All
 *    calls are asynchronous on that stream except ada_read_status.
 *  - Host-side validation happens before any launch and returns ADA_EINVAL /
 *    ADA_EUNSUPPORTED without touching memory.  Errors found on the device
 *    (non-finite key or utility, capacity) are written to a device status
 *    word; the writing kernels of that call then do nothing (all-or-nothing)
 *    and the caller reads and clears the word with ada_read_status.  Calls
 *    made while the status word is non-zero do not modify the cache.
 *  - Shape limits, checked on the host (ADA_EUNSUPPORTED): B * num_q_heads
 *    and max_pages_per_head * page_size fit in int32; a workspace never
 *    exceeds 2^48 bytes (a query that would need more returns
 *    ADA_EUNSUPPORTED instead of a wrapped size).
 *  - No C++ exception crosses this boundary.
 */
#ifndef ADA_H
#define ADA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ADA_OK = 0,
    ADA_EINVAL = 1,          /* bad argument, or non-finite / negative input on the device */
    ADA_ENOSPC = 2,          /* page / arena / row capacity would be exceeded */
    ADA_EUNSUPPORTED = 3,    /* valid but unsupported shape (head dim, page size, group size) */
    ADA_EHIP = 4,            /* a HIP runtime call failed */
    ADA_EINTERNAL = 5        /* an exact code decision could not be made (never expected; the
                                cache is then unspecified: a slot booked by ada_decode_append may
                                be left unwritten) */
} ada_status_t;

enum {
    ADA_TIER_T8 = 0, ADA_TIER_T4 = 1, ADA_TIER_T2 = 2,           /* fp16 values */
    ADA_TIER_T8V8 = 3, ADA_TIER_T4V8 = 4, ADA_TIER_T2V8 = 5,     /* V8 values */
    ADA_NUM_TIERS = 6
};

/* Shape of one attention layer's cache (host struct). */
typedef struct {
    int32_t head_dim;           /* must be 128 */
    int32_t page_size;          /* P: 16 or 32 */
    int32_t num_q_heads;        /* Hq */
    int32_t num_kv_heads;       /* Hkv; Hq / Hkv must be 1, 2, 4 or 8 (query head hq uses KV head hq / (Hq/Hkv)) */
    uint32_t rdr_tier_mask;     /* tiers RDR may assign (bit i = tier id i, i < 6); 0 means
                                   the three fp16 tiers (0x7) */
    int32_t decode_chunk_pages; /* split-K chunk length in pages for ada_decode; 0 = automatic: about
                                   one round of resident work-groups over B * Hkv rows of
                                   max_pages_per_head pages on the current device.  Rounded up to
                                   64 tokens' worth of pages, at most 256.  The same value must be
                                   in effect for the workspace query and the decode calls. */
    int32_t pair_layout;        /* which components of a key (and of a query) form the 64 pairs
                                   (abstract: keys as a radius plus per-pair angle codes; the pairing
                                   is this library's choice): ADA_PAIRS_ADJACENT (k[2j], k[2j+1]) or
                                   ADA_PAIRS_HALF_SPLIT (k[j], k[j+64]), the pairing of the
                                   rotate-half form of rotary position embeddings.  A cache must be
                                   written and read with one layout. */
    int32_t value_tiers;        /* 0: the cache holds tiers 0-2 (fp16 values) only; 1: it may also
                                   hold tiers 3-5 (V8 values): pack and append accept them, RDR may
                                   assign them, and the decode runs its V8-capable kernels.  A
                                   cache must be written and read with one setting. */
} ada_config_t;

enum { ADA_PAIRS_ADJACENT = 0, ADA_PAIRS_HALF_SPLIT = 1 };

/* Metadata of one page, 8 bytes. */
typedef struct {
    uint8_t tier;        /* tier id */
    uint8_t count;       /* filled slots, 1..P */
    uint16_t reserved;   /* zero */
    uint32_t code_off16; /* offset of the page's block in the arena, 16-byte units */
} ada_page_meta_t;

/* The cache: every pointer is device memory owned by the caller.  Row r of
 * the page table belongs to (sequence r / Hkv, KV head r % Hkv). */
typedef struct {
    int32_t num_seqs;           /* rows = num_seqs * Hkv */
    int32_t max_pages_per_head; /* page-table row length */
    int64_t page_capacity;      /* pages in page_meta */
    int64_t arena_capacity16;   /* arena size in 16-byte units (at most 2^32: 64 GiB) */
    int32_t *page_table;        /* [rows][max_pages_per_head] physical page ids */
    int32_t *num_pages;         /* [rows] pages in use per row */
    int32_t *open_page;         /* [rows][ADA_NUM_TIERS] last non-full page per tier, -1 = none */
    ada_page_meta_t *page_meta; /* [page_capacity] */
    uint8_t *code_arena;        /* [arena_capacity16 * 16], 16-byte aligned: the pages' blocks */
    int64_t *alloc;             /* [2]: next page id, next code unit */
    int32_t *status;            /* [1] device error word (0 = OK) */
    int32_t *row_order;         /* [rows] or NULL: the rows by decreasing page count, a schedule hint
                                   for the decode (the longest rows are started first).  A
                                   permutation of 0..rows-1: ada_cache_init writes the identity,
                                   ada_pack and ada_repack (destination) re-sort it (for up to
                                   16384 rows; more keep the identity), appends leave it as it
                                   is.  It changes no result. */
} ada_cache_t;

/* Human-readable name of a status code (static string, never NULL). */
const char *ada_status_str(ada_status_t s);

/* Bytes of one page's block (key part and value part) for a tier and page
 * size (see layout above); -1 for an invalid tier or page size.  Pure host
 * function. */
int64_t ada_block_bytes(int32_t tier, int32_t page_size);

/* Floats of the angle LUT of one query head as written by ada_build_lut:
 * 64 * (256 + 16 + 4) = 17664 (T8, T4, T2 tables in tier-id order). */
size_t ada_lut_floats(const ada_config_t *cfg);

/* Reset the rows, counters and status of a cache: num_pages = 0,
 * open_page = -1, alloc = {0, 0}, status = 0, row_order = 0..rows-1 (when
 * not NULL).  Page contents are left as
 * they are (pages are zeroed when they are allocated). */
ada_status_t ada_cache_init(const ada_config_t *cfg, const ada_cache_t *cache, void *stream);

/* Check the page lists of sequences 0..B-1 before decoding them.  The
 * decode calls do not range-check page ids on their hot path: a page table
 * corrupted or filled by hand (restored from a checkpoint, pages permuted
 * over a shared pool) can make them read outside the buffers.  This call
 * reads, within the buffers only, every row's page count (must be
 * 0..max_pages_per_head), every listed page id (must be 0..page_capacity-1)
 * and that page's metadata (tier id below 3, or below 6 with value_tiers;
 * count 1..page_size; reserved 0; block inside the arena).  Any
 * violation sets the cache's status word to ADA_EINVAL (read and clear it
 * with ada_read_status); nothing is written otherwise.  When the cache has
 * a row_order, it is checked over all num_seqs * num_kv_heads rows too:
 * every entry must lie in 0..rows-1 and, for up to 65536 rows, no entry may
 * appear twice.  Asynchronous on `stream`; one work-group per row, and one
 * more for the row order. */
ada_status_t ada_validate_cache(const ada_config_t *cfg, const ada_cache_t *cache, int32_t B, void *stream);

/* Angle lookup table (the per-query table of the abstract's angle-domain
 * logits): for each query row (b, hq) and each tier, LUT[j][c] =
 * q[2j] cos(th_c) + q[2j+1] sin(th_c), fp32, no softmax scale.
 *   q   device fp32 [B][Hq][128]
 *   lut device fp32 [B][Hq][17664]: T8 [64][256], then T4 [64][16], then T2 [64][4].
 * ada_decode stages the same values in on-chip memory itself and does not
 * read this buffer; this call exists for callers that want the table. */
ada_status_t ada_build_lut(const ada_config_t *cfg, const float *q, int32_t B, float *lut, void *stream);

/* Workspace bytes for ada_decode / ada_decode_partials / ada_decode_reduce
 * on sequences 0..B-1 of `cache` (split-K partials). */
ada_status_t ada_decode_workspace(const ada_config_t *cfg, const ada_cache_t *cache, int32_t B, size_t *bytes);

/* ADA paged decode (abstract: logits from the codes, paged block-local
 * decode path) for sequences 0..B-1: one query per (sequence, query head).
 *   q     device fp32 [B][Hq][128]
 *   scale softmax scale applied to the logits (typically 1/sqrt(128))
 *   out   device fp32 [B][Hq][128]: softmax-weighted sum of kept fp16 values
 *   lse   device fp32 [B][Hq] natural-log sum-exp of the scaled logits, or NULL
 *   ws    device workspace of at least ada_decode_workspace() bytes
 * A row with no kept token gives out = 0 and lse = -inf.  Runs the split-K
 * pass (LUT staging, logits, online softmax, value accumulation per context
 * chunk) then the reduction pass.  Page ids are not range-checked. */
ada_status_t ada_decode(const ada_config_t *cfg, const ada_cache_t *cache, const float *q, int32_t B,
                        float scale, float *out, float *lse, void *ws, size_t ws_bytes, void *stream);

/* ada_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * allocation-free harnesses).  Same arguments, kernels and results as
 * ada_decode (bit for bit); the split-K partials go to a device array of
 * 16 MiB inside the library instead of a caller workspace.  Each GPU the
 * library runs on holds its own copy of that array until the process ends;
 * this call allocates and frees nothing.  Limit: the partials of the call,
 * about 520 bytes per (sequence, query head, split-K chunk) -- the size
 * ada_decode_workspace reports -- must fit in 16 MiB, else ADA_EUNSUPPORTED
 * before any launch (llama8b-like layer: 1.6 MB at B = 8, 32k context).
 * ADA_EHIP if the array's address cannot be obtained.  All calls on one GPU
 * share the array: calls whose executions overlap on one GPU (other streams,
 * other host threads) race and give undefined results; calls ordered on one
 * stream do not. */
ada_status_t ada_decode_noalloc(const ada_config_t *cfg, const ada_cache_t *cache, const float *q, int32_t B,
                                float scale, float *out, float *lse, void *stream);

/* The two passes of ada_decode, callable separately (same arguments). */
ada_status_t ada_decode_partials(const ada_config_t *cfg, const ada_cache_t *cache, const float *q, int32_t B,
                                 float scale, void *ws, size_t ws_bytes, void *stream);
ada_status_t ada_decode_reduce(const ada_config_t *cfg, const ada_cache_t *cache, int32_t B,
                               float *out, float *lse, void *ws, size_t ws_bytes, void *stream);

/* Multi-query decode: Q queries per sequence (speculative drafts, beams,
 * several positions' queries), all attending to the same cached tokens.
 * One pass over the cache serves every query: the Q * G queries of a KV head
 * share each code and value read (G = Hq / Hkv).  Q must be a power of two
 * with Q * G <= 64, else ADA_EUNSUPPORTED.  Up to Q * G = 8 one work-group
 * computes every query of its chunk; beyond that the Q * G virtual heads are
 * cut into slices of 8, each computed by its own work-group of the chunk
 * (placed so that the slices read the chunk's pages at the same time, on one
 * of the chip's dies).
 *   q     device fp32 [B][Q][Hq][128]
 *   out   device fp32 [B][Q][Hq][128]; lse device fp32 [B][Q][Hq] or NULL
 *   ws    device workspace of at least ada_decode_multi_workspace() bytes
 * Query (b, i) gives exactly what ada_decode gives for the query q[b][i]
 * (up to rounding: the split-K chunking may differ).  ada_decode is this
 * call with Q = 1. */
ada_status_t ada_decode_multi_workspace(const ada_config_t *cfg, const ada_cache_t *cache, int32_t B, int32_t Q,
                                        size_t *bytes);
ada_status_t ada_decode_multi(const ada_config_t *cfg, const ada_cache_t *cache, const float *q, int32_t B,
                              int32_t Q, float scale, float *out, float *lse, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes for ada_encode_append with n requests. */
ada_status_t ada_append_workspace(const ada_config_t *cfg, const ada_cache_t *cache, int32_t n, size_t *bytes);

/* Encode n new keys into their tiers and append them with their values
 * (abstract: keys stored as radius + angle codes in tier-homogeneous pages).
 * Sequential semantics in request order: request i fills the open page of
 * (seq[i], kv_head[i], tier[i]) at its next slot, or opens a new page (next
 * page id, next block of the arena) appended to that row.
 *   seq, kv_head device int32 [n]; tier device uint8 [n]
 *   keys   device fp32 [n][128]; values device fp16 bits [n][128]
 * Device errors: out-of-range seq / head / tier, non-finite key or non-finite
 * value of a V8 token -> ADA_EINVAL; capacity -> ADA_ENOSPC; in both cases
 * nothing is written. */
ada_status_t ada_encode_append(const ada_config_t *cfg, const ada_cache_t *cache, int32_t n,
                               const int32_t *seq, const int32_t *kv_head, const uint8_t *tier,
                               const float *keys, const uint16_t *values, void *ws, size_t ws_bytes,
                               void *stream);

/* Workspace bytes for ada_decode_utility on sequences 0..B-1 (grows with
 * the cache's page_capacity: 4 * P * Hq/Hkv bytes per page).  The logit
 * buffer is addressed with 32-bit offsets: page_capacity * P * Hq/Hkv must
 * not exceed 2^32 - 1, else ADA_EUNSUPPORTED (here and in the call). */
ada_status_t ada_decode_utility_workspace(const ada_config_t *cfg, const ada_cache_t *cache, int32_t B,
                                          size_t *bytes);

/* ADA decode that also emits each kept token's utility for RDR (abstract:
 * retention chosen by estimated future utility; the estimator is not
 * defined there, and this is the attention the token receives in this
 * step): for every kept token of sequences 0..B-1,
 *     util[page * P + slot] = sum over the KV head's query heads hq of
 *                             exp(logit_t(hq) - lse(hq)),
 * the token's softmax weights in this decode summed over its query heads
 * (the values over one KV row sum to Hq / Hkv).  Other entries of util are
 * not written.
 *   util  device fp32 [page_capacity][P]
 *   out, lse, q, scale as for ada_decode (lse may be NULL)
 * Runs the split-K pass (which also stores the kept tokens' logits, 4 bytes
 * per token and query head), the reduction, and the utility pass. */
ada_status_t ada_decode_utility(const ada_config_t *cfg, const ada_cache_t *cache, const float *q, int32_t B,
                                float scale, float *out, float *lse, float *util, void *ws, size_t ws_bytes,
                                void *stream);

/* Workspace bytes for ada_repack of sequences 0..B-1 of `src`. */
ada_status_t ada_repack_workspace(const ada_config_t *cfg, const ada_cache_t *src, int32_t B, size_t *bytes);

/* RDR re-pack (abstract: retention and precision chosen per token and head
 * under a fixed budget from estimated future utility; here the budget may
 * shrink over time and the cache is re-fitted to it).  The items of sequence
 * b are the kept tokens of its rows in `src`: item (h, t) is slot t % P of
 * page-list entry t / P of row (b, h), t playing the part of the position in
 * the RDR order; its utility is util[page * P + slot] (for instance from
 * ada_decode_utility).  Each item may keep its tier, move to an enabled tier
 * holding no more angle, magnitude or value bits, or be dropped (the codes
 * hold nothing finer); the enabled tiers in rate order must each hold no
 * fewer bits than the one before (else ADA_EUNSUPPORTED),
 * under budget[b] bytes with the rate / distortion model of ada_rdr_assign.
 * Kept items are transcoded in code space -- angle codes to the nearest
 * point of the nested coarser grid (half up), magnitude codes to the nearest
 * level (no ties occur between these tiers), radius unchanged, values
 * re-encoded from their decoded fp16 numbers in the new tier's format --
 * and packed into `dst` exactly as ada_pack lays out a tier map over
 * positions 0 .. src.max_pages_per_head * P - 1 (tier id ascending, then
 * position).  dst must be a different cache; its rows of sequences < B are
 * rewritten and its pages are allocated from its alloc counters.
 *   util    device fp32 [src.page_capacity][P], finite and >= 0 where kept
 *   budget  host int64 [B] bytes
 * Device errors land in dst's status word (bad utility -> ADA_EINVAL,
 * capacity -> ADA_ENOSPC; then dst is not written). */
ada_status_t ada_repack(const ada_config_t *cfg, const ada_cache_t *src, int32_t B, const float *util,
                        const int64_t *budget, const ada_cache_t *dst, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes for ada_decode_append on sequences 0..B-1. */
ada_status_t ada_decode_append_workspace(const ada_config_t *cfg, const ada_cache_t *cache, int32_t B,
                                         size_t *bytes);

/* Fused append + decode for one decode step: each (sequence b < B, KV
 * head h) gets one new token, which is encoded into its tier's open page
 * (abstract: keys stored as radius + angle codes in tier-homogeneous pages)
 * and attended to in the same split-K launch.  The result equals
 * ada_encode_append of the B * Hkv requests in row order (b, h ascending)
 * followed by ada_decode(q): the same pages, bytes and metadata, and the
 * same outputs.
 *   q          device fp32 [B][Hq][128]
 *   new_keys   device fp32 [B][Hkv][128]; new_values device fp16 bits [B][Hkv][128]
 *   new_tier   device uint8 [B][Hkv] (tier id)
 *   out, lse   as for ada_decode
 *   ws         device workspace of at least ada_decode_append_workspace() bytes
 * The new slots are booked first (metadata updated, new pages zeroed); in the
 * split-K launch the work-group whose context chunk holds a booked slot
 * encodes the key and writes the slot before reading any of its pages.
 * Device errors are the append's (bad tier, non-finite key or non-finite
 * value of a V8 token -> ADA_EINVAL,
 * capacity -> ADA_ENOSPC, in the status word): then nothing is written and
 * out / lse cover the tokens cached before the call. */
ada_status_t ada_decode_append(const ada_config_t *cfg, const ada_cache_t *cache, const float *q, int32_t B,
                               float scale, const float *new_keys, const uint16_t *new_values,
                               const uint8_t *new_tier, float *out, float *lse, void *ws, size_t ws_bytes,
                               void *stream);

/* Workspace bytes for ada_rdr_assign over B sequences of stride ctx_stride. */
ada_status_t ada_rdr_workspace(const ada_config_t *cfg, int32_t B, int64_t ctx_stride, size_t *bytes);

/* RDR keep/drop + tier choice under a byte budget (abstract: RDR gives each
 * (token, KV head) a precision tier or a drop, within a budget).
 * Items are (KV head, position) of one sequence, all heads sharing the
 * sequence's budget.  Rate of a tier: 2 + 8 (tb + sb) + 256 bytes (fp16
 * values) or + 132 (V8 values); distortion 2^-(tb + sb), plus 2^-14 for V8
 * values; drop: rate 0, distortion 1.  Enabled tiers in
 * rate order form upgrade steps drop -> ... with cost dR_k and priority
 * w * (dD_k / dR_k) (fp64); steps are taken in order of priority descending,
 * position descending, head ascending, step ascending, while the byte total
 * stays within the budget, stopping at the first step that does not fit.
 *   ctx_len    host int32 [B] (<= ctx_stride)
 *   utility    device fp32 [B][Hkv][ctx_stride], finite and >= 0
 *   budget     host int64 [B] bytes
 *   tier_out   device int8 [B][Hkv][ctx_stride]: tier id or -1 (dropped, or
 *              position >= ctx_len)
 *   status     device int32 [1]: set to ADA_EINVAL for a bad utility
 * Returns ADA_EUNSUPPORTED when the enabled tiers' savings per byte do not
 * strictly decrease. */
ada_status_t ada_rdr_assign(const ada_config_t *cfg, int32_t B, const int32_t *ctx_len, int64_t ctx_stride,
                            const float *utility, const int64_t *budget, int8_t *tier_out, int32_t *status,
                            void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes for ada_pack over B sequences of stride ctx_stride. */
ada_status_t ada_pack_workspace(const ada_config_t *cfg, const ada_cache_t *cache, int32_t B, int64_t ctx_stride,
                                size_t *bytes);

/* Bulk pack (prefill) of sequences 0..B-1 from a tier map (abstract:
 * tier-homogeneous pages with lightweight metadata).  For each sequence,
 * KV head and tier id ascending, the kept tokens in ascending position are
 * cut into pages of P with consecutive page ids and blocks taken from
 * alloc; the rows of sequences 0..B-1 are (re)initialised; open_page holds
 * each (row, tier)'s last page if it is not full.
 *   ctx_len host int32 [B]
 *   tier    device int8 [B][Hkv][ctx_stride] (-1 = drop)
 *   keys    device fp32 [B][Hkv][ctx_stride][128]; values device fp16 bits, same shape
 * Device errors (tier out of range, non-finite kept key, non-finite value
 * of a V8 token -> ADA_EINVAL; capacity -> ADA_ENOSPC) leave the cache
 * unmodified. */
ada_status_t ada_pack(const ada_config_t *cfg, const ada_cache_t *cache, int32_t B, const int32_t *ctx_len,
                      int64_t ctx_stride, const int8_t *tier, const float *keys, const uint16_t *values,
                      void *ws, size_t ws_bytes, void *stream);

/* Synchronise `stream`, return the device status word of `cache` (or
 * ADA_EHIP if the copy fails) and reset it to 0. */
ada_status_t ada_read_status(const int32_t *status, void *stream);

/* ---- Measurement companions (not part of the method) ------------------ */

/* Dense fp16 paged decode over un-compressed keys and values, with the same
 * split-K skeleton as ada_decode; used as a traffic and footprint reference.
 *   page_table device int32 [B*Hkv][max_pages_per_head]; ctx_len device int32 [B]
 *   (every row of sequence b holds ctx_len[b] tokens in its pages, in order)
 *   k_pool device fp16 [pages][P*128]: element (slot, d) at (d/8)*P*8 + slot*8 + d%8
 *   v_pool device fp16 [pages][P*128]: same layout as ADA value pages
 *   other arguments as ada_decode. */
ada_status_t ada_dense_workspace(const ada_config_t *cfg, int32_t B, int32_t max_pages_per_head, size_t *bytes);
ada_status_t ada_dense_decode(const ada_config_t *cfg, int32_t B, int32_t max_pages_per_head,
                              const int32_t *page_table, const int32_t *ctx_len, const uint16_t *k_pool,
                              const uint16_t *v_pool, const float *q, float scale, float *out, float *lse,
                              void *ws, size_t ws_bytes, void *stream);

/* Plain streaming copy of `bytes` (multiple of 16) from src to dst, device
 * pointers: calibration of memory counters and the stream bandwidth ceiling. */
ada_status_t ada_probe_copy(const void *src, void *dst, size_t bytes, void *stream);

/* Streaming read of `bytes` (multiple of 16) from device memory: the
 * bandwidth ceiling a read-dominated kernel can reach on this device.
 * variant 0: one 16-byte load per lane in flight, grid-stride (the active
 * work-groups read a moving window); 1: four loads; 2: four with the
 * non-temporal hint; 3: eight with the hint; 4: each work-group reads its
 * own contiguous region (many distant streams); 5: each wavefront reads
 * whole 16 KB chunks (sixteen loads per lane in flight) in a scrambled
 * order, at most three 256-thread work-groups per compute unit -- the
 * access pattern of the decode's value reads; it reads the largest
 * power-of-two number of 16 KB chunks that fits in `bytes`.  `out` (device,
 * 1 word) is only written when the xor of the data hits a fixed value. */
ada_status_t ada_probe_read(const void *src, size_t bytes, int32_t variant, uint32_t *out, void *stream);

/* Host-side evaluation of the library's fp64 -> fp16 radius rounding (round
 * to nearest even straight from fp64, saturating at 65504): the same code the
 * encoder runs on the device, exported so CPU tests can check it. */
uint16_t ada_host_f64_to_f16(double x);

#ifdef __cplusplus
}
#endif
#endif /* ADA_H */
