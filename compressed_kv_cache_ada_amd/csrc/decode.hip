// decode.hip -- ADA paged decode for gfx950: angle-LUT staging, tier-specialised
// logits from codes, wavefront online softmax, fp16 value accumulation,
// split-K partials over context chunks and the reduction pass.
//
// Method: "SPHERICAL KV" (arXiv 2605.18856), Abstract: logits come straight
// from the radius + angle codes (no dense key is rebuilt) on a paged,
// block-local decode path that streams tier-homogeneous pages.
//
// The split-K skeleton (page staging, value loads, online softmax, value
// accumulation on the matrix cores, chunk partials) is decode_core.h; this
// file supplies the ADA logits.  The G = Hq/Hkv query heads of a KV head
// share every code and value read.
//   logits:  lane = token; the token's 16-byte code units arrive through a
//            per-wavefront LDS stage filled by direct global-to-LDS 128-bit
//            loads one group ahead (units are token-minor, so the 64 lanes
//            read contiguous memory); per pair j the lane gathers
//            LUT_g[j][theta_code] from LDS for every head g and accumulates
//            s_code * entry.  T8 uses the factorised form
//            s (cos th, sin th) . (q[2j], q[2j+1]) with a 256-entry cos/sin
//            table in LDS instead of a 64 KB-per-head table.
// There is no matrix-core work in the logit path: it is a gather-reduce over
// small per-pair tables, not a dense contraction.
#include "decode_core.h"
#include "encode_core.h"

namespace ada {
namespace {

using core::ldg;

// ---- logits per tier (lane = token) --------------------------------------
// Each returns base-2 scaled logits: scale * log2(e) * r * sum_j s_j LUT[j][c].

// T8: at most 16 table reads in flight -- a compiler barrier every JB pairs
// stops the scheduler from hoisting all reads of an unrolled unit into
// registers.
template <int G>
__device__ __forceinline__ void pair_fence(int j) {
    constexpr int JB = 16 / G;
    if ((j + 1) % JB == 0) asm volatile("" ::: "memory");
}

// Makes a code word opaque at this point of the program, so the field
// extractions that use it cannot be hoisted above the preceding pairs.
__device__ __forceinline__ uint32_t pin(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Code units of one token in registers.  Unit use per tier:
//   T4: u[0..1] angle units, u[2..3] magnitude units
//   T2: u[0] angle unit, u[1] magnitude unit, h the 8-byte magnitude unit
//       (u[2], u[3] repeat u[1])
//   T8: u[0..1] angle units 0-1, u[2..3] magnitude units 0-1 (pairs 0-31);
//       units 2-3 (pairs 32-63) are read by the T8 logit routine itself
struct CodeRegs {
    uint4 u[4];
    uint2 h;
    uint32_t r;         // fp16 radius bits
    const uint8_t *c;   // the token's first angle unit
    bool v8_fma;        // V8 values: the group's scales allow the fused conversion
};

// Per-work-group LUT layout, per pair j with NC codes: slices of SW =
// min(G, 4) heads, [j][slice][code][SW] -- [j][code][head] for G <= 4.  One
// LDS read per slice returns a lane's SW heads; with at most 16 bytes per
// code the 16 codes of a slice span 256 contiguous bytes, so the lanes'
// random codes fall in distinct bank groups.
template <int G>
constexpr int lut_sw() { return G < 4 ? G : 4; }

template <int G, int NC>
__device__ __forceinline__ int lut_index(int j, int c, int g) {
    constexpr int SW = lut_sw<G>();
    return ((j * (G / SW) + g / SW) * NC + c) * SW + g % SW;
}

// Gathers the LUT entries of one (pair, code) for the G heads into e[];
// `pair` points at the pair's NC * G floats.
template <int G, int NC>
__device__ __forceinline__ void lut_load(const float *pair, uint32_t c, float (&e)[G]) {
    constexpr int SW = lut_sw<G>();
#pragma unroll
    for (int sl = 0; sl < G / SW; ++sl) {
        const float *src = pair + (sl * NC + c) * SW;
        if constexpr (SW == 4) {
            const float4 v = *reinterpret_cast<const float4 *>(src);
            e[4 * sl] = v.x;
            e[4 * sl + 1] = v.y;
            e[4 * sl + 2] = v.z;
            e[4 * sl + 3] = v.w;
        } else if constexpr (SW == 2) {
            const float2 v = *reinterpret_cast<const float2 *>(src);
            e[0] = v.x;
            e[1] = v.y;
        } else {
            e[0] = src[0];
        }
    }
}

// lut_load for G >= 4 (16-byte entries), from the code's byte offset c * 16
template <int G, int NC>
__device__ __forceinline__ void lut_load16(const float *pair, uint32_t c16, float (&e)[G]) {
    static_assert(lut_sw<G>() == 4, "16-byte LUT entries");
#pragma unroll
    for (int sl = 0; sl < G / 4; ++sl) {
        const float4 v = *reinterpret_cast<const float4 *>(reinterpret_cast<const char *>(pair) + sl * NC * 16 + c16);
        e[4 * sl] = v.x;
        e[4 * sl + 1] = v.y;
        e[4 * sl + 2] = v.z;
        e[4 * sl + 3] = v.w;
    }
}

template <int G>
__device__ __forceinline__ void logits_t4(const CodeRegs &k, const float *lut4, float mul, float (&lg)[G]) {
    const uint32_t tw[8] = {k.u[0].x, k.u[0].y, k.u[0].z, k.u[0].w, k.u[1].x, k.u[1].y, k.u[1].z, k.u[1].w};
    const uint32_t sw[8] = {k.u[2].x, k.u[2].y, k.u[2].z, k.u[2].w, k.u[3].x, k.u[3].y, k.u[3].z, k.u[3].w};
    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.f;
    // word by word (8 pairs): the 8 gathers are issued together, then the
    // FMAs; a compiler fence keeps the next word's work after this one.
    // Magnitude nibbles are split into even / odd bytes (made opaque, so
    // that the compiler does not fold the split back into per-nibble field
    // extractions) and each converts to float with one byte-select
    // conversion.  With 16-byte table entries (G >= 4) a code's byte offset
    // c * 16 is a byte's high nibble: in place for odd pairs, in t << 4 for
    // even ones, one byte-select AND each.
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        const uint32_t t = tw[w];
        const uint32_t se = pin(sw[w] & 0x0F0F0F0Fu), so = pin((sw[w] >> 4) & 0x0F0F0F0Fu);
        const float *lu = lut4 + w * 8 * 16 * G;
        float e[8][G];
        if constexpr (lut_sw<G>() == 4) {
            const uint32_t te = pin(t << 4);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                lut_load16<G, 16>(lu + j * 16 * G, (((j & 1) ? t : te) >> (8 * (j >> 1))) & 0xF0u, e[j]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) lut_load<G, 16>(lu + j * 16 * G, (t >> (4 * j)) & 15u, e[j]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t sb = (j & 1) ? so : se;
            const float s = (float)((sb >> (8 * (j >> 1))) & 0xFFu);
#pragma unroll
            for (int g = 0; g < G; ++g) acc[g] = fmaf(s, e[j][g], acc[g]);
        }
        asm volatile("" ::: "memory");
    }
    const float m = h2f(k.r) * mul * (1.0f / 15.0f);
#pragma unroll
    for (int g = 0; g < G; ++g) lg[g] = acc[g] * m;
}

// T2 angles are the 4-bit grid's points 4 c (both grids start at -pi), so
// the T4 table serves T2 codes at index 4 c: the same entries, bit for bit,
// without a table of their own
template <int G>
__device__ __forceinline__ void logits_t2(const CodeRegs &k, const float *lut4, float mul, float (&lg)[G]) {
    // quarter q covers pairs 16q..16q+15: angle word q (2-bit codes) and
    // magnitude bits [48q, 48q+48) (3-bit codes)
    const uint32_t tw[4] = {k.u[0].x, k.u[0].y, k.u[0].z, k.u[0].w};
    // the 192 magnitude bits are words u[1].x..w, h.x, h.y; quarter q
    // starts at bit 48q: windows at bits 0, 48, 96 and 144
    const uint64_t win4[4] = {
        ((uint64_t)k.u[1].y << 32) | k.u[1].x,
        (((uint64_t)k.u[1].z << 32) | k.u[1].y) >> 16,
        ((uint64_t)k.h.x << 32) | k.u[1].w,
        (((uint64_t)k.h.y << 32) | k.h.x) >> 16,
    };
    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t t = tw[q];
        const uint64_t win = win4[q];
        const float *lu = lut4 + q * 16 * 16 * G;
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {   // 8 pairs at a time
            float e[8][G];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int jj = 8 * h8 + j;
                lut_load<G, 16>(lu + jj * 16 * G, 4u * ((t >> (2 * jj)) & 3u), e[j]);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int jj = 8 * h8 + j;
                const float s = (float)((uint32_t)(win >> (3 * jj)) & 7u);
#pragma unroll
                for (int g = 0; g < G; ++g) acc[g] = fmaf(s, e[j][g], acc[g]);
            }
            asm volatile("" ::: "memory");
        }
    }
    const float m = h2f(k.r) * mul * (1.0f / 7.0f);
#pragma unroll
    for (int g = 0; g < G; ++g) lg[g] = acc[g] * m;
}

// 16 pairs of 8-bit codes: angle word array tw[4], magnitude word array sw[4]
template <int G>
__device__ __forceinline__ void t8_unit(const uint32_t (&tw)[4], const uint32_t (&sw)[4], const float2 *cs8,
                                        const float *qu, float (&acc)[G]) {
    uint32_t tcur = 0, scur = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        if ((j & 3) == 0) {
            tcur = pin(tw[j >> 2]);
            scur = pin(sw[j >> 2]);
        }
        const uint32_t c = (tcur >> ((j & 3) * 8)) & 255u;
        const float s = (float)((scur >> ((j & 3) * 8)) & 255u);
        const float2 cs = cs8[c];
        const float ux = s * cs.x, uy = s * cs.y;
        const float *qq = qu + j * G * 2;
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g] = fmaf(ux, qq[2 * g], fmaf(uy, qq[2 * g + 1], acc[g]));
        pair_fence<G>(j);
    }
}

template <int G, int P>
__device__ __forceinline__ void logits_t8(const CodeRegs &k, const float2 *cs8, const float *q8, float mul,
                                          float (&lg)[G]) {
    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const uint32_t tw[4] = {k.u[u].x, k.u[u].y, k.u[u].z, k.u[u].w};
        const uint32_t sw[4] = {k.u[2 + u].x, k.u[2 + u].y, k.u[2 + u].z, k.u[2 + u].w};
        t8_unit<G>(tw, sw, cs8, q8 + u * 16 * G * 2, acc);
    }
#pragma unroll
    for (int u = 2; u < 4; ++u) {
        const uint4 t = ldg<uint4>(k.c + u * 16 * P);
        const uint4 v = ldg<uint4>(k.c + (4 + u) * 16 * P);
        const uint32_t tw[4] = {t.x, t.y, t.z, t.w};
        const uint32_t sw[4] = {v.x, v.y, v.z, v.w};
        t8_unit<G>(tw, sw, cs8, q8 + u * 16 * G * 2, acc);
    }
    const float m = h2f(k.r) * mul * (1.0f / 255.0f);
#pragma unroll
    for (int g = 0; g < G; ++g) lg[g] = acc[g] * m;
}

// ---- ADA logit policy for the split-K core -------------------------------
// Per-wavefront LDS staging of one 64-token group's code units, filled by
// direct global-to-LDS loads (lane = token): units 0-3 as in CodeRegs, the
// aligned 16 bytes holding the token's 8-byte T2 unit, and the aligned
// dword holding its fp16 radius.
struct CodeStage {
    uint4 u[4][64];
    uint4 h[64];
    uint32_t r[64];
};

template <int G, int P, int NW, bool APPEND, bool VT>
struct AdaPolicy {
    static constexpr bool kStaged = true;
    static constexpr bool kEarlyStage = !APPEND;   // the fused append writes before any read
    static constexpr bool kValueTiers = VT;   // the cache may hold pages of tiers 3-5 (V8 values)
    struct Smem {
        float lut4[64 * 16 * G];   // 4-bit angle grid (and the 2-bit one), lut_index<G, 16> layout
        float2 cs8[256];           // cos / sin of the 8-bit grid
        float2 cs4[16];            // the 4-bit sub-grid, contiguous (conflict-free reads)
        float q8[64 * G * 2];      // [j][g][x|y] query pairs (T8, factorised)
        CodeStage st[NW];          // the next group's code units, per wavefront
        uint32_t enc_words[2][16]; // bit-string packing of the fused append's key
        int app_status;            // the status word as read once by the work-group (fused append)
        // V8 scale word of each token of the next group (lane = token)
        uint32_t vs[NW][VT ? 64 : 1];
        // the current group's fp16 scales per dimension block (lane = token),
        // so that a lane reads eight tokens' scales of a block at once
        alignas(16) uint16_t vsc[NW][VT ? 4 : 1][64];
    };
    const int32_t *num_pages_;
    const ada_page_meta_t *page_meta;
    const uint8_t *arena;
    const float *q;
    int32_t Q, Hq, Gr;   // queries per sequence, query heads, query heads per KV head
    int32_t voff;        // first virtual head of this work-group (slices of 8 when Q * Gr > 8)
    int32_t half;        // pair j = (x[j], x[j + 64]) instead of (x[2j], x[2j + 1])
    float mul;   // softmax scale * log2(e)
    // fused append (APPEND)
    const int32_t *app_page, *app_slot;
    const float *app_keys;
    const uint16_t *app_values;
    uint8_t *arena_w;
    int32_t *status;

    // Fused append: the work-group whose chunk holds the page booked for the
    // row's new token encodes it (wavefront 0) and writes radius, codes and
    // value into its slot before any wavefront reads the chunk's pages.  No
    // other work-group reads that page.  Skipped when the booking failed.
    // The status word is read once per work-group (thread 0, through LDS),
    // so that all its wavefronts take the same path through the barriers.
    __device__ bool after_pages(Smem &s, const int *pages, int nch, int row, int w, int lane) const {
        if constexpr (!APPEND) {
            return false;
        } else {
            if (threadIdx.x == 0) s.app_status = enc::read_status(status);
            __syncthreads();
            if (s.app_status != 0) return false;
            const int dp = app_page[row];
            bool own = false;
            for (int i = lane; i < nch; i += 64) own |= pages[i] == dp;
            own = __any(own);   // the same in every wavefront
            if (!own) return false;
            const int slot = app_slot[row];
            const uint2 m = ldg<uint2>(page_meta + dp);
            if (slot == 0) {   // a new page: zero its block (key and value parts)
                const int tid = threadIdx.x;
                uint4 *cb = reinterpret_cast<uint4 *>(arena_w + (size_t)m.y * 16);
                for (int k = tid; k < block16(m.x & 0xFF, P); k += NW * 64) cb[k] = make_uint4(0u, 0u, 0u, 0u);
                __threadfence_block();
                __syncthreads();
            }
            if (w == 0) {
                enc::encode_write_one(app_keys + (size_t)row * kD, app_values + (size_t)row * kD, slot, m, arena_w, P,
                                      status, s.enc_words, half != 0);
                __threadfence_block();
            }
            return true;
        }
    }

    __device__ int num_pages(int row, int) const { return num_pages_[row]; }
    __device__ int num_pages_lane(int row, int, uint32_t z) const { return num_pages_[row + z]; }
    __device__ uint2 meta(int page, int, int) const { return ldg<uint2>(page_meta + page); }
    // a page's value part: its block's bytes after the key part
    __device__ const uint8_t *value_part(int, uint2 m) const {
        // key part units per 16 tokens by key tier, one byte each (130, 66, 42)
        static_assert(key16(0, 16) == 130 && key16(1, 16) == 66 && key16(2, 16) == 42, "key part sizes");
        const uint32_t k16 = (0x2A4282u >> (8 * key_tier(m.x & 0xFF))) & 0xFFu;
        return arena + (size_t)(m.y + k16 * (P / 16)) * 16;
    }

    // phase 1: query pairs and the grid directions.  Virtual head voff + v
    // of the KV head is query qi = (voff + v) / Gr, head h * Gr + (voff + v)
    // % Gr of q [B][Q][Hq][128]; component d is x (0) or y (1) of pair j in
    // the cache's pair layout.
    __device__ void prologue(Smem &s, int b, int h, int tid, int nt) const {
        // every query load of the thread is issued before the first store
        constexpr int NTQ = NW * 64;
        constexpr int NQ = (G * kD + NTQ - 1) / NTQ;
        float qv[NQ];
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            const int i = tid + k * NTQ;
            const int v = i >> 7, d = i & 127;
            const int qi = (voff + v) / Gr, g = (voff + v) % Gr;
            qv[k] = i < G * kD ? q[(((size_t)b * Q + qi) * Hq + (size_t)h * Gr + g) * kD + d] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            const int i = tid + k * NTQ;
            const int v = i >> 7, d = i & 127;
            const int j = half ? (d & 63) : (d >> 1), xy = half ? (d >> 6) : (d & 1);
            if (i < G * kD) s.q8[(j * G + v) * 2 + xy] = qv[k];
        }
        for (int c = tid; c < 256; c += nt) {
            const float2 d = grid_dir(c);
            s.cs8[c] = d;
            if ((c & 15) == 0) s.cs4[c >> 4] = d;
        }
    }

    // phase 2 (after a barrier): the T4 table (T2 codes use its entries 4 c)
    __device__ void build(Smem &s, int tid, int nt) const {
        // consecutive threads fill consecutive heads, then codes; every
        // thread fills the same number of entries, a compile-time count, so
        // that the table reads of four entries are in flight together
        constexpr int NTB = NW * 64;
        static_assert((64 * 16 * G) % NTB == 0, "LUT entries per thread");
#pragma unroll 4
        for (int k = 0; k < 64 * 16 * G / NTB; ++k) {
            const int i = tid + k * NTB;
            const int g = i % G, c = (i / G) & 15, j = i / (16 * G);
            s.lut4[lut_index<G, 16>(j, c, g)] =
                lut_entry(s.q8[(j * G + g) * 2], s.q8[(j * G + g) * 2 + 1], s.cs4[c]);
        }
    }

    using Codes = CodeRegs;

    // fp16 scales of dimension block b for tokens tok .. tok + 7 of the
    // current group (tok a multiple of 8), as the pairs (tok + 2i, tok + 2i + 1)
    __device__ void scale_pairs(const Smem &s, int w, int tok, int b, uint32_t (&sp)[4]) const {
        if constexpr (VT) {
            const uint4 v = *reinterpret_cast<const uint4 *>(&s.vsc[w][b][tok]);
            sp[0] = v.x;
            sp[1] = v.y;
            sp[2] = v.z;
            sp[3] = v.w;
        }
    }

    // Issues the direct-to-LDS loads of a group's code units into wavefront
    // w's stage (lane = token, wave-uniform destinations).  Branch-free:
    // every address stays inside the lane's own code block (and, for the
    // V8 scale word, inside its page's value slot).
    __device__ void stage(Smem &s, int w, uint2 meta, int page, int slot_) const {
        // slot-derived offsets are formed here, from an opaque copy of the
        // slot: hoisted out of the group loop they would hold registers
        // for all of it (and, spilled, their reloads would wait for every
        // load in flight)
        uint32_t slot = slot_;
        if constexpr (VT) asm volatile("" : "+v"(slot));
        if constexpr (VT) {
            const uint8_t *vb = value_part(page, meta);
            __builtin_amdgcn_global_load_lds(vb + (slot >> 4) * kV8Group + (slot & 15) * 4, &s.vs[w][0], 4, 0, 0);
        }
        const uint8_t *blk = arena + (size_t)meta.y * 16;
        const int tier = key_tier(meta.x & 0xFF);
        const uint8_t *c = blk + 2 * P + slot * 16;
        const bool t2 = tier == ADA_TIER_T2;
        const int so = (tier == ADA_TIER_T4) ? 32 * P : 64 * P;   // first magnitude unit
        const int o2 = t2 ? 16 * P : so;
        const int o3 = t2 ? 16 * P : so + 16 * P;
        CodeStage &st = s.st[w];
        __builtin_amdgcn_global_load_lds(c, &st.u[0][0], 16, 0, 0);
        __builtin_amdgcn_global_load_lds(c + 16 * P, &st.u[1][0], 16, 0, 0);
        __builtin_amdgcn_global_load_lds(c + o2, &st.u[2][0], 16, 0, 0);
        __builtin_amdgcn_global_load_lds(c + o3, &st.u[3][0], 16, 0, 0);
        __builtin_amdgcn_global_load_lds(t2 ? blk + 34 * P + (slot & ~1) * 8 : c, &st.h[0], 16, 0, 0);
        __builtin_amdgcn_global_load_lds(blk + 4 * (slot >> 1), &st.r[0], 4, 0, 0);
    }

    // The lane's code units from wavefront w's stage (after its loads
    // landed); with V8 pages, its token's four block scales go to the
    // wavefront's scale table, read after the weights' LDS sync.
    __device__ Codes unstage(Smem &s, int w, uint2 meta, int slot, int lane) const {
        const CodeStage &st = s.st[w];
        CodeRegs k;
#pragma unroll
        for (int u = 0; u < 4; ++u) k.u[u] = st.u[u][lane];
        const uint4 hh = st.h[lane];
        k.h = (slot & 1) ? make_uint2(hh.z, hh.w) : make_uint2(hh.x, hh.y);
        const uint32_t rr = st.r[lane];
        k.r = (slot & 1) ? rr >> 16 : rr & 0xFFFFu;
        if constexpr (VT) {
            const uint32_t word = s.vs[w][lane];
            const uint2 vs = core::v8_scale_halves(word);
            s.vsc[w][0][lane] = (uint16_t)vs.x;
            s.vsc[w][1][lane] = (uint16_t)(vs.x >> 16);
            s.vsc[w][2][lane] = (uint16_t)vs.y;
            s.vsc[w][3][lane] = (uint16_t)(vs.y >> 16);
            // every scale byte of a V8 token 0 or in the fused conversion's
            // range (other pages' words are not scales)
            bool out = false;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const uint32_t sb = (word >> (8 * kb)) & 0xFFu;
                out |= sb != 0 && (sb < core::kV8FmaMinScale || sb > core::kV8FmaMaxScale);
            }
            k.v8_fma = !__any(out && tier_v8(meta.x & 0xFF));
        }
        // the slot offset is made opaque here so that arena + slot offset (a
        // 64-bit per-lane value) is not hoisted out of the group loop, where
        // it would hold two more registers for the whole loop
        uint32_t soff = 2 * P + slot * 16;
        asm volatile("" : "+v"(soff));
        k.c = arena + (size_t)meta.y * 16 + soff;
        return k;
    }

    __device__ void logits(const Smem &s, const Codes &k, uint2 meta, bool valid, float (&lg)[G]) const {
        const int tier = key_tier(meta.x & 0xFF);
        if (__any(valid && tier == ADA_TIER_T4)) {
            if (valid && tier == ADA_TIER_T4) logits_t4<G>(k, s.lut4, mul, lg);
        }
        if (__any(valid && tier == ADA_TIER_T2)) {
            if (valid && tier == ADA_TIER_T2) logits_t2<G>(k, s.lut4, mul, lg);
        }
        if (__any(valid && tier == ADA_TIER_T8)) {
            if (valid && tier == ADA_TIER_T8) logits_t8<G, P>(k, s.cs8, s.q8, mul, lg);
        }
    }
};

// MODE: 0 plain, 1 fused append, 2 utility emission
// VT: the cache may hold V8-value pages (a separate instantiation, so that
// caches of fp16 tiers only run the kernel without the V8 paths)
template <int G, int P, int NW, int WPE, int MODE, bool VT>
__global__ __launch_bounds__(NW * 64, WPE) void decode_partials_kernel(DecodeLaunch a) {
    using Pol = AdaPolicy<G, P, NW, MODE == 1, VT>;
    constexpr size_t RED = (size_t)NW * G * 130 * sizeof(float);
    constexpr size_t RAW = sizeof(typename Pol::Smem) > RED ? sizeof(typename Pol::Smem) : RED;
    __shared__ __align__(16) unsigned char raw[RAW];   // policy tables, later the wave-merge buffer
    __shared__ core::CoreSmem<G, NW> cs;
    Pol pol;
    pol.num_pages_ = a.num_pages;
    pol.page_meta = a.page_meta;
    pol.arena = a.arena;
    pol.q = a.q;
    pol.Q = a.Q;
    pol.Hq = a.Hq;
    pol.Gr = a.Hq / a.Hkv;
    // grid x: the chunk, or for nslice > 1 (chunk, slice) with the slices of
    // a chunk 8 work-groups apart, i.e. on one of the chip's dies (work-groups
    // go to the dies in turn) and dispatched together: the second slice's
    // code and value reads can hit that die's L2 / the memory-side cache
    // the row: in the cache's order (longest rows first) when it is given,
    // so that the longest rows' work-groups are dispatched first
    int h = blockIdx.y, b = blockIdx.z;
    if (a.row_order) {
        const int r = a.row_order[blockIdx.z * a.Hkv + blockIdx.y];
        h = r % a.Hkv;
        b = r / a.Hkv;
    }
    int chunk = blockIdx.x, slice = 0;
    if (a.nslice > 1) {
        const int x = blockIdx.x;
        chunk = (x / (8 * a.nslice)) * 8 + x % 8;
        slice = (x / 8) % a.nslice;
        if (chunk >= a.S) return;
    }
    pol.voff = slice * G;
    pol.half = a.half_pairs;
    pol.app_page = a.app_page;
    pol.app_slot = a.app_slot;
    pol.app_keys = a.app_keys;
    pol.app_values = a.app_values;
    pol.arena_w = a.arena_w;
    pol.status = a.status;
    pol.mul = a.scale * core::kLog2e;
    core::CoreArgs c;
    c.page_table = a.page_table;
    c.pm = a.pm;
    c.pl = a.pl;
    c.pacc = a.pacc;
    c.Hq = a.Hq;
    c.Hkv = a.Hkv;
    c.maxp = a.maxp;
    c.chunk_pages = a.chunk_pages;
    c.S = a.S;
    c.logit_buf = a.logit_buf;
    c.gv = a.Q * pol.Gr;
    c.voff = pol.voff;
    core::split_k<G, P, NW, MODE == 2>(c, pol, *reinterpret_cast<typename Pol::Smem *>(raw), cs,
                            reinterpret_cast<float *>(raw), chunk, h, b);
}

// one work-group per virtual row (b, h, v); writes query qi = v / Gr, head
// h * Gr + v % Gr
__global__ __launch_bounds__(core::kReduceThreads) void decode_reduce_kernel(DecodeLaunch a) {
    const int vr = blockIdx.x;
    const int Gr = a.Hq / a.Hkv, GV = a.Q * Gr;
    const int b = vr / (a.Hkv * GV), rem = vr % (a.Hkv * GV);
    const int h = rem / GV, v = rem % GV;
    const size_t orow = ((size_t)b * a.Q + v / Gr) * a.Hq + (size_t)h * Gr + v % Gr;
    // the page count as a per-lane load (an opaque zero offset): waiting for
    // a scalar load would also wait for the launch arguments' loads, which
    // must land before the first partials are requested
    uint32_t z = 0;
    asm volatile("" : "+v"(z));
    const int np = a.num_pages[b * a.Hkv + h + z];
    core::reduce_chunks(a.pm, a.pl, a.pacc, a.S, core::chunks_with_data(np, 64 / a.P, a.S), (size_t)vr, orow,
                        threadIdx.x, a.out, a.lse);
}

// ---- utility pass ---------------------------------------------------------
// Attention mass of every kept token (the signal RDR consumes as "estimated
// future utility"): u = sum over the KV head's G query heads of
// exp2(logit2 - lse2), logit2 the stored base-2 logit, lse2 = lse * log2(e)
// from the reduction.  One work-group per (row, block of 64 pages).
constexpr int kUtilPages = 64;

template <int G>
__global__ __launch_bounds__(256) void decode_utility_kernel(DecodeLaunch a) {
    __shared__ int s_page[kUtilPages], s_count[kUtilPages];
    const int row = blockIdx.y, b = row / a.Hkv, h = row % a.Hkv;
    const int np = a.num_pages[row];
    const int p0 = blockIdx.x * kUtilPages;
    if (p0 >= np) return;
    const int npg = min(kUtilPages, np - p0);
    if (threadIdx.x < npg) {
        const int page = a.page_table[(size_t)row * a.maxp + p0 + threadIdx.x];
        s_page[threadIdx.x] = page;
        s_count[threadIdx.x] = a.page_meta[page].count;
    }
    float lse2[G];
#pragma unroll
    for (int g = 0; g < G; ++g) lse2[g] = a.lse[(size_t)b * a.Hq + (size_t)h * G + g] * core::kLog2e;
    __syncthreads();
    const int P = a.P, n = npg * P;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int pi = i / P, slot = i % P;
        if (slot >= s_count[pi]) continue;
        const size_t tok = (size_t)s_page[pi] * P + slot;
        const float *lg = a.logit_buf + tok * G;
        float u = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) u += exp2f(lg[g] - lse2[g]);
        a.util[tok] = u;
    }
}

// ---- stand-alone LUT builder --------------------------------------------
// qs holds the query's pairs as [x_0..x_63][y_0..y_63] in either layout.
__global__ __launch_bounds__(256) void build_lut_kernel(const float *q, float *lut, bool half) {
    __shared__ float2 cs8[256];
    __shared__ float qs[kD];
    const int rowq = blockIdx.x, tid = threadIdx.x;
    cs8[tid] = grid_dir(tid);
    if (tid < kD) qs[half ? tid : (tid & 1) * 64 + (tid >> 1)] = q[(size_t)rowq * kD + tid];
    __syncthreads();
    float *out = lut + (size_t)rowq * (64 * (256 + 16 + 4));
    for (int i = tid; i < 64 * 256; i += 256) {
        const int j = i >> 8, c = i & 255;
        out[i] = lut_entry(qs[j], qs[64 + j], cs8[c]);
    }
    out += 64 * 256;
    for (int i = tid; i < 64 * 16; i += 256) {
        const int j = i >> 4, c = i & 15;
        out[i] = lut_entry(qs[j], qs[64 + j], cs8[c * 16]);
    }
    out += 64 * 16;
    for (int i = tid; i < 64 * 4; i += 256) {
        const int j = i >> 2, c = i & 3;
        out[i] = lut_entry(qs[j], qs[64 + j], cs8[c * 64]);
    }
}

template <int G, int P, bool VT>
hipError_t launch_gpv(const DecodeLaunch &a, hipStream_t s) {
    constexpr int NW = 4;
    constexpr int WPE = decode_waves_per_simd(G);
    const int gx = a.nslice > 1 ? (a.S + 7) / 8 * 8 * a.nslice : a.S;
    const dim3 grid(gx, a.Hkv, a.B), block(NW * 64);
    if (a.app_page)
        hipLaunchKernelGGL((decode_partials_kernel<G, P, NW, WPE, 1, VT>), grid, block, 0, s, a);
    else if (a.logit_buf)
        hipLaunchKernelGGL((decode_partials_kernel<G, P, NW, WPE, 2, VT>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((decode_partials_kernel<G, P, NW, WPE, 0, VT>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int G>
hipError_t launch_g(const DecodeLaunch &a, hipStream_t s) {
    if (a.value_tiers) return a.P == 16 ? launch_gpv<G, 16, true>(a, s) : launch_gpv<G, 32, true>(a, s);
    return a.P == 16 ? launch_gpv<G, 16, false>(a, s) : launch_gpv<G, 32, false>(a, s);
}

}  // namespace

hipError_t launch_decode_partials(const DecodeLaunch &a, hipStream_t s) {
    switch (slice_heads(a.Q * (a.Hq / a.Hkv))) {   // virtual heads per work-group
        case 1: return launch_g<1>(a, s);
        case 2: return launch_g<2>(a, s);
        case 4: return launch_g<4>(a, s);
        case 8: return launch_g<8>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_reduce(const DecodeLaunch &a, hipStream_t s) {
    hipLaunchKernelGGL(decode_reduce_kernel, dim3(a.B * a.Q * a.Hq), dim3(kD * core::reduce_groups(a.S)), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_decode_utility(const DecodeLaunch &a, hipStream_t s) {
    const dim3 grid((a.maxp + kUtilPages - 1) / kUtilPages, a.B * a.Hkv), block(256);
    switch (a.Hq / a.Hkv) {
        case 1: hipLaunchKernelGGL(decode_utility_kernel<1>, grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL(decode_utility_kernel<2>, grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL(decode_utility_kernel<4>, grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL(decode_utility_kernel<8>, grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_build_lut(const float *q, int32_t rows, float *lut, bool half_pairs, hipStream_t s) {
    hipLaunchKernelGGL(build_lut_kernel, dim3(rows), dim3(256), 0, s, q, lut, half_pairs);
    return hipGetLastError();
}

}  // namespace ada
