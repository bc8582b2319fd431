// decode_core.h -- split-K paged decode skeleton shared by the ADA decode and
// the dense fp16 reference decode (they differ only in how logits are made).
//
// One work-group = one (context chunk, KV head, sequence).  Prologue: the
// chunk's page ids and page metadata are staged in LDS (so the per-group
// critical path has no dependent global loads before the code fetch), and
// the policy stages its per-query tables.  The prologue is two memory round
// trips (page count, page ids and query; then page metadata), after which
// each wavefront requests its first group's codes.  Then each wavefront walks 64-token
// groups (4 pages of 16 / 2 pages of 32):
//   1. the tokens' codes (lane = token, policy); a staged policy has them
//      requested into LDS one group ahead;
//   2. logits for the G query heads, lane = token (policy);
//   3. issue the group's value loads (16 x 128-bit per lane): each lane gets
//      8 consecutive tokens of one head dimension, which is exactly the A
//      operand of v_mfma_f32_16x16x32_f16 (value pages are stored in 8-token
//      groups, dimension-major).  They are issued after the logit arithmetic
//      so they are not held in registers through it;
//   4. online softmax per head: wavefront max, exp2, running sums; the
//      weights are written to LDS as fp16 hi + lo parts (p ~ hi + lo to
//      about 2^-22 relative), head-major;
//   5. value accumulation O^T[dims x heads] += V^T[dims x 32 tokens] .
//      P^T[32 tokens x heads] on the matrix cores: 8 dimension tiles of 16,
//      two 32-token K steps, hi and lo weights -> 32 MFMAs per group.  This
//      product is a genuine dense contraction; the logit path is not.
// The waves of the work-group are merged in LDS and one partial (running
// max, running sum, unnormalised accumulator) per (query head, chunk) is
// written; a reduction pass combines the chunks.
#pragma once

#include "ada_internal.h"

namespace ada {
namespace core {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
// Lazy running maximum of the online softmax (base-2 logits): weights are
// taken against a maximum at most this far below the largest logit seen.
constexpr float kLazyMax = 8.0f;

// DPP lane permutation of a float (row_mask and bank_mask all on)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// +inf in a scalar register, hidden from the optimiser (see max2).
__device__ __forceinline__ float opaque_inf() {
    float x = INFINITY;
    asm volatile("" : "+s"(x));
    return x;
}

// max(a, b).  MED3: as the median of a, b and +inf (`inf` from
// opaque_inf), one v_med3_f32.  fmaxf -- and a median with a literal
// infinity, which the optimiser turns back into it -- first quiets operands
// that come from a lane permutation or a readlane (the kernels run in IEEE
// mode): two more instructions per step.  Measured: the median form is the
// faster one with eight query heads per KV head, fmaxf with four or fewer.
// Operands here are logits or -inf, never NaN.
template <bool MED3>
__device__ __forceinline__ float max2(float a, float b, float inf) {
    if constexpr (MED3) return __builtin_amdgcn_fmed3f(a, b, inf);
    else return fmaxf(a, b);
}

// Wavefront maximum on the VALU: within each row of 16 lanes by DPP (quad
// xor 1, quad xor 2, half-row mirror, row mirror), then across the four
// rows by reading one lane of each.  The result is wave-uniform.
template <bool MED3>
__device__ __forceinline__ float wave_max(float v, float inf) {
    v = max2<MED3>(v, dpp_f<0xB1>(v), inf);    // quad_perm(1, 0, 3, 2)
    v = max2<MED3>(v, dpp_f<0x4E>(v), inf);    // quad_perm(2, 3, 0, 1)
    v = max2<MED3>(v, dpp_f<0x141>(v), inf);   // row_half_mirror
    v = max2<MED3>(v, dpp_f<0x140>(v), inf);   // row_mirror
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return max2<MED3>(max2<MED3>(r0, r1, inf), max2<MED3>(r2, r3, inf), inf);
}

// V8 values -> fp16 MFMA operand.
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// A token's four scale bytes s (one per dimension block) -> the fp16 factors
// 2^(s - 133), packed [block 0 | block 1] and [block 2 | block 3]: exact (the
// fp32 bits (s - 6) << 23 are that power of two, an fp16 number since
// s >= 109).  The zero byte of an empty slot gives 0, so that its zero code
// bytes (c = -128) give a zero value.
__device__ __forceinline__ uint2 v8_scale_halves(uint32_t word) {
    float f[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t b = (word >> (8 * k)) & 0xFFu;
        f[k] = b ? __builtin_bit_cast(float, (b - 6u) << 23) : 0.f;
    }
    return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f[0], f[1])),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f[2], f[3])));
}

// two tokens' code bytes u = c + 128 (bytes b and b + 1 of w, b = 0 or 2)
// times their scale pair: two fp16 values of the MFMA A operand.  The
// permute forms the halves 0x6400 | u = 1152 + c, so subtracting 1152 gives
// c exactly; the product with a power of two is exact.
template <int B>
__device__ __forceinline__ uint32_t v8_pair(uint32_t w, uint32_t scale_pair) {
    constexpr uint32_t sel = B == 0 ? 0x04010400u : 0x04030402u;   // [b, 0x64, b + 1, 0x64]
    const uint32_t x = __builtin_amdgcn_perm(0x64646464u, w, sel);
    const half2_t c = __builtin_bit_cast(half2_t, x) - half2_t{(_Float16)1152.0f, (_Float16)1152.0f};
    return __builtin_bit_cast(uint32_t, c * __builtin_bit_cast(half2_t, scale_pair));
}

// The fused conversion below needs each block scale 2^(s - 133) as a
// normal fp16 number at most 2^5: s in [kV8FmaMinScale, kV8FmaMaxScale]
// (or 0, an empty slot, whose weight is 0).  Its bias -1152 * 2^(s - 133)
// = -1.125 * 2^(s - 123) then has the scale's fp16 bits plus 0xA880: the
// sign, ten more in the exponent field, mantissa 0x080 (no carry into the
// next half, so a scale pair becomes its bias pair in one integer add).
constexpr uint32_t kV8FmaMinScale = 119, kV8FmaMaxScale = 138;
constexpr uint32_t kV8BiasAdd = 0xA880A880u;

// v8_pair in one fused multiply-add: (1152 + c) * s + (-1152 * s) is c * s
// exactly (a small integer times a power of two, rounded once), the same
// bits as the subtract-then-multiply form, for scales in the range above.
template <int B>
__device__ __forceinline__ uint32_t v8_pair_fma(uint32_t w, uint32_t scale_pair, uint32_t bias_pair) {
    constexpr uint32_t sel = B == 0 ? 0x04010400u : 0x04030402u;   // [b, 0x64, b + 1, 0x64]
    const uint32_t x = __builtin_amdgcn_perm(0x64646464u, w, sel);
    const half2_t v = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, x), __builtin_bit_cast(half2_t, scale_pair),
                                                __builtin_bit_cast(half2_t, bias_pair));
    return __builtin_bit_cast(uint32_t, v);
}

// Wavefront sum in the same pattern (a fixed order, identical in every lane).
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x140>(v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (r0 + r1) + (r2 + r3);
}


// LDS writes by one lane become visible to the other lanes of its wavefront.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T>
__device__ __forceinline__ T ldg(const void *p) {
    return *reinterpret_cast<const T *>(p);
}

// Shared arguments of a split-K pass.
struct CoreArgs {
    const int32_t *page_table;
    float *pm, *pl, *pacc;
    int32_t Hq, Hkv, maxp, chunk_pages, S;
    float *logit_buf;   // EMIT: [page * P + slot][G] base-2 logits of every kept token
    // virtual heads per KV head (partial rows of a KV head) and the first of
    // the G this work-group computes (several queries per sequence: slices of
    // at most 8 virtual heads go to different work-groups)
    int32_t gv, voff;
};

template <int G, int NW>
struct CoreSmem {
    int pages[kMaxChunkPages];
    uint2 meta[kMaxChunkPages];
    _Float16 pb[NW][2][G][64];   // [wave][hi|lo][head][token]
};

// Reduction pass.  A work-group per (sequence, query head): kD threads per
// group, one per dimension, and up to kReduceGroups groups (blockDim.x / kD,
// chosen by the launch from the chunk count).  Group q merges the chunk
// tiles q, q + groups, ... (kReduceTile chunks each) with all of a tile's
// loads issued before any arithmetic; the groups' results are then merged
// in group order through LDS.  The first tile of each group is requested
// before the row's chunk count nc is known (its slots past nc hold nothing
// of this launch and are masked), so rows of up to groups * kReduceTile
// chunks cost one round trip in all.  The order is fixed: deterministic.
constexpr int kReduceTile = 16;
constexpr int kReduceGroups = 4;
constexpr int kReduceThreads = kD * kReduceGroups;   // the largest work-group
__host__ __device__ constexpr int reduce_groups(int S) {
    return S <= kReduceTile ? 1 : (S <= 2 * kReduceTile ? 2 : kReduceGroups);
}

// prow: partial row, orow: output row
__device__ __forceinline__ void reduce_chunks(const float *pm, const float *pl, const float *pacc, int S, int nc,
                                              size_t prow, size_t orow, int tid, float *out, float *lse) {
    __shared__ float gm[kReduceGroups][kD], gl[kReduceGroups][kD], go[kReduceGroups][kD];
    const int d = tid % kD, q = tid / kD, groups = blockDim.x / kD;
    const size_t base = prow * S;
    float M = -INFINITY, L = 0.f, O = 0.f;
    float mv[kReduceTile], lv[kReduceTile], av[kReduceTile];
    // merges chunks c0 .. c0 + kReduceTile - 1 below nc from mv / lv / av
    // (branch-free, so the tile's loads are not held back behind a test:
    // while no chunk had a kept token, M = -inf and L = O = 0 stay so)
    auto merge = [&](int c0) {
        float Mt = M;
#pragma unroll
        for (int i = 0; i < kReduceTile; ++i)
            if (c0 + i < nc) Mt = fmaxf(Mt, mv[i]);
        const float so = (M == -INFINITY) ? 0.f : exp2f(M - Mt);
        L *= so;
        O *= so;
#pragma unroll
        for (int i = 0; i < kReduceTile; ++i) {
            if (c0 + i < nc && mv[i] != -INFINITY) {   // masked slots may hold anything
                const float f = exp2f(mv[i] - Mt);
                L = fmaf(lv[i], f, L);
                O = fmaf(av[i], f, O);
            }
        }
        M = Mt;
    };
    // the chunk scalars as per-lane loads (an opaque zero offset), so that
    // the whole first tile is in flight before the chunk count arrives
    uint32_t z = 0;
    asm volatile("" : "+v"(z));
#pragma unroll
    for (int i = 0; i < kReduceTile; ++i) {
        const int c = min(q * kReduceTile + i, S - 1);   // a slot of the row's S; chunks at or past nc are masked
        mv[i] = pm[base + c + z];
        lv[i] = pl[base + c + z];
        av[i] = pacc[(base + c) * kD + d];
    }
    __builtin_amdgcn_sched_barrier(0);   // every load above is issued before the merge starts
    merge(q * kReduceTile);
    for (int c0 = (q + groups) * kReduceTile; c0 < nc; c0 += groups * kReduceTile) {
#pragma unroll
        for (int i = 0; i < kReduceTile; ++i) {
            const int c = min(c0 + i, nc - 1);   // in range; repeats are masked
            mv[i] = pm[base + c + z];
            lv[i] = pl[base + c + z];
            av[i] = pacc[(base + c) * kD + d];
        }
        merge(c0);
    }
    if (groups > 1) {   // the groups' results, merged in group order by group 0
        gm[q][d] = M;
        gl[q][d] = L;
        go[q][d] = O;
        __syncthreads();
        if (q != 0) return;
        for (int g = 1; g < groups; ++g) {
            const float Mg = gm[g][d];
            if (Mg == -INFINITY) continue;
            const float Mt = fmaxf(M, Mg);
            const float so = (M == -INFINITY) ? 0.f : exp2f(M - Mt), sg = exp2f(Mg - Mt);
            L = L * so + gl[g][d] * sg;
            O = O * so + go[g][d] * sg;
            M = Mt;
        }
    }
    if (M == -INFINITY) {
        out[orow * kD + d] = 0.f;
        if (lse && d == 0) lse[orow] = -INFINITY;
        return;
    }
    out[orow * kD + d] = O / L;
    if (lse && d == 0) lse[orow] = (M + log2f(L)) * 0.69314718055994531f;
}

// Policy interface (see decode.hip / dense.hip):
//   Smem                      policy LDS (per-query tables)
//   int num_pages(row, b)     pages in the row
//   int num_pages_lane(row, b, z)  the same as a per-lane load (z an opaque
//                             zero), so that it travels with the page-table
//                             loads of the prologue's first round trip
//   uint2 meta(page, idx, b)  x = tier | count << 8, y = policy data
//   const uint8_t *value_part(page, meta)   the page's values: fp16 pages
//                                           in 8-token groups of [128 dims]
//                                           [8 tokens]; V8 pages as in
//                                           ada_internal.h
//   void prologue(smem, b, h, tid, nthreads)   stores before a barrier
//   void build(smem, tid, nthreads)            tables after that barrier
//   bool after_pages(smem, pages, n, row, w, lane)  work before any page of
//                                              the chunk is read; returns
//                                              (uniformly) whether a barrier
//                                              must follow
//   kValueTiers: pages of tiers 3-5 hold V8 values (see include/ada.h)
//     codes.v8_fma                              wave-uniform: every V8 token of
//                                              the group has its block scales
//                                              in the fused conversion's range
//     void scale_pairs(smem, w, tok, b, sp[4])  fp16 scales of dimension
//                                              block b of tokens tok ..
//                                              tok + 7 of the current group,
//                                              in pairs of tokens (after the
//                                              weights' LDS sync)
//   kEarlyStage: the first group's codes may be requested before
//     after_pages (from the registers that fetched its page ids), i.e.
//     before the prologue's barriers
//   kStaged = true:
//     void stage(smem, w, meta, page, slot)    request a group's codes (and
//                                              V8 scale words) into
//                                              wavefront w's LDS stage
//     Codes unstage(smem, w, meta, slot, lane) read them (after they landed)
//   kStaged = false:
//     Codes fetch(page, meta, slot, valid)     issue the token's code loads
//   void logits(smem, codes, meta, valid, lg[G]) lane = token, base-2 scaled
template <int G, int P, int NW, bool EMIT, class Pol>
__device__ __forceinline__ void split_k(const CoreArgs &a, const Pol &pol, typename Pol::Smem &ps,
                                        CoreSmem<G, NW> &cs, float *red, int chunk, int h, int b) {
    constexpr int TPG = 64 / P;     // pages per group
    constexpr int KB = P / 8;       // 8-token value blocks per page
    constexpr int NT = NW * 64;
    const int row = b * a.Hkv + h;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    static_assert(NT >= kMaxChunkPages, "one page-list entry per thread");
    // an upper bound of the chunk's page slots from the row capacity
    const int ngr_cap = (a.maxp + TPG - 1) / TPG;
    if (chunk >= ngr_cap) return;
    const int nch_cap = (ngr_cap - chunk + a.S - 1) / a.S * TPG;
    const int32_t *ptab = a.page_table + (size_t)row * a.maxp;
    // round trip 1: the row's page count (a per-lane load), the page ids of
    // the chunk's slots up to the capacity bound, the page ids of this
    // wavefront's first group, and the query
    uint32_t z = 0;
    asm volatile("" : "+v"(z));
    const int np_l = pol.num_pages_lane(row, b, z);
    const int pslot = (chunk + (tid / TPG) * a.S) * TPG + tid % TPG;   // page index of this thread's slot
    int praw = -1;
    if (tid < nch_cap && pslot < a.maxp) praw = ptab[pslot];
    const int pf = (chunk + w * a.S) * TPG;          // first page of this wavefront's first group
    const int pl = pf + lane / P;                    // this lane's page of it
    int pg_own = -1, pg_first = -1;
    const bool has_first = pf < a.maxp;
    if (has_first) {
        pg_first = ptab[pf];
        if (pl < a.maxp) pg_own = ptab[pl];
    }
    pol.prologue(ps, b, h, tid, NT);   // query loads (stored to LDS below their wait)
    const int np = __builtin_amdgcn_readfirstlane(np_l);
    // chunk c owns the row's 64-token page groups c, c + S, c + 2S, ...: the
    // work-groups running at the same time stream neighbouring pages
    const int ngr_row = (np + TPG - 1) / TPG;
    if (chunk >= ngr_row) return;
    const int ngr = (ngr_row - chunk + a.S - 1) / a.S;   // groups of this chunk
    const int nch = ngr * TPG;                           // page slots of this chunk
    const int n_groups = (nch + TPG - 1) / TPG;
    const int pg = lane / P, slot = lane % P;
    // round trip 2: page metadata of the slots and of the first group's pages
    int page = -1;
    uint2 m = make_uint2(0u, 0u);
    if (tid < nch && pslot < np) {
        page = praw;
        m = pol.meta(page, pslot, b);
    }
    int fpage = 0;
    uint2 fmeta = make_uint2(0u, 0u);
    const bool first = w < n_groups;   // wave-uniform
    if (first) {
        fpage = pl < np ? pg_own : pg_first;   // lanes past the row's last page use the group's first page
        fmeta = pol.meta(fpage, pl, b);
    }
    if constexpr (Pol::kStaged && Pol::kEarlyStage) {
        if (first) pol.stage(ps, w, fmeta, fpage, slot);
    }
    if (tid < nch) {
        cs.pages[tid] = page;
        cs.meta[tid] = m;
    }
    __syncthreads();
    // policy work that must precede every code / value read of the chunk
    // (the fused append writes the row's new token into its slot)
    if (pol.after_pages(ps, cs.pages, nch, row, w, lane)) __syncthreads();
    // the group's page for this lane (lane = token); lanes past the row's
    // last page use the group's first page (weight 0)
    auto group_meta = [&](int g, bool &valid) {
        const int gbase = g * TPG;
        const int pidx = gbase + pg;
        const bool pvalid = cs.pages[pidx] >= 0;
        const uint2 meta = cs.meta[pvalid ? pidx : gbase];
        valid = pvalid && slot < (int)((meta.x >> 8) & 0xFF);
        return meta;
    };
    auto group_page = [&](int g) {
        const int gbase = g * TPG;
        return cs.pages[gbase + pg] >= 0 ? cs.pages[gbase + pg] : cs.pages[gbase];
    };
    // staged policies whose first reads may not start before after_pages:
    // the first group's code units are requested here, before the tables
    // are built
    if constexpr (Pol::kStaged && !Pol::kEarlyStage) {
        if (w < n_groups) {
            bool v;
            const uint2 m0 = group_meta(w, v);
            pol.stage(ps, w, m0, group_page(w), slot);
        }
    }
    pol.build(ps, tid, NT);
    __syncthreads();

    float m_run[G], l_run[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m_run[g] = -INFINITY;
        l_run[g] = 0.f;
    }
    floatx4_t acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    const int n_head = lane & 15;       // MFMA column = query head of this lane
    const int kq = lane >> 4;           // MFMA K quarter: tokens 8*kq .. 8*kq + 7 of a 32-token step

    for (int grp = w; grp < n_groups; grp += NW) {
        asm volatile("" ::: "memory");   // keep LDS reads of the tables inside the loop
        const int gbase = grp * TPG;

        // 1. the tokens' code units (lane = token).  Staged: this group's were
        //    requested into LDS one iteration earlier; once copied to
        //    registers the next group's are requested, so their latency
        //    overlaps this group's logits, values and softmax.
        bool valid;
        const uint2 meta = group_meta(grp, valid);
        typename Pol::Codes codes;
        if constexpr (Pol::kStaged) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");     // the stage has landed
            codes = pol.unstage(ps, w, meta, slot, lane);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // read before it is refilled
            if (grp + NW < n_groups) {
                bool vn;
                const uint2 mn = group_meta(grp + NW, vn);
                pol.stage(ps, w, mn, group_page(grp + NW), slot);
            }
        } else {
            const int pidx = gbase + pg;
            const int page = cs.pages[pidx] >= 0 ? cs.pages[pidx] : cs.pages[gbase];
            codes = pol.fetch(page, meta, slot, valid);
        }

        // 2. logits, lane = token
        float lg[G];
#pragma unroll
        for (int g = 0; g < G; ++g) lg[g] = -INFINITY;
        pol.logits(ps, codes, meta, valid, lg);
        if constexpr (EMIT) {   // keep the token's logits for the utility pass
            if (valid) {
                // a 32-bit element offset formed here: a 64-bit per-lane base
                // hoisted out of the loop costs registers the loop needs
                const uint32_t off = ((uint32_t)cs.pages[gbase + pg] * P + slot) * G;
                float *dst = a.logit_buf + off;
                // streaming (non-temporal) stores: read back once by the
                // utility pass, they should not displace cached lines
#pragma unroll
                for (int g = 0; g < G; ++g) __builtin_nontemporal_store(lg[g], dst + g);
            }
        }

        // 3. values -> MFMA A operands, issued after the logit arithmetic so
        //    they are not held in registers through it (other wavefronts'
        //    work covers their latency).  The K index of the MFMAs is
        //    permuted: lane (n_head, kq) takes tokens 16 kq .. 16 kq + 15 of
        //    the group, the first eight at step kc = 0, the others at kc = 1,
        //    so that its tokens are consecutive slots of one page.  A lane
        //    past the row's last page reads the group's first page instead
        //    (weight 0).  fp16 page: 16 bytes (8 tokens of one dimension) per
        //    tile and step; V8 page: 8 code bytes per tile and step, converted
        //    before the MFMAs.
        uint4 va[2][8];
        bool v8 = false;
        {
            // the lane's place in the MFMA operands, made opaque here so that
            // the per-lane value offsets are formed in the loop rather than
            // hoisted out of it (they would hold registers for all of it)
            uint32_t ln = lane;
            if constexpr (Pol::kValueTiers) asm volatile("" : "+v"(ln));
            const int vq = ln >> 4, vh = ln & 15;   // kq, n_head
            const int vslot = gbase + (16 * vq) / P;
            const int pidx = cs.pages[vslot] >= 0 ? vslot : gbase;
            const uint2 vmeta = cs.meta[pidx];
            const uint8_t *vpart = pol.value_part(cs.pages[pidx], vmeta);
            const int tok = (16 * vq) % P;           // the lane's first slot in that page
            if constexpr (Pol::kValueTiers) v8 = tier_v8(vmeta.x & 0xFF);
            // V8 page: the 16 code bytes of the lane's dimension (its 16
            // tokens, both steps) per tile, one read into va[0]; va[1] is
            // formed from it by the conversion
            const uint8_t *b8 = vpart + (tok / 16) * kV8Group + kV8Codes + vh * 16;
            const uint8_t *b16 = vpart + (tok / 8) * 2048 + vh * 16;
            const uint8_t *base = v8 ? b8 : b16;
#pragma unroll
            for (int t = 0; t < 8; ++t) va[0][t] = ldg<uint4>(base + t * 256);
            if (!v8) {
#pragma unroll
                for (int t = 0; t < 8; ++t) va[1][t] = ldg<uint4>(b16 + 2048 + t * 256);
            }
        }

        // 4. online softmax, weights to LDS as fp16 hi + lo.  A head's
        //    running maximum moves only when one of the group's logits
        //    passes it by more than kLazyMax (base 2); otherwise the weights
        //    are taken against the maximum already held (so at most
        //    2^kLazyMax, within fp16 and its hi + lo split) and the group
        //    needs neither wavefront maxima nor a rescale of the sums.
        bool grow = false;
        if constexpr (G >= 8) {
#pragma unroll
            for (int g = 0; g < G; ++g) grow |= valid && lg[g] > m_run[g] + kLazyMax;
        }
        // (eight heads: the wavefront maxima are a large share of the VALU work;
        // at four or fewer the branch costs registers the loop needs)
        if (G < 8 || __any(grow)) {
            float alpha_n = 1.f;
            const float pinf = opaque_inf();
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float mx = wave_max<(G >= 8)>(valid ? lg[g] : -INFINITY, pinf);
                const float mnew = max2<(G >= 8)>(m_run[g], mx, pinf);
                // v_exp_f32 directly: arguments are <= 0, results below 2^-126
                // flush to zero, far below the weights' resolution
                const float alpha = (m_run[g] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[g] - mnew);
                const float p = valid ? __builtin_amdgcn_exp2f(lg[g] - mnew) : 0.f;
                l_run[g] = l_run[g] * alpha + p;
                m_run[g] = mnew;
                const _Float16 hi = (_Float16)p;
                const _Float16 lo = (_Float16)(p - (float)hi);
                cs.pb[w][0][g][lane] = hi;
                cs.pb[w][1][g][lane] = lo;
                if (n_head == g) alpha_n = alpha;
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) acc[t] *= alpha_n;
        } else {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                // arguments at most kLazyMax; an invalid lane's weight is 0
                const float p = valid ? __builtin_amdgcn_exp2f(lg[g] - m_run[g]) : 0.f;
                l_run[g] += p;
                const _Float16 hi = (_Float16)p;
                const _Float16 lo = (_Float16)(p - (float)hi);
                cs.pb[w][0][g][lane] = hi;
                cs.pb[w][1][g][lane] = lo;
            }
        }
        wave_lds_sync();

        // 5. O^T += V^T P^T on the matrix cores.  V8 lanes first turn codes
        //    x scales into fp16: tile t's bytes 0-7 into va[0][t] (step 0),
        //    bytes 8-15 into va[1][t] (step 1); tiles 2k, 2k + 1 use
        //    dimension block k, whose scales for a step's eight tokens come
        //    from the policy's scale table in one read.
        if constexpr (Pol::kValueTiers) {
            if (v8 && codes.v8_fma) {   // every block scale of the group's V8 tokens at most 2^5
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    uint32_t s0[4], s1[4], b0[4], b1[4];
                    pol.scale_pairs(ps, w, 16 * kq, kb, s0);
                    pol.scale_pairs(ps, w, 16 * kq + 8, kb, s1);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        b0[i] = s0[i] + kV8BiasAdd;
                        b1[i] = s1[i] + kV8BiasAdd;
                    }
#pragma unroll
                    for (int t = 2 * kb; t < 2 * kb + 2; ++t) {
                        const uint4 c = va[0][t];
                        va[1][t] = make_uint4(v8_pair_fma<0>(c.z, s1[0], b1[0]), v8_pair_fma<2>(c.z, s1[1], b1[1]),
                                              v8_pair_fma<0>(c.w, s1[2], b1[2]), v8_pair_fma<2>(c.w, s1[3], b1[3]));
                        va[0][t] = make_uint4(v8_pair_fma<0>(c.x, s0[0], b0[0]), v8_pair_fma<2>(c.x, s0[1], b0[1]),
                                              v8_pair_fma<0>(c.y, s0[2], b0[2]), v8_pair_fma<2>(c.y, s0[3], b0[3]));
                    }
                }
            } else if (v8) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    uint32_t s0[4], s1[4];   // scale pairs of tokens (2i, 2i + 1), block kb, steps 0 and 1
                    pol.scale_pairs(ps, w, 16 * kq, kb, s0);
                    pol.scale_pairs(ps, w, 16 * kq + 8, kb, s1);
#pragma unroll
                    for (int t = 2 * kb; t < 2 * kb + 2; ++t) {
                        const uint4 c = va[0][t];
                        va[1][t] = make_uint4(v8_pair<0>(c.z, s1[0]), v8_pair<2>(c.z, s1[1]),
                                              v8_pair<0>(c.w, s1[2]), v8_pair<2>(c.w, s1[3]));
                        va[0][t] = make_uint4(v8_pair<0>(c.x, s0[0]), v8_pair<2>(c.x, s0[1]),
                                              v8_pair<0>(c.y, s0[2]), v8_pair<2>(c.y, s0[3]));
                    }
                }
            }
        }
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            half8_t bh = {}, bl = {};
            if (n_head < G) {
                bh = *reinterpret_cast<const half8_t *>(&cs.pb[w][0][n_head][16 * kq + 8 * kc]);
                bl = *reinterpret_cast<const half8_t *>(&cs.pb[w][1][n_head][16 * kq + 8 * kc]);
            }
#pragma unroll
            for (int t = 0; t < 8; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, va[kc][t]), bh, acc[t], 0, 0, 0);
#pragma unroll
            for (int t = 0; t < 8; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, va[kc][t]), bl, acc[t], 0, 0, 0);
        }
        wave_lds_sync();
    }

    // merge the wavefronts of the work-group, write this chunk's partial
#pragma unroll
    for (int g = 0; g < G; ++g) l_run[g] = wave_sum(l_run[g]);
    __syncthreads();   // LDS tables are dead from here on; `red` may alias them
    // red: [w][g][130] = m, l, acc[128]; lane holds dims 16t + 4kq + j of head n_head
    if (n_head < G) {
        float *rr = red + (w * G + n_head) * 130 + 2;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) rr[16 * t + 4 * kq + j] = acc[t][j];
    }
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            red[(w * G + g) * 130] = m_run[g];
            red[(w * G + g) * 130 + 1] = l_run[g];
        }
    }
    __syncthreads();
    const size_t bq0 = ((size_t)b * a.Hkv + h) * a.gv + a.voff;   // first partial row of this work-group
    for (int i = tid; i < G * kD; i += NT) {
        const int g = i >> 7, d = i & 127;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, red[(ww * G + g) * 130]);
        float o = 0.f, L = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const float mw = red[(ww * G + g) * 130];
            const float f = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
            o = fmaf(red[(ww * G + g) * 130 + 2 + d], f, o);
            L = fmaf(red[(ww * G + g) * 130 + 1], f, L);
        }
        const size_t pidx = (bq0 + g) * a.S + chunk;
        a.pacc[pidx * kD + d] = o;
        if (d == 0) {
            a.pm[pidx] = M;
            a.pl[pidx] = L;
        }
    }
}

// number of chunks holding data for a row of np pages (page groups of tpg)
__device__ __forceinline__ int chunks_with_data(int np, int tpg, int S) { return min(S, (np + tpg - 1) / tpg); }

}  // namespace core
}  // namespace ada
