// decode_core.h -- split-K paged decode skeleton shared by the ADA decode and
// the dense fp16 reference decode (they differ only in how logits are made).
//
// One work-group = one (context chunk, KV head, sequence).  Prologue: the
// chunk's page ids and page metadata are staged in LDS (so the per-group
// critical path has no dependent global loads before the code fetch), and
// the policy stages its per-query tables.  Then each wavefront walks 64-token
// groups (4 pages of 16 / 2 pages of 32):
//   1. fetch the tokens' codes (lane = token, policy);
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

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
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
    const uint16_t *value_pool;
    float *pm, *pl, *pacc;
    int32_t Hq, Hkv, maxp, chunk_pages, S;
};

template <int G, int NW>
struct CoreSmem {
    int pages[kMaxChunkPages];
    uint2 meta[kMaxChunkPages];
    _Float16 pb[NW][2][G][64];   // [wave][hi|lo][head][token]
};

// Policy interface (see decode.hip / dense.hip):
//   Smem                      policy LDS (per-query tables)
//   int num_pages(row, b)     pages in the row
//   uint2 meta(page, idx, b)  x = tier | count << 8, y = policy data
//   void prologue(smem, b, h, tid, nthreads)
//   Codes fetch(page, meta, slot, valid)        issue the token's code loads
//   void logits(smem, codes, meta, valid, lg[G]) lane = token, base-2 scaled
template <int G, int P, int NW, int PF, class Pol>
__device__ __forceinline__ void split_k(const CoreArgs &a, const Pol &pol, typename Pol::Smem &ps,
                                        CoreSmem<G, NW> &cs, float *red, int chunk, int h, int b) {
    constexpr int TPG = 64 / P;     // pages per group
    constexpr int KB = P / 8;       // 8-token value blocks per page
    constexpr int NT = NW * 64;
    const int row = b * a.Hkv + h;
    const int np = pol.num_pages(row, b);
    // chunk c owns the row's 64-token page groups c, c + S, c + 2S, ...: the
    // work-groups running at the same time stream neighbouring pages
    const int ngr_row = (np + TPG - 1) / TPG;
    if (chunk >= ngr_row) return;
    const int ngr = (ngr_row - chunk + a.S - 1) / a.S;   // groups of this chunk
    const int nch = ngr * TPG;                           // page slots of this chunk
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int32_t *ptab = a.page_table + (size_t)row * a.maxp;
    for (int i = tid; i < nch; i += NT) {
        const int p = (chunk + (i / TPG) * a.S) * TPG + i % TPG;   // page index in the row
        int page = -1;
        uint2 m = make_uint2(0u, 0u);
        if (p < np) {
            page = ptab[p];
            m = pol.meta(page, p, b);
        }
        cs.pages[i] = page;
        cs.meta[i] = m;
    }
    pol.prologue(ps, b, h, tid, NT);
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

    const int n_groups = (nch + TPG - 1) / TPG;
    const int pg = lane / P, slot = lane % P;
    struct Tok {
        typename Pol::Codes codes;
        uint2 meta;
        bool valid;
    };
    // the tokens' code units of group g (lane = token); lanes past the row's
    // last page read the group's first page (weight 0)
    auto stage = [&](int g) {
        const int gbase = g * TPG;
        const int pidx = gbase + pg;
        const int page_raw = cs.pages[pidx];
        const bool pvalid = page_raw >= 0;
        const int page = pvalid ? page_raw : cs.pages[gbase];
        Tok t;
        t.meta = cs.meta[pvalid ? pidx : gbase];
        t.valid = pvalid && slot < (int)((t.meta.x >> 8) & 0xFF);
        t.codes = pol.fetch(page, t.meta, slot, t.valid);
        return t;
    };
    // the group's value blocks -> MFMA A operands; a block past the row's
    // last page is read from the group's first page instead (weight 0)
    auto load_values = [&](int g, uint4 (&va)[2][8]) {
        const int gb = g * TPG;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            const int blk = 4 * kc + kq;            // 8-token block of the group
            const int vpage = cs.pages[gb + blk / KB];
            const uint16_t *base =
                a.value_pool + (size_t)(vpage >= 0 ? vpage : cs.pages[gb]) * P * kD + (blk % KB) * 1024 + n_head * 8;
#pragma unroll
            for (int t = 0; t < 8; ++t) va[kc][t] = ldg<uint4>(base + t * 128);
        }
    };
    Tok nxt{};
    uint4 va_nxt[2][8];
    if (PF >= 1 && w < n_groups) nxt = stage(w);
    if (PF == 2 && w < n_groups) load_values(w, va_nxt);
    for (int grp = w; grp < n_groups; grp += NW) {
        asm volatile("" ::: "memory");   // keep LDS reads of the tables inside the loop

        // 1. the tokens' code units; with PF the next group's codes (and with
        //    PF = 2 its values) are issued now, this group's one iteration
        //    earlier
        Tok cur;
        uint4 va[2][8];
        if constexpr (PF >= 1) {
            cur = nxt;
            if constexpr (PF == 2) {
#pragma unroll
                for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                    for (int t = 0; t < 8; ++t) va[kc][t] = va_nxt[kc][t];
            }
            if (grp + NW < n_groups) {
                nxt = stage(grp + NW);
                if constexpr (PF == 2) load_values(grp + NW, va_nxt);
            }
        } else {
            cur = stage(grp);
        }
        const typename Pol::Codes &codes = cur.codes;
        const uint2 meta = cur.meta;
        const bool valid = cur.valid;
        // PF = 3: this group's values are issued before its logits
        if constexpr (PF == 3) load_values(grp, va);

        // 2. logits, lane = token
        float lg[G];
#pragma unroll
        for (int g = 0; g < G; ++g) lg[g] = -INFINITY;
        pol.logits(ps, codes, meta, valid, lg);

        // 3. values (without PF = 2), issued after the logit arithmetic so
        //    they are not held in registers through it (other wavefronts'
        //    work covers their latency)
        if constexpr (PF < 2) load_values(grp, va);

        // 4. online softmax, weights to LDS as fp16 hi + lo
        float alpha_n = 1.f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mx = wave_max(valid ? lg[g] : -INFINITY);
            const float mnew = fmaxf(m_run[g], mx);
            const float alpha = (m_run[g] == -INFINITY) ? 0.f : exp2f(m_run[g] - mnew);
            const float p = valid ? exp2f(lg[g] - mnew) : 0.f;
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
        wave_lds_sync();

        // 5. O^T += V^T P^T on the matrix cores
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            half8_t bh = {}, bl = {};
            if (n_head < G) {
                bh = *reinterpret_cast<const half8_t *>(&cs.pb[w][0][n_head][32 * kc + 8 * kq]);
                bl = *reinterpret_cast<const half8_t *>(&cs.pb[w][1][n_head][32 * kc + 8 * kq]);
            }
#pragma unroll
            for (int t = 0; t < 8; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, va[kc][t]), bh, acc[t],
                                                                0, 0, 0);
#pragma unroll
            for (int t = 0; t < 8; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, va[kc][t]), bl, acc[t],
                                                                0, 0, 0);
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
    const size_t bq0 = (size_t)b * a.Hq + (size_t)h * G;
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

// Reduction pass.  One work-group of kReduceThreads per (sequence, query
// head, 32-dimension slice): the running max and the weighted sum of the
// chunks' partial sums are block reductions over the chunks; the output
// slice is summed by 8 chunk lanes x 32 dimensions, each lane taking every
// 8th chunk, then merged in LDS.  Every order is fixed, so the result is
// deterministic.
constexpr int kReduceThreads = 256;
constexpr int kReduceSlices = 4;   // 128 dimensions / 32

template <bool MAX>
__device__ __forceinline__ float block_reduce(float v, float *scratch) {
    v = MAX ? wave_max(v) : wave_sum(v);
    const int wv = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[wv] = v;
    __syncthreads();
    float r = scratch[0];
#pragma unroll
    for (int i = 1; i < kReduceThreads / 64; ++i) r = MAX ? fmaxf(r, scratch[i]) : r + scratch[i];
    return r;
}

__device__ __forceinline__ void reduce_chunks(const float *pm, const float *pl, const float *pacc, int S, int nc,
                                              int bq, int slice, float *out, float *lse) {
    __shared__ float scratch[kReduceThreads / 64];
    __shared__ float part_sum[8][32];
    const int tid = threadIdx.x;
    const size_t base = (size_t)bq * S;
    const int d = slice * 32 + (tid & 31), part = tid >> 5;
    // the first 64 chunks' accumulators are loaded before the reductions
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = part + 8 * i;
        pv[i] = c < nc ? pacc[(base + c) * kD + d] : 0.f;
    }
    float M = -INFINITY;
    for (int c = tid; c < nc; c += kReduceThreads) M = fmaxf(M, pm[base + c]);
    M = block_reduce<true>(M, scratch);
    if (M == -INFINITY) {   // no chunk holds a kept token (uniform over the block)
        if (tid < 32) out[(size_t)bq * kD + d] = 0.f;
        if (lse && slice == 0 && tid == 0) lse[bq] = -INFINITY;
        return;
    }
    float L = 0.f;
    for (int c = tid; c < nc; c += kReduceThreads) L = fmaf(pl[base + c], exp2f(pm[base + c] - M), L);
    L = block_reduce<false>(L, scratch);
    float o = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = part + 8 * i;
        if (c < nc) o = fmaf(pv[i], exp2f(pm[base + c] - M), o);
    }
#pragma unroll 4
    for (int c = part + 64; c < nc; c += 8) o = fmaf(pacc[(base + c) * kD + d], exp2f(pm[base + c] - M), o);
    part_sum[part][tid & 31] = o;
    __syncthreads();
    if (tid < 32) {
        float t = part_sum[0][tid];
#pragma unroll
        for (int i = 1; i < 8; ++i) t += part_sum[i][tid];
        out[(size_t)bq * kD + d] = t / L;
    }
    if (lse && slice == 0 && tid == 0) lse[bq] = (M + log2f(L)) * 0.69314718055994531f;
}

}  // namespace core
}  // namespace ada
