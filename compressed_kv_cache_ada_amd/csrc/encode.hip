// encode.hip -- page writers for gfx950: bulk pack from a tier map,
// sequential-semantics append, page zeroing, cache reset.  The exact key
// encoder itself is encode_core.h.
// Compiled with -ffp-contract=off: every rounding below is the one written.
//
// Method: "SPHERICAL KV" (arXiv 2605.18856), Abstract: keys are stored as a
// scalar radius plus compact angle codes in tier-homogeneous pages with
// lightweight metadata.
#include "encode_core.h"

namespace ada {
namespace {

using enc::f64_to_f16_rne_sat;
using enc::v8_value_bits;
using enc::read_status;
using enc::set_status;

// ------------------------------------------------ encode + write one key
// One wavefront per item; 4 wavefronts per work-group; grid-stride.  Four
// wavefronts per SIMD (128 registers; the rarely taken exact-boundary path
// spills a few bytes) run the pack 10% faster than the three the
// unconstrained register count allows.
__global__ __launch_bounds__(256, 4) void encode_write_kernel(EncodeLaunch a) {
    __shared__ uint32_t words[4][2][16];
    const int wv = threadIdx.x >> 6;
    if (read_status(a.status) != 0) return;
    for (int64_t item = (int64_t)blockIdx.x * 4 + wv; item < a.n; item += (int64_t)gridDim.x * 4) {
        const int page = a.dest_page[item];
        if (page < 0) continue;
        const uint2 meta = *reinterpret_cast<const uint2 *>(a.page_meta + page);
        enc::encode_write_one(a.keys + item * kD, a.values + item * kD, a.dest_slot[item], meta, a.arena, a.P,
                              a.status, words[wv], a.half_pairs != 0);
    }
}

// ------------------------------------------------- transcode (re-pack)
// Code-space transcoding of one token from tier TO to tier TN (TN = TO or
// coarser): angle codes to the nearest point of the nested coarser grid
// (exactly half-way rounds up, then wraps), magnitude codes to the nearest
// level c * LN / LO (never a tie for these tiers); radius unchanged.  One
// thread per token; every bit position is static once the loops unroll.
template <int B>
__device__ inline uint32_t get_code(const uint32_t *w, int j) {
    const int bit = j * B, wi = bit >> 5, sh = bit & 31;
    uint32_t v = w[wi] >> sh;
    if (sh + B > 32) v |= w[wi + 1] << (32 - sh);
    return v & ((1u << B) - 1u);
}

template <int B>
__device__ inline void put_code(uint32_t *w, int j, uint32_t c) {
    const int bit = j * B, wi = bit >> 5, sh = bit & 31;
    w[wi] |= c << sh;
    if (sh + B > 32) w[wi + 1] |= c >> (32 - sh);
}

// component of B bits per code: 8*B bytes per token as 16-byte units
// (token-minor), then one 8-byte unit when 8*B % 16 == 8
template <int B>
__device__ inline void load_comp(const uint8_t *comp, int P, int slot, uint32_t (&w)[2 * B]) {
#pragma unroll
    for (int u = 0; u < B / 2; ++u) {
        const uint4 v = *reinterpret_cast<const uint4 *>(comp + (size_t)u * 16 * P + slot * 16);
        w[4 * u] = v.x;
        w[4 * u + 1] = v.y;
        w[4 * u + 2] = v.z;
        w[4 * u + 3] = v.w;
    }
    if constexpr (B % 2) {
        const uint2 v = *reinterpret_cast<const uint2 *>(comp + (size_t)(B / 2) * 16 * P + slot * 8);
        w[2 * B - 2] = v.x;
        w[2 * B - 1] = v.y;
    }
}

template <int B>
__device__ inline void store_comp(uint8_t *comp, int P, int slot, const uint32_t (&w)[2 * B]) {
#pragma unroll
    for (int u = 0; u < B / 2; ++u)
        *reinterpret_cast<uint4 *>(comp + (size_t)u * 16 * P + slot * 16) =
            make_uint4(w[4 * u], w[4 * u + 1], w[4 * u + 2], w[4 * u + 3]);
    if constexpr (B % 2)
        *reinterpret_cast<uint2 *>(comp + (size_t)(B / 2) * 16 * P + slot * 8) = make_uint2(w[2 * B - 2], w[2 * B - 1]);
}

template <int TO, int TN>
__device__ inline void transcode_token(const uint8_t *sblk, int sslot, uint8_t *dblk, int slot, int P) {
    constexpr int BO = tier_tb(TO), SO = tier_sb(TO), BN = tier_tb(TN), SN = tier_sb(TN);
    {
        uint32_t wi[2 * BO], wo[2 * BN];
        load_comp<BO>(sblk + 2 * P, P, sslot, wi);
#pragma unroll
        for (int k = 0; k < 2 * BN; ++k) wo[k] = 0u;
#pragma unroll
        for (int j = 0; j < 64; ++j) {
            uint32_t c = get_code<BO>(wi, j);
            if constexpr (BO > BN) c = ((c + (1u << (BO - BN - 1))) >> (BO - BN)) & ((1u << BN) - 1u);
            put_code<BN>(wo, j, c);
        }
        store_comp<BN>(dblk + 2 * P, P, slot, wo);
    }
    {
        constexpr uint32_t LO = (1u << SO) - 1u, LN = (1u << SN) - 1u;
        uint32_t wi[2 * SO], wo[2 * SN];
        load_comp<SO>(sblk + 2 * P + 8 * BO * P, P, sslot, wi);
#pragma unroll
        for (int k = 0; k < 2 * SN; ++k) wo[k] = 0u;
#pragma unroll
        for (int j = 0; j < 64; ++j) {
            uint32_t c = get_code<SO>(wi, j);
            if constexpr (SO != SN) c = (2u * c * LN + LO) / (2u * LO);
            put_code<SN>(wo, j, c);
        }
        store_comp<SN>(dblk + 2 * P + 8 * BN * P, P, slot, wo);
    }
    reinterpret_cast<uint16_t *>(dblk)[slot] = reinterpret_cast<const uint16_t *>(sblk)[sslot];
}

template <int TN>
__device__ inline void zero_token(uint8_t *dblk, int slot, int P) {
    constexpr int BN = tier_tb(TN), SN = tier_sb(TN);
    uint32_t zt[2 * BN], zs[2 * SN];
#pragma unroll
    for (int k = 0; k < 2 * BN; ++k) zt[k] = 0u;
#pragma unroll
    for (int k = 0; k < 2 * SN; ++k) zs[k] = 0u;
    store_comp<BN>(dblk + 2 * P, P, slot, zt);
    store_comp<SN>(dblk + 2 * P + 8 * BN * P, P, slot, zs);
    reinterpret_cast<uint16_t *>(dblk)[slot] = 0;
}

// The transcoder's three steps for one new page m (metadata) whose source
// entries s sit in LDS.  Threads are dimensions (dim = thread index).
template <int P>
__device__ __forceinline__ void tc_load_values(const PackLaunch &a, const int4 (&s)[P], int dim, uint32_t (&wa)[P],
                                               uint32_t (&wb)[P]) {
    // 1. this dimension's value of every source token, all loads issued
    //    before any is used (branch-free: an empty slot reads the arena's
    //    first word, unused).  fp16 source: the dword holding the value
    //    (twice); V8 source: the dwords holding its code and scale bytes.
    //    A source page's values follow its key part in its block.
#pragma unroll
    for (int k = 0; k < P; ++k) {
        const int4 ek = s[k];
        const size_t vpart = ((size_t)(uint32_t)ek.w + key16(ek.z, P)) * 16;
        size_t oa, ob;
        if (tier_v8(ek.z)) {
            const size_t grp = vpart + (ek.y >> 4) * kV8Group;
            oa = grp + kV8Codes + dim * 16 + (ek.y & 12);
            ob = grp + (ek.y & 15) * 4;
        } else {
            oa = vpart + (ek.y >> 3) * 2048 + dim * 16 + ((ek.y & 7) >> 1) * 4;
            ob = oa;
        }
        if (ek.x < 0) oa = ob = 0;
        wa[k] = *reinterpret_cast<const uint32_t *>(a.src_arena + oa);
        wb[k] = *reinterpret_cast<const uint32_t *>(a.src_arena + ob);
    }
}

template <int P>
__device__ __forceinline__ void tc_codes(const PackLaunch &a, const ada_page_meta_t &m, int4 e, int tid) {
    const int count = m.count, tier = m.tier;
    // 2. threads 0..P-1: token tid's codes
    if (tid < P) {
        uint8_t *dblk = a.arena + (size_t)m.code_off16 * 16;
        const int k = tid;
        // key tiers (0 T8, 1 T4, 2 T2) of source and destination
        const int st = key_tier(e.z), dt = key_tier(tier);
        const bool upgrade = k < count && (st > dt || (tier_v8(e.z) && !tier_v8(tier)));
        if (k >= count || upgrade) {   // past the count; or an upgrade, which the caps rule out
            if (upgrade) set_status(a.status, ADA_EINTERNAL);
            if (dt == 0) zero_token<0>(dblk, k, P);
            else if (dt == 1) zero_token<1>(dblk, k, P);
            else zero_token<2>(dblk, k, P);
        } else {
            const uint8_t *sblk = a.src_arena + (size_t)(uint32_t)e.w * 16;
            const int sslot = e.y;
            if (dt == 0) transcode_token<0, 0>(sblk, sslot, dblk, k, P);
            else if (dt == 1 && st == 0) transcode_token<0, 1>(sblk, sslot, dblk, k, P);
            else if (dt == 1) transcode_token<1, 1>(sblk, sslot, dblk, k, P);
            else if (st == 0) transcode_token<0, 2>(sblk, sslot, dblk, k, P);
            else if (st == 1) transcode_token<1, 2>(sblk, sslot, dblk, k, P);
            else transcode_token<2, 2>(sblk, sslot, dblk, k, P);
        }
    }
}

template <int P>
__device__ __forceinline__ void tc_values(const PackLaunch &a, const ada_page_meta_t &m, const int4 (&s)[P],
                                          const uint32_t (&wa)[P], const uint32_t (&wb)[P], int dim) {
    const int tier = m.tier;
    // 3. the value part, per 16 tokens and dimension: one thread per
    //    dimension; a V8 source is decoded first (its values are fp16
    //    numbers exactly)
    uint8_t *dvb = a.arena + ((size_t)m.code_off16 + key16(tier, P)) * 16;
    const bool dst_v8 = tier_v8(tier);
#pragma unroll
    for (int g = 0; g < P / 16; ++g) {
        uint32_t h[16];
        bool live[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int4 ek = s[16 * g + k];
            const uint32_t ra = wa[16 * g + k], rb = wb[16 * g + k];
            live[k] = ek.x >= 0;
            if (!live[k]) h[k] = 0u;
            else if (tier_v8(ek.z))
                h[k] = v8_value_bits((int)((ra >> (8 * (ek.y & 3))) & 0xFFu) - 128, (rb >> (8 * (dim >> 5))) & 0xFFu);
            else h[k] = (ra >> ((ek.y & 1) * 16)) & 0xFFFFu;
        }
        if (!dst_v8) {   // two 8-token groups, [128 dims][8 tokens] fp16 each
#pragma unroll
            for (int hg = 0; hg < 2; ++hg) {
                uint32_t w[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) w[k] = h[8 * hg + 2 * k] | (h[8 * hg + 2 * k + 1] << 16);
                *reinterpret_cast<uint4 *>(dvb + (2 * g + hg) * 2048 + dim * 16) = make_uint4(w[0], w[1], w[2], w[3]);
            }
        } else {
            // V8: per token, the exponent of its 32-dimension block (32
            // consecutive lanes), then this dimension's code; empty slots
            // are zero
            uint32_t cw[4] = {0u, 0u, 0u, 0u};
            uint32_t sw[4] = {0u, 0u, 0u, 0u};   // scale bytes of this block, tokens 4i .. 4i + 3
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                int mx = (int)(h[k] & 0x7FFFu);
                mx = max(mx, __shfl_xor(mx, 1, 64));
                mx = max(mx, __shfl_xor(mx, 2, 64));
                mx = max(mx, __shfl_xor(mx, 4, 64));
                mx = max(mx, __shfl_xor(mx, 8, 64));
                mx = max(mx, __shfl_xor(mx, 16, 64));
                const int ex = enc::v8_exponent((uint32_t)mx);
                const uint32_t c = live[k] ? (uint32_t)(enc::v8_code(h[k], ex) + 128) : 0u;
                const uint32_t sbyte = live[k] ? (uint32_t)(ex + 127) : 0u;
                cw[k >> 2] |= c << (8 * (k & 3));
                sw[k >> 2] |= sbyte << (8 * (k & 3));
            }
            uint8_t *grp = dvb + g * kV8Group;
            *reinterpret_cast<uint4 *>(grp + kV8Codes + dim * 16) = make_uint4(cw[0], cw[1], cw[2], cw[3]);
            if ((dim & 31) == 0)   // token k's scale byte of this block
#pragma unroll
                for (int k = 0; k < 16; ++k) grp[k * 4 + (dim >> 5)] = (uint8_t)(sw[k >> 2] >> (8 * (k & 3)));
        }
    }
}

// Re-pack: the order the transcoder writes the new pages in.  Pages are
// allocated row by row and, within a row, tier by tier, each tier's pages in
// the order of their tokens' source positions.  Here a row's pages of all
// tiers are merged by the source position of their first token (distinct
// for distinct pages of a row): a page's rank is its index in its tier plus,
// for every other tier of the row, the number of that tier's pages that
// start earlier (a binary search in its increasing first positions).  So
// the pages that draw from one stretch of a source row are written close
// together in time, and the source value groups they share are read once.
__global__ __launch_bounds__(256) void repack_order_kernel(PackLaunch a) {
    if (read_status(a.status) != 0) return;
    const int first = a.n_new[0];
    const int n = (int)min((int64_t)a.n_new[1], a.src_of_slot_pages);
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int page = first + i;
    const int rows = a.B * a.Hkv;
    // the row: the last one whose first page id is at most this page (an
    // empty row shares its first page id with the next row)
    int lo = 0, hi = rows - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (a.row_base[mid * kNumTiers] <= page) lo = mid;
        else hi = mid - 1;
    }
    const int row = lo;
    const int tier = a.page_meta[page].tier;
    const int my = a.first_pos[i];
    int rank = page - a.row_base[row * kNumTiers + tier];
    for (int t = 0; t < kNumTiers; ++t) {
        if (t == tier) continue;
        const int np = (a.row_counts[row * kNumTiers + t] + a.P - 1) / a.P;
        const int base = a.row_base[row * kNumTiers + t] - first;
        int l = 0, h = np;   // pages of tier t that start before `my`
        while (l < h) {
            const int mid = (l + h) / 2;
            if (a.first_pos[base + mid] < my) l = mid + 1;
            else h = mid;
        }
        rank += l;
    }
    a.page_order[a.row_base[row * kNumTiers] - first + rank] = i;
}

// About one round of resident 128-thread work-groups, each writing new
// destination pages in turn (grid-stride).  Every byte of a page's code
// block and value page is written, slots past the count as zeros.  A page's
// source entries {page, slot, tier, code offset} pass through LDS once; each
// thread (one dimension) then issues the loads of all P source values of its
// dimension together (the 4-byte word holding a token's fp16 value, or a V8
// token's code and scale bytes) while threads 0..P-1 transcode one token's
// codes each.  The next page's metadata and entries are requested while the
// current page is written, so a page costs one dependent memory step of its
// own (its codes and values) besides the stores.
// (Four wavefronts per SIMD: P = 32 then holds 128 registers and spills a
// few bytes, and runs about 20% faster than at three.)
template <int P>
__global__ __launch_bounds__(128, 4) void transcode_pages_kernel(PackLaunch a) {
    __shared__ int4 s_ent[2][P];   // the current page's source entries, and the next page's
    __shared__ int s_stop;
    const int tid = threadIdx.x, dim = tid;
    // one reading of the status word for the whole work-group: its waves
    // must agree, since they meet at barriers below
    if (tid == 0) s_stop = read_status(a.status);
    __syncthreads();
    if (s_stop != 0) return;
    const int first = a.n_new[0];
    const int n = (int)min((int64_t)a.n_new[1], a.src_of_slot_pages);   // bounded by construction
    // the next page's metadata and entries are requested while the current
    // page is written (entries past a page's count are empty)
    auto fetch = [&](int i, ada_page_meta_t &m, int4 &e) {
        m = a.page_meta[first + i];
        e = tid < P ? a.src_of_slot[(int64_t)i * P + tid] : make_int4(-1, 0, 0, 0);
    };
    auto publish = [&](int buf, const ada_page_meta_t &m, const int4 &e) {
        if (tid < P) s_ent[buf][tid] = tid < (int)m.count ? e : make_int4(-1, 0, 0, 0);
    };
    // positions j of the write order (page_order[j] is a page): work-groups
    // go to the chip's 8 dies in turn, and die x = b % 8 takes the x-th
    // contiguous eighth of the order, so the pages that share source lines
    // share one L2
    int lo = 0, hi = n, j = blockIdx.x, step = gridDim.x;
    if (gridDim.x % 8 == 0) {
        const int part = (n + 7) / 8, x = blockIdx.x % 8;
        lo = x * part;
        hi = min(n, lo + part);
        step = gridDim.x / 8;
        j = lo + blockIdx.x / 8;
    }
    if (j >= hi) return;
    int i = a.page_order[j];
    ada_page_meta_t m;
    int4 e_raw;
    fetch(i, m, e_raw);
    publish(0, m, e_raw);
    __syncthreads();
    for (int buf = 0; j < hi; buf ^= 1) {
        const int jnext = j + step;
        const int inext = jnext < hi ? a.page_order[jnext] : 0;
        ada_page_meta_t m_next = m;
        int4 e_next = make_int4(-1, 0, 0, 0);
        if (jnext < hi) fetch(inext, m_next, e_next);
        const int4 (&s_cur)[P] = s_ent[buf];
        const int4 e = tid < P ? s_cur[tid] : make_int4(-1, 0, 0, 0);

        uint32_t wa[P], wb[P];
        tc_load_values<P>(a, s_cur, dim, wa, wb);
        tc_codes<P>(a, m, e, tid);
        tc_values<P>(a, m, s_cur, wa, wb, dim);
        if (jnext < hi) publish(buf ^ 1, m_next, e_next);
        m = m_next;
        j = jnext;
        i = inext;
        __syncthreads();   // the next page's entries are in place; this page's buffer is refilled after the next barrier
    }
}

// The same transcoder with each page's value loads issued one page ahead
// (16-token pages: two pages' values fit the registers).  The entries of the
// next page are in LDS while the current page is written: after this page's
// code loads, the next page's value loads are issued, and this page's values
// (loaded one iteration earlier) are assembled and written while they are in
// flight.  The barriers wait for LDS work only (s_waitcnt lgkmcnt(0), then
// s_barrier): a full __syncthreads would also wait for the loads in flight.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int P>
__global__ __launch_bounds__(128, 4) void transcode_pages_pipe_kernel(PackLaunch a) {
    __shared__ int4 s_ent[2][P];   // the current page's source entries, and the next page's
    __shared__ int s_stop;
    const int tid = threadIdx.x, dim = tid;
    if (tid == 0) s_stop = read_status(a.status);
    __syncthreads();
    if (s_stop != 0) return;
    const int first = a.n_new[0];
    const int n = (int)min((int64_t)a.n_new[1], a.src_of_slot_pages);   // bounded by construction
    auto fetch = [&](int i, ada_page_meta_t &m, int4 &e) {
        m = a.page_meta[first + i];
        e = tid < P ? a.src_of_slot[(int64_t)i * P + tid] : make_int4(-1, 0, 0, 0);
    };
    auto publish = [&](int buf, const ada_page_meta_t &m, const int4 &e) {
        if (tid < P) s_ent[buf][tid] = tid < (int)m.count ? e : make_int4(-1, 0, 0, 0);
    };
    // die x = b % 8 takes the x-th contiguous eighth of the write order
    int lo = 0, hi = n, j = blockIdx.x, step = gridDim.x;
    if (gridDim.x % 8 == 0) {
        const int part = (n + 7) / 8, x = blockIdx.x % 8;
        lo = x * part;
        hi = min(n, lo + part);
        step = gridDim.x / 8;
        j = lo + blockIdx.x / 8;
    }
    if (j >= hi) return;
    // pages at write positions j (current), j1, j2: entries of j and j1 in
    // LDS, of j2 in registers; the page of j3 is requested one iteration
    // before its entries are
    int j1 = j + step, j2 = j1 + step;
    const int i0 = a.page_order[j];
    const int i1 = j1 < hi ? a.page_order[j1] : 0;
    int i2 = j2 < hi ? a.page_order[j2] : 0;
    ada_page_meta_t m, m1;
    int4 e0, e1 = make_int4(-1, 0, 0, 0);
    fetch(i0, m, e0);
    m1 = m;
    if (j1 < hi) fetch(i1, m1, e1);
    publish(0, m, e0);
    lds_barrier();
    uint32_t wa[P], wb[P];
    tc_load_values<P>(a, s_ent[0], dim, wa, wb);
    if (j1 < hi) publish(1, m1, e1);
    lds_barrier();
    for (int buf = 0; j < hi; buf ^= 1) {
        ada_page_meta_t m2 = m1;
        int4 e2 = make_int4(-1, 0, 0, 0);
        if (j2 < hi) fetch(i2, m2, e2);
        const int j3 = j2 + step;
        const int i3 = j3 < hi ? a.page_order[j3] : 0;
        const int4 e = tid < P ? s_ent[buf][tid] : make_int4(-1, 0, 0, 0);
        tc_codes<P>(a, m, e, tid);
        uint32_t wa1[P], wb1[P];
#pragma unroll
        for (int k = 0; k < P; ++k) wa1[k] = wb1[k] = 0u;
        if (j1 < hi) tc_load_values<P>(a, s_ent[buf ^ 1], dim, wa1, wb1);
        tc_values<P>(a, m, s_ent[buf], wa, wb, dim);
        lds_barrier();   // every thread is done with this page's entries
        if (j2 < hi) publish(buf, m2, e2);
        lds_barrier();   // the entries of the page after the next one are in place
#pragma unroll
        for (int k = 0; k < P; ++k) {
            wa[k] = wa1[k];
            wb[k] = wb1[k];
        }
        m = m1;
        m1 = m2;
        j = j1;
        j1 = j2;
        j2 = j3;
        i2 = i3;
    }
}

// ------------------------------------------------------- zero new pages
// pages: explicit list, or (when list == nullptr) the range [first, first+n)
__global__ __launch_bounds__(256) void zero_pages_kernel(const int32_t *list, const int32_t *first_and_n,
                                                         const ada_page_meta_t *page_meta, uint8_t *arena,
                                                         int32_t P, const int32_t *status) {
    if (read_status(status) != 0) return;
    const int n = first_and_n[1];
    for (int i = blockIdx.x; i < n; i += gridDim.x) {
        const int page = list ? list[i] : first_and_n[0] + i;
        const uint2 meta = *reinterpret_cast<const uint2 *>(page_meta + page);
        const int tier = meta.x & 0xFF;
        uint4 *cb = reinterpret_cast<uint4 *>(arena + (size_t)meta.y * 16);
        const int nb = block16(tier, P);
        for (int k = threadIdx.x; k < nb; k += blockDim.x) cb[k] = make_uint4(0u, 0u, 0u, 0u);
    }
}

// ------------------------------------------------------------ row order
// One work-group: the rows by decreasing page count, ties in row order
// (rank of row r = rows with more pages + rows before r with as many).
// Up to kMaxOrderRows rows; beyond that the order is left as it is.
constexpr int kMaxOrderRows = 16384;
__global__ __launch_bounds__(1024) void row_order_kernel(int32_t rows, const int32_t *num_pages, int32_t *row_order) {
    __shared__ int32_t tile[4096];
    if (rows > kMaxOrderRows) return;
    for (int base_r = 0; base_r < rows; base_r += 1024) {
        const int r = base_r + threadIdx.x;
        const int np = r < rows ? num_pages[r] : 0;
        int rank = 0;
        for (int base_j = 0; base_j < rows; base_j += 4096) {
            __syncthreads();
            for (int k = threadIdx.x; k < 4096 && base_j + k < rows; k += 1024) tile[k] = num_pages[base_j + k];
            __syncthreads();
            const int n = rows - base_j < 4096 ? rows - base_j : 4096;
            for (int k = 0; k < n; ++k) {
                const int v = tile[k];
                rank += (v > np) || (v == np && base_j + k < r);
            }
        }
        if (r < rows) row_order[rank] = r;
    }
}

// ------------------------------------------------------- pack page writer
// One work-group (four wavefronts) per new page of a pack, in turn: the
// page's tokens are encoded one per wavefront into a copy of the page's
// block in LDS (empty slots stay zero), which is then written out whole in
// 16-byte stores.  Every byte of the block is written once, by full 16-byte
// units (the token-by-token writer leaves 1- to 4-byte pieces of each unit
// to be merged in the caches, and zeroes the page beforehand).
template <int P>
__global__ __launch_bounds__(256, 3) void pack_write_pages_kernel(PackLaunch a) {
    constexpr int kMaxBlock16 = block16(0, P);   // T8 with fp16 values: the largest block
    __shared__ uint4 blk[kMaxBlock16];
    __shared__ uint32_t words[4][2][16];
    __shared__ int s_stop;
    const int tid = threadIdx.x, wv = tid >> 6;
    if (tid == 0) s_stop = read_status(a.status);
    __syncthreads();
    if (s_stop != 0) return;
    const int first = a.n_new[0];
    const int64_t n = min((int64_t)a.n_new[1], a.item_slot_pages);
    for (int64_t i = blockIdx.x; i < n; i += gridDim.x) {
        const uint2 meta = *reinterpret_cast<const uint2 *>(a.page_meta + first + i);
        const int tier = meta.x & 0xFF, count = (meta.x >> 8) & 0xFF;
        const int nb = block16(tier, P);
        for (int k = tid; k < nb; k += 256) blk[k] = make_uint4(0u, 0u, 0u, 0u);
        __syncthreads();
        // the LDS copy stands in for the arena: block at offset 0
        const uint2 lmeta = make_uint2(meta.x, 0u);
        for (int slot = wv; slot < count; slot += 4) {
            const int64_t item = a.item_of_slot[i * P + slot];
            enc::encode_write_one(a.keys + item * kD, a.values + item * kD, slot, lmeta,
                                  reinterpret_cast<uint8_t *>(blk), P, a.status, words[wv], a.half_pairs != 0);
        }
        __syncthreads();
        uint4 *dst = reinterpret_cast<uint4 *>(a.arena + (size_t)meta.y * 16);
        for (int k = tid; k < nb; k += 256) dst[k] = blk[k];
        __syncthreads();   // the LDS copy is refilled for the next page
    }
}

// ------------------------------------------------------------- pack
constexpr int kTile = 1024;

// per (row, tile): validate tiers, check kept keys (and the values of V8
// tokens) are finite, count per tier
__global__ __launch_bounds__(256) void pack_count_kernel(PackLaunch a) {
    __shared__ int cnt[kNumTiers];
    __shared__ int8_t s_tier[kTile];   // the tile's tiers, for the key checks below
    const int tile = blockIdx.x, row = blockIdx.y;
    const int b = row / a.Hkv;
    const int ctx = a.ctx_len_dev[b];
    if (threadIdx.x < kNumTiers) cnt[threadIdx.x] = 0;
    __syncthreads();
    const int64_t rbase = (int64_t)row * a.stride;
    const int t0 = tile * kTile;
    for (int i = threadIdx.x; i < kTile; i += 256) {
        const int t = t0 + i;
        const int tv = t < ctx ? a.tier[rbase + t] : -1;
        s_tier[i] = (int8_t)tv;
        if (t >= ctx) continue;
        if (tv < -1 || tv >= a.n_tiers) set_status(a.status, ADA_EINVAL);
        else if (tv >= 0) atomicAdd(&cnt[tv], 1);
    }
    __syncthreads();
    // finiteness of kept keys: one wavefront per position (no keys when
    // re-packing from a cache).  The tiers come from LDS and every position's
    // key is read (a dropped one is ignored), so the loads of successive
    // positions do not wait on each other.
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    bool bad = false;
#pragma unroll 4
    for (int i = wv; a.keys && i < kTile; i += 4) {
        const int t = t0 + i;
        if (t >= ctx) break;
        const int tv = s_tier[i];
        const float2 kk = *reinterpret_cast<const float2 *>(a.keys + (rbase + t) * kD + 2 * lane);
        bad |= tv >= 0 && !(isfinite(kk.x) && isfinite(kk.y));
        if (tv >= 0 && tv < kNumTiers && tier_v8(tv))
            bad |= !values_finite(*reinterpret_cast<const uint32_t *>(a.values + (rbase + t) * kD + 2 * lane));
    }
    if (__any(bad) && lane == 0) set_status(a.status, ADA_EINVAL);
    __syncthreads();
    if (threadIdx.x < kNumTiers)
        a.tile_counts[((size_t)row * a.n_tiles + tile) * kNumTiers + threadIdx.x] = cnt[threadIdx.x];
}

// per row: exclusive scan of tile counts (in place) and row totals
__global__ __launch_bounds__(256) void pack_rowscan_kernel(PackLaunch a) {
    const int row = blockIdx.x;
    if (threadIdx.x >= kNumTiers) return;
    const int tau = threadIdx.x;
    int run = 0;
    int32_t *tc = a.tile_counts + (size_t)row * a.n_tiles * kNumTiers;
    for (int tl = 0; tl < a.n_tiles; ++tl) {
        const int c = tc[tl * kNumTiers + tau];
        tc[tl * kNumTiers + tau] = run;
        run += c;
    }
    a.row_counts[row * kNumTiers + tau] = run;
}

// single work-group: page and code-unit bases of every (row, tier), capacity
// checks, row metadata and the allocation counters
__global__ __launch_bounds__(1024) void pack_plan_kernel(PackLaunch a, int32_t *range /* [2] first, n */) {
    __shared__ long long sp[1024], su[1024];
    __shared__ long long carry_p, carry_u;
    __shared__ int bad;
    if (threadIdx.x == 0) {
        carry_p = 0;
        carry_u = 0;
        bad = read_status(a.status);
    }
    __syncthreads();
    if (bad) return;
    const int rows = a.B * a.Hkv;
    const int n_ent = rows * kNumTiers;
    const int64_t a0 = a.alloc[0], a1 = a.alloc[1];
    for (int base = 0; base < n_ent; base += 1024) {
        const int i = base + threadIdx.x;
        long long pg = 0, un = 0;
        if (i < n_ent) {
            const int n = a.row_counts[i];
            pg = (n + a.P - 1) / a.P;
            un = pg * block16(i % kNumTiers, a.P);
        }
        sp[threadIdx.x] = pg;
        su[threadIdx.x] = un;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {   // inclusive scan
            long long vp = 0, vu = 0;
            if (threadIdx.x >= off) {
                vp = sp[threadIdx.x - off];
                vu = su[threadIdx.x - off];
            }
            __syncthreads();
            sp[threadIdx.x] += vp;
            su[threadIdx.x] += vu;
            __syncthreads();
        }
        if (i < n_ent) {
            a.row_base[i] = (int32_t)(a0 + carry_p + sp[threadIdx.x] - pg);
            a.row_unit[i] = a1 + carry_u + su[threadIdx.x] - un;
        }
        __syncthreads();
        if (threadIdx.x == 1023) {
            carry_p += sp[1023];
            carry_u += su[1023];
        }
        __syncthreads();
    }
    // capacity
    if (threadIdx.x == 0) {
        if (a0 + carry_p > a.page_capacity || a1 + carry_u > a.arena_capacity16) set_status(a.status, ADA_ENOSPC);
    }
    for (int r = threadIdx.x; r < rows; r += 1024) {
        int tot = 0;
        for (int tau = 0; tau < kNumTiers; ++tau) tot += (a.row_counts[r * kNumTiers + tau] + a.P - 1) / a.P;
        if (tot > a.maxp) set_status(a.status, ADA_ENOSPC);
    }
    __syncthreads();
    if (read_status(a.status) != 0) return;
    for (int r = threadIdx.x; r < rows; r += 1024) {
        int tot = 0;
        for (int tau = 0; tau < kNumTiers; ++tau) {
            const int n = a.row_counts[r * kNumTiers + tau];
            const int pg = (n + a.P - 1) / a.P;
            tot += pg;
            a.open_page[r * kNumTiers + tau] = (n % a.P != 0) ? a.row_base[r * kNumTiers + tau] + pg - 1 : -1;
        }
        a.num_pages[r] = tot;
    }
    if (threadIdx.x == 0) {
        a.alloc[0] = a0 + carry_p;
        a.alloc[1] = a1 + carry_u;
        range[0] = (int32_t)a0;
        range[1] = (int32_t)carry_p;
    }
}

// per row: page-table entries and page metadata of the row's new pages
__global__ __launch_bounds__(256) void pack_pages_kernel(PackLaunch a) {
    if (read_status(a.status) != 0) return;
    const int row = blockIdx.x;
    int pos = 0;
    for (int tau = 0; tau < kNumTiers; ++tau) {
        const int n = a.row_counts[row * kNumTiers + tau];
        const int pg = (n + a.P - 1) / a.P;
        const int base = a.row_base[row * kNumTiers + tau];
        const int64_t ubase = a.row_unit[row * kNumTiers + tau];
        for (int i = threadIdx.x; i < pg; i += 256) {
            const int page = base + i;
            a.page_table[(size_t)row * a.maxp + pos + i] = page;
            ada_page_meta_t m;
            m.tier = (uint8_t)tau;
            m.count = (uint8_t)((i == pg - 1) ? n - i * a.P : a.P);
            m.reserved = 0;
            m.code_off16 = (uint32_t)(ubase + (int64_t)i * block16(tau, a.P));
            a.page_meta[page] = m;
        }
        pos += pg;
    }
}

// per (row, tile): rank of every kept token within its (row, tier) ->
// destination page and slot
__global__ __launch_bounds__(256) void pack_dest_kernel(PackLaunch a) {
    __shared__ int sc[kNumTiers][256];
    const int tile = blockIdx.x, row = blockIdx.y;
    const int b = row / a.Hkv;
    const int ctx = a.ctx_len_dev[b];
    const int64_t rbase = (int64_t)row * a.stride;
    const int t0 = tile * kTile + threadIdx.x * 4;
    if (read_status(a.status) != 0) return;
    int tv[4], c[kNumTiers] = {};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int t = t0 + k;
        tv[k] = (t < ctx && t < a.stride) ? a.tier[rbase + t] : -1;
        if (tv[k] >= 0) c[tv[k]]++;
    }
    for (int tau = 0; tau < kNumTiers; ++tau) sc[tau][threadIdx.x] = c[tau];
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        int v[kNumTiers] = {};
        if (threadIdx.x >= off)
            for (int tau = 0; tau < kNumTiers; ++tau) v[tau] = sc[tau][threadIdx.x - off];
        __syncthreads();
        for (int tau = 0; tau < kNumTiers; ++tau) sc[tau][threadIdx.x] += v[tau];
        __syncthreads();
    }
    int run[kNumTiers];
    for (int tau = 0; tau < kNumTiers; ++tau)
        run[tau] = sc[tau][threadIdx.x] - c[tau] + a.tile_counts[((size_t)row * a.n_tiles + tile) * kNumTiers + tau];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int t = t0 + k;
        if (t >= a.stride) break;
        int dp = -1, ds = 0;
        if (tv[k] >= 0) {
            const int r = run[tv[k]]++;
            dp = a.row_base[row * kNumTiers + tv[k]] + r / a.P;
            ds = r % a.P;
        }
        a.dest_page[rbase + t] = dp;
        a.dest_slot[rbase + t] = ds;
        if (a.item_of_slot && dp >= 0) {   // pack: the item of the destination slot, for the page writer
            const int64_t j = (int64_t)(dp - a.n_new[0]) * a.P + ds;
            if (j < a.item_slot_pages * a.P) a.item_of_slot[j] = rbase + t;
        }
        if (a.src_of_slot && dp >= 0) {   // re-pack: where the destination slot's token comes from
            const int64_t j = (int64_t)(dp - a.n_new[0]) * a.P + ds;
            if (j < a.src_of_slot_pages * a.P) {
                const int sp = a.src_page_table[(int64_t)row * a.src_maxp + t / a.P];
                const ada_page_meta_t sm = a.src_page_meta[sp];
                a.src_of_slot[j] = make_int4(sp, t % a.P, sm.tier, (int)sm.code_off16);
                if (ds == 0) a.first_pos[dp - a.n_new[0]] = t;
            }
        }
    }
}

// ------------------------------------------------------------- append
struct AppendKernelArgs {
    AppendLaunch a;
    int32_t *key_off;   // [keys] code offset of the current page
};

__global__ __launch_bounds__(256) void append_init_kernel(AppendKernelArgs k) {
    const AppendLaunch &a = k.a;
    const int nkeys = a.num_seqs * a.Hkv * kNumTiers;
    for (int i = blockIdx.x * 256 + threadIdx.x; i < nkeys; i += gridDim.x * 256) {
        const int op = a.open_page[i];
        a.key_cnt[i] = 0;
        a.key_done[i] = 0;
        a.key_page[i] = op;
        int c0 = 0, off = 0;
        if (op >= 0) {
            const uint2 meta = *reinterpret_cast<const uint2 *>(a.page_meta + op);
            c0 = (meta.x >> 8) & 0xFF;
            off = (int)meta.y;
        }
        a.key_c0[i] = c0;
        k.key_off[i] = off;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        a.totals[0] = 0;
        a.totals[1] = 0;
        a.n_new[0] = 0;
    }
}

// request i's sequence and KV head; without seq / head arrays request i is
// row i (sequence i / Hkv, head i % Hkv)
__device__ inline int req_seq(const AppendLaunch &a, int i) { return a.seq ? a.seq[i] : i / a.Hkv; }
__device__ inline int req_head(const AppendLaunch &a, int i) { return a.head ? a.head[i] : i % a.Hkv; }

__global__ __launch_bounds__(256) void append_validate_kernel(AppendLaunch a) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    for (int i = blockIdx.x * 4 + wv; i < a.n; i += gridDim.x * 4) {
        const int s = req_seq(a, i), h = req_head(a, i), tau = a.tier[i];
        const bool in_range = s >= 0 && s < a.num_seqs && h >= 0 && h < a.Hkv && tau < a.n_tiers;
        const float2 kk = *reinterpret_cast<const float2 *>(a.keys + (int64_t)i * kD + 2 * lane);
        bool bad_l = !(isfinite(kk.x) && isfinite(kk.y));
        if (tau < kNumTiers && tier_v8(tau))
            bad_l |= !values_finite(*reinterpret_cast<const uint32_t *>(a.values + (int64_t)i * kD + 2 * lane));
        const bool bad = __any(bad_l);
        if (lane == 0) {
            if (!in_range || bad) set_status(a.status, ADA_EINVAL);
            else atomicAdd(&a.key_cnt[(s * a.Hkv + h) * kNumTiers + tau], 1);
        }
    }
}

__device__ inline int floordiv(int x, int P) { return x >= 0 ? x / P : -((-x + P - 1) / P); }

__global__ __launch_bounds__(256) void append_capacity_kernel(AppendLaunch a) {
    if (read_status(a.status) != 0) return;
    const int rows = a.num_seqs * a.Hkv;
    for (int r = blockIdx.x * 256 + threadIdx.x; r < rows; r += gridDim.x * 256) {
        int row_new = 0;
        long long units = 0;
        for (int tau = 0; tau < kNumTiers; ++tau) {
            const int key = r * kNumTiers + tau;
            const int cnt = a.key_cnt[key];
            if (cnt == 0) continue;
            const int c0 = a.key_c0[key];
            const int allocs = floordiv(c0 + cnt - 1, a.P) - floordiv(c0 - 1, a.P);
            row_new += allocs;
            units += (long long)allocs * block16(tau, a.P);
        }
        if (row_new == 0) continue;
        if (a.num_pages[r] + row_new > a.maxp) set_status(a.status, ADA_ENOSPC);
        atomicAdd((unsigned long long *)&a.totals[0], (unsigned long long)row_new);
        atomicAdd((unsigned long long *)&a.totals[1], (unsigned long long)units);
    }
}

// One request per row (request r = row r), single work-group: validates the
// tiers and keys, books each row's slot -- the next slot of its tier's open
// page, or a new page, new pages numbered in row order -- checks every
// capacity, and only if everything fits updates the metadata and the
// allocation counters (the same result as the general append of the same
// requests).  New pages are left to the caller to zero: their booked slot
// is 0, and new_pages[r] holds their code block offset (16-byte units).
__global__ __launch_bounds__(1024) void append_rows_kernel(AppendLaunch a) {
    __shared__ int s_need[16];         // per-wavefront totals of the tile scan
    __shared__ long long s_units[16];
    __shared__ int s_bad, s_stop, s_nospace, c_pages;
    __shared__ long long c_units;
    const int tid = threadIdx.x;
    if (tid == 0) {
        s_bad = 0;
        s_stop = 0;
        s_nospace = 0;
        c_pages = 0;
        c_units = 0;
    }
    const int P = a.P, rows = a.n;
    // The status word, the allocation counters and the first tile's booking
    // lookups are read together with the keys and values being checked, so
    // that the checks and the lookups share memory round trips; nothing is
    // written before every check has passed.
    const int status0 = read_status(a.status);
    const long long base_p = a.alloc[0], base_u = a.alloc[1];
    int tau0 = 0, np0 = 0;
    if (tid < rows) {
        tau0 = a.tier[tid];
        np0 = a.num_pages[tid];
    }
    int open0 = -1, cnt0 = P;
    if (tid < rows && tau0 < a.n_tiers) {   // a tier out of range fails the checks below
        open0 = a.open_page[tid * kNumTiers + tau0];
        if (open0 >= 0) cnt0 = (int)a.page_meta[open0].count;
    }
    // tiers and keys, coalesced: one thread per 16 bytes of key; then the
    // values of V8 tokens, one thread per 16 bytes of values
    const float4 *k4 = reinterpret_cast<const float4 *>(a.keys);
    bool ok = true;
    for (int i = tid; i < rows * (kD / 4); i += 1024) {
        const float4 v = k4[i];
        ok &= isfinite(v.x) & isfinite(v.y) & isfinite(v.z) & isfinite(v.w);
        if ((i & 31) == 0) ok &= a.tier[i >> 5] < a.n_tiers;
    }
    const uint4 *v4 = reinterpret_cast<const uint4 *>(a.values);
    for (int i = tid; i < rows * (kD / 8); i += 1024) {
        const int tau = a.tier[i >> 4];
        if (tau < kNumTiers && tier_v8(tau)) {
            const uint4 v = v4[i];
            ok &= values_finite(v.x) & values_finite(v.y) & values_finite(v.z) & values_finite(v.w);
        }
    }
    __syncthreads();   // the flags' initial values are in place
    if (status0 != 0) atomicOr(&s_stop, 1);
    if (!ok) atomicOr(&s_bad, 1);
    __syncthreads();
    if (s_stop) return;   // an earlier error: leave everything as it is
    if (s_bad) {
        if (tid == 0) set_status(a.status, ADA_EINVAL);
        return;
    }
    int f_page = -1, f_slot = 0;   // the first tile's booking of row tid, kept for the updates
    uint32_t f_unit = 0;
    for (int t0 = 0; t0 < rows; t0 += 1024) {
        const int r = t0 + tid;
        int need = 0, page = -1, slot = 0;
        long long units = 0;
        if (r < rows) {
            int tau, open, cnt, np;
            if (t0 == 0) {   // read above
                tau = tau0;
                open = open0;
                cnt = cnt0;
                np = np0;
            } else {
                tau = a.tier[r];
                open = a.open_page[r * kNumTiers + tau];
                cnt = open >= 0 ? (int)a.page_meta[open].count : P;
                np = a.num_pages[r];
            }
            if (cnt < P) {
                page = open;
                slot = cnt;
            } else {
                need = 1;
                units = block16(tau, P);
                if (np >= a.maxp) atomicOr(&s_nospace, 1);
            }
        }
        // inclusive scans of new pages and code units over the tile: within
        // each wavefront by shuffles, then the wavefronts' totals through LDS
        const int lane = tid & 63, wv = tid >> 6;
        int need_in = need;
        long long units_in = units;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int v = __shfl_up(need_in, off, 64);
            const long long u = __shfl_up(units_in, off, 64);
            if (lane >= off) {
                need_in += v;
                units_in += u;
            }
        }
        if (lane == 63) {
            s_need[wv] = need_in;
            s_units[wv] = units_in;
        }
        __syncthreads();
        for (int w = 0; w < wv; ++w) {
            need_in += s_need[w];
            units_in += s_units[w];
        }
        if (r < rows) {
            uint32_t unit = 0;
            if (need) {
                page = (int)(base_p + c_pages + need_in - 1);
                slot = 0;
                unit = (uint32_t)(base_u + c_units + units_in - units);
                a.new_pages[r] = (int32_t)unit;
            }
            a.dest_page[r] = page;
            a.dest_slot[r] = slot;
            if (t0 == 0) {
                f_page = page;
                f_slot = slot;
                f_unit = unit;
            }
        }
        __syncthreads();
        if (tid == 1023) {   // the tile's totals
            c_pages += need_in;
            c_units += units_in;
        }
        __syncthreads();
    }
    if (tid == 0 && (base_p + c_pages > a.page_capacity || base_u + c_units > a.arena_capacity16)) s_nospace = 1;
    __syncthreads();
    if (s_nospace) {
        if (tid == 0) set_status(a.status, ADA_ENOSPC);
        return;
    }
    for (int r = tid; r < rows; r += 1024) {
        int tau, page, slot, np;
        uint32_t unit;
        if (r == tid) {   // the first tile's row: everything is in registers
            tau = tau0;
            page = f_page;
            slot = f_slot;
            np = np0;
            unit = f_unit;
        } else {
            tau = a.tier[r];
            page = a.dest_page[r];
            slot = a.dest_slot[r];
            np = a.num_pages[r];
            unit = (uint32_t)a.new_pages[r];
        }
        if (slot == 0) {   // a new page (an open page always holds at least one token)
            ada_page_meta_t m;
            m.tier = (uint8_t)tau;
            m.count = 1;
            m.reserved = 0;
            m.code_off16 = unit;
            a.page_meta[page] = m;
            a.page_table[(size_t)r * a.maxp + np] = page;
            a.num_pages[r] = np + 1;
            a.open_page[r * kNumTiers + tau] = P > 1 ? page : -1;
        } else {
            a.page_meta[page].count = (uint8_t)(slot + 1);
            if (slot + 1 == P) a.open_page[r * kNumTiers + tau] = -1;
        }
    }
    if (tid == 0) {
        a.alloc[0] = base_p + c_pages;
        a.alloc[1] = base_u + c_units;
    }
}

// single work-group: place every request in order (tiles of 1024)
__global__ __launch_bounds__(1024) void append_book_kernel(AppendKernelArgs k) {
    const AppendLaunch &a = k.a;
    __shared__ int s_key[1024], s_row[1024], s_rank[1024], s_alloc[1024], s_page[1024], s_off[1024];
    __shared__ long long s_scan_p[16], s_scan_u[16];   // per-wavefront totals of the tile scan
    __shared__ long long base_p, base_u;
    __shared__ int nnew, bad;
    const int tid = threadIdx.x;
    if (tid == 0) {
        bad = read_status(a.status);
        if (!bad && (a.alloc[0] + a.totals[0] > a.page_capacity || a.alloc[1] + a.totals[1] > a.arena_capacity16)) {
            set_status(a.status, ADA_ENOSPC);
            bad = 1;
        }
        base_p = a.alloc[0];
        base_u = a.alloc[1];
        nnew = 0;
    }
    __syncthreads();
    if (bad) return;
    const int P = a.P;
    for (int t0 = 0; t0 < a.n; t0 += 1024) {
        const int nt = min(1024, a.n - t0);
        const int i = t0 + tid;
        const bool act = tid < nt;
        int key = -1, row = -1, tau = 0;
        if (act) {
            tau = a.tier[i];
            row = req_seq(a, i) * a.Hkv + req_head(a, i);
            key = row * kNumTiers + tau;
        }
        s_key[tid] = key;
        s_row[tid] = row;
        __syncthreads();
        int rank = 0;
        bool last_in_tile = true;
        if (act) {
            for (int j = 0; j < nt; ++j) {
                if (s_key[j] != key) continue;
                if (j < tid) ++rank;
                else if (j > tid) last_in_tile = false;
            }
        }
        int r = 0, pos = 0, alloc = 0;
        if (act) {
            r = a.key_done[key] + rank;
            pos = a.key_c0[key] + r;
            alloc = (pos % P) == 0;
        }
        s_rank[tid] = rank;
        s_alloc[tid] = alloc;
        // inclusive scans of new pages and code units over the tile: within
        // each wavefront by shuffles, then the wavefronts' totals through LDS
        const int lane = tid & 63, wv = tid >> 6;
        long long in_p = alloc, in_u = alloc ? block16(tau, P) : 0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const long long vp = __shfl_up(in_p, o, 64), vu = __shfl_up(in_u, o, 64);
            if (lane >= o) {
                in_p += vp;
                in_u += vu;
            }
        }
        if (lane == 63) {
            s_scan_p[wv] = in_p;
            s_scan_u[wv] = in_u;
        }
        __syncthreads();
        for (int w = 0; w < wv; ++w) {
            in_p += s_scan_p[w];
            in_u += s_scan_u[w];
        }
        const long long ex_p = in_p - alloc;
        const long long ex_u = in_u - (alloc ? block16(tau, P) : 0);
        s_page[tid] = alloc ? (int)(base_p + ex_p) : -1;
        s_off[tid] = alloc ? (int)(base_u + ex_u) : -1;
        __syncthreads();
        int page = -1, off16 = 0;
        if (act) {
            if (alloc) {
                page = s_page[tid];
                off16 = s_off[tid];
            } else {
                const int want = rank - (pos % P);
                if (want >= 0) {
                    for (int j = 0; j < nt; ++j)
                        if (s_key[j] == key && s_rank[j] == want) {
                            page = s_page[j];
                            off16 = s_off[j];
                            break;
                        }
                } else {
                    page = a.key_page[key];
                    off16 = k.key_off[key];
                }
            }
        }
        // row positions of newly opened pages
        int rowrank = 0;
        bool last_alloc_of_row = true;
        if (act && alloc) {
            for (int j = 0; j < nt; ++j) {
                if (!s_alloc[j] || s_row[j] != row) continue;
                if (j < tid) ++rowrank;
                else if (j > tid) last_alloc_of_row = false;
            }
        }
        const int np_row = act ? a.num_pages[row] : 0;
        __syncthreads();   // every read of carried state precedes the updates below
        if (act) {
            if (alloc) {
                a.page_table[(size_t)row * a.maxp + np_row + rowrank] = page;
                a.new_pages[nnew + ex_p] = page;
            }
            a.dest_page[i] = page;
            a.dest_slot[i] = pos % P;
            const bool last_overall = (r == a.key_cnt[key] - 1);
            if ((pos + 1) % P == 0 || last_overall) {
                ada_page_meta_t m;
                m.tier = (uint8_t)tau;
                m.count = (uint8_t)(pos % P + 1);
                m.reserved = 0;
                m.code_off16 = (uint32_t)off16;
                a.page_meta[page] = m;
            }
            if (last_in_tile) {
                a.key_done[key] = r + 1;
                a.key_page[key] = page;
                k.key_off[key] = off16;
            }
            if (last_overall) a.open_page[key] = ((pos + 1) % P == 0) ? -1 : page;
            if (alloc && last_alloc_of_row) a.num_pages[row] = np_row + rowrank + 1;
        }
        __syncthreads();
        if (tid == 1023) {   // the tile's totals
            base_p += in_p;
            base_u += in_u;
            nnew += (int)in_p;
        }
        __syncthreads();
    }
    if (tid == 0) {
        a.alloc[0] = base_p;
        a.alloc[1] = base_u;
        a.n_new[0] = 0;          // list start
        a.n_new[1] = nnew;       // list length
    }
}

__global__ void cache_init_kernel(int32_t rows, int32_t *num_pages, int32_t *open_page, int64_t *alloc,
                                  int32_t *status, int32_t *row_order) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < rows * kNumTiers; i += gridDim.x * blockDim.x) {
        open_page[i] = -1;
        if (i < rows) {
            num_pages[i] = 0;
            if (row_order) row_order[i] = i;
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        alloc[0] = 0;
        alloc[1] = 0;
        *status = 0;
    }
}

// Cache check: every row's page count within the row's table, every listed
// page id within the pool, and each such page's metadata well formed (a known
// tier, 1..P tokens, zero reserved field, code block inside the arena).  A
// page's metadata is read only after its id has been range-checked; nothing
// outside the buffers is read.  Any failure sets the status word to
// ADA_EINVAL.  One work-group per row (grid-stride).
__global__ __launch_bounds__(256) void validate_kernel(int32_t rows, int32_t maxp, int64_t page_capacity,
                                                       int64_t arena16, int32_t P, int32_t n_tiers,
                                                       const int32_t *num_pages, const int32_t *page_table,
                                                       const ada_page_meta_t *page_meta, int32_t *status) {
    for (int row = blockIdx.x; row < rows; row += gridDim.x) {
        const int np = num_pages[row];
        if (np < 0 || np > maxp) {
            if (threadIdx.x == 0) enc::set_status(status, ADA_EINVAL);
            continue;
        }
        for (int i = threadIdx.x; i < np; i += blockDim.x) {
            const int pid = page_table[(size_t)row * maxp + i];
            if (pid < 0 || (int64_t)pid >= page_capacity) {
                enc::set_status(status, ADA_EINVAL);
                continue;
            }
            const ada_page_meta_t m = page_meta[pid];
            const bool ok = m.tier < n_tiers && m.count >= 1 && m.count <= P && m.reserved == 0 &&
                            (int64_t)m.code_off16 + block16(m.tier, P) <= arena16;
            if (!ok) enc::set_status(status, ADA_EINVAL);
        }
    }
}

// The row order must be a permutation of 0..rows-1: every entry in range
// (else the decode would read rows outside the tables), and, for up to
// 65536 rows, none twice (a bitmap in LDS).  One work-group.
__global__ __launch_bounds__(1024) void validate_order_kernel(int32_t rows, const int32_t *row_order,
                                                             int32_t *status) {
    __shared__ uint32_t seen[2048];
    const bool dup_check = rows <= 65536;
    for (int i = threadIdx.x; i < 2048; i += 1024) seen[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < rows; i += 1024) {
        const int r = row_order[i];
        if (r < 0 || r >= rows) {
            enc::set_status(status, ADA_EINVAL);
            continue;
        }
        if (dup_check && (atomicOr(&seen[r >> 5], 1u << (r & 31)) >> (r & 31)) & 1u) enc::set_status(status, ADA_EINVAL);
    }
}

__global__ void fill_i32_kernel(int32_t *p, int64_t n, int32_t v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

inline int grid_for(int64_t n, int per_block, int cap = 8192) {
    int64_t g = (n + per_block - 1) / per_block;
    if (g < 1) g = 1;
    return (int)(g > cap ? cap : g);
}

}  // namespace

uint16_t host_f64_to_f16(double x) { return f64_to_f16_rne_sat(x); }

hipError_t launch_encode_write(const EncodeLaunch &a, hipStream_t s) {
    hipLaunchKernelGGL(encode_write_kernel, dim3(grid_for(a.n, 4, 16384)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_zero_pages(const int32_t *pages, const int32_t *n_pages, int64_t max_n,
                             const ada_page_meta_t *page_meta, uint8_t *arena, int32_t P, const int32_t *status,
                             hipStream_t s) {
    hipLaunchKernelGGL(zero_pages_kernel, dim3(grid_for(max_n, 1, 4096)), dim3(256), 0, s, pages, n_pages,
                       page_meta, arena, P, status);
    return hipGetLastError();
}

hipError_t launch_validate(int32_t rows, int32_t maxp, int64_t page_capacity, int64_t arena16, int32_t P,
                           int32_t n_tiers, const int32_t *num_pages, const int32_t *page_table,
                           const ada_page_meta_t *page_meta, const int32_t *row_order, int32_t order_rows,
                           int32_t *status, hipStream_t s) {
    hipLaunchKernelGGL(validate_kernel, dim3(grid_for(rows, 1, 4096)), dim3(256), 0, s, rows, maxp, page_capacity,
                       arena16, P, n_tiers, num_pages, page_table, page_meta, status);
    if (row_order && order_rows > 0)
        hipLaunchKernelGGL(validate_order_kernel, dim3(1), dim3(1024), 0, s, order_rows, row_order, status);
    return hipGetLastError();
}

hipError_t launch_cache_init(int32_t rows, int32_t *num_pages, int32_t *open_page, int64_t *alloc, int32_t *status,
                             int32_t *row_order, hipStream_t s) {
    hipLaunchKernelGGL(cache_init_kernel, dim3(grid_for((int64_t)rows * kNumTiers, 256, 1024)), dim3(256), 0, s, rows,
                       num_pages, open_page, alloc, status, row_order);
    return hipGetLastError();
}

hipError_t launch_pack(const PackLaunch &a, hipStream_t s) {
    const int rows = a.B * a.Hkv;
    hipLaunchKernelGGL(pack_count_kernel, dim3(a.n_tiles, rows), dim3(256), 0, s, a);
    hipLaunchKernelGGL(pack_rowscan_kernel, dim3(rows), dim3(64), 0, s, a);
    hipLaunchKernelGGL(pack_plan_kernel, dim3(1), dim3(1024), 0, s, a, a.n_new);
    hipLaunchKernelGGL(pack_pages_kernel, dim3(rows), dim3(256), 0, s, a);
    hipLaunchKernelGGL(pack_dest_kernel, dim3(a.n_tiles, rows), dim3(256), 0, s, a);
    const int64_t max_pages = (int64_t)rows * a.maxp;
    if (a.src_page_table) {   // re-pack: the transcoder writes every byte of each new page
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        const dim3 grid(grid_for(a.src_of_slot_pages, 1, 8 * cus));   // about one round of resident work-groups
        hipLaunchKernelGGL(repack_order_kernel, dim3(grid_for(a.src_of_slot_pages, 256, 1 << 20)), dim3(256), 0, s, a);
        if (a.P == 16) hipLaunchKernelGGL(transcode_pages_pipe_kernel<16>, grid, dim3(128), 0, s, a);
        else hipLaunchKernelGGL(transcode_pages_kernel<32>, grid, dim3(128), 0, s, a);
        if (a.row_order)
            hipLaunchKernelGGL(row_order_kernel, dim3(1), dim3(1024), 0, s, a.rows_total, (const int32_t *)a.num_pages,
                               a.row_order);
        return hipGetLastError();
    }
    // pack from keys: the page writer encodes and writes every byte of each
    // new page
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    const dim3 grid(grid_for(max_pages < a.item_slot_pages ? max_pages : a.item_slot_pages, 1, 16 * cus));
    if (a.P == 16) hipLaunchKernelGGL(pack_write_pages_kernel<16>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(pack_write_pages_kernel<32>, grid, dim3(256), 0, s, a);
    if (a.row_order)
        hipLaunchKernelGGL(row_order_kernel, dim3(1), dim3(1024), 0, s, a.rows_total, (const int32_t *)a.num_pages,
                           a.row_order);
    return hipGetLastError();
}

hipError_t launch_append_rows(const AppendLaunch &a, hipStream_t s) {
    hipLaunchKernelGGL(append_rows_kernel, dim3(1), dim3(1024), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_append(const AppendLaunch &a, bool encode, hipStream_t s) {
    AppendKernelArgs k;
    k.a = a;
    // key_off lives right after key_page in the workspace (same length)
    const int nkeys = a.num_seqs * a.Hkv * kNumTiers;
    k.key_off = a.key_page + nkeys;
    hipLaunchKernelGGL(append_init_kernel, dim3(grid_for(nkeys, 256, 1024)), dim3(256), 0, s, k);
    hipLaunchKernelGGL(append_validate_kernel, dim3(grid_for(a.n, 4, 4096)), dim3(256), 0, s, a);
    hipLaunchKernelGGL(append_capacity_kernel, dim3(grid_for((int64_t)a.num_seqs * a.Hkv, 256, 1024)), dim3(256),
                       0, s, a);
    hipLaunchKernelGGL(append_book_kernel, dim3(1), dim3(1024), 0, s, k);
    hipLaunchKernelGGL(zero_pages_kernel, dim3(grid_for(a.n, 1, 4096)), dim3(256), 0, s,
                       (const int32_t *)a.new_pages, (const int32_t *)a.n_new, (const ada_page_meta_t *)a.page_meta,
                       a.arena, a.P, (const int32_t *)a.status);
    if (!encode) return hipGetLastError();
    EncodeLaunch e;
    e.keys = a.keys;
    e.values = a.values;
    e.n = a.n;
    e.dest_page = a.dest_page;
    e.dest_slot = a.dest_slot;
    e.page_meta = a.page_meta;
    e.arena = a.arena;
    e.P = a.P;
    e.status = a.status;
    e.half_pairs = a.half_pairs;
    hipLaunchKernelGGL(encode_write_kernel, dim3(grid_for(e.n, 4, 16384)), dim3(256), 0, s, e);
    return hipGetLastError();
}

}  // namespace ada
