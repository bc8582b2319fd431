// rdr.hip -- Rate-Distortion Retention: keep/drop and tier per (KV head,
// position) under a per-sequence byte budget, on gfx950.
//
// Method: "SPHERICAL KV" (arXiv 2605.18856), Abstract: RDR gives each
// (token, KV head) either a precision tier or a drop, within a byte budget.
// Rate / distortion model and order (this library's reading):
// upgrade steps drop -> tier_1 -> tier_2 ... (tiers in rate order) with cost
// dR_k bytes and priority p = w * (dD_k / dR_k) in fp64; the steps taken are
// the longest prefix of the order (p desc, position desc, head asc, step asc)
// whose byte total fits the budget.
//
// GPU formulation: the cut of that prefix is found by a radix select on the
// 64-bit pattern of p (monotone for p >= 0): eight passes each build a
// 256-bin histogram of step bytes among steps that share the already chosen
// high bytes, and pick the bin where the running byte total crosses the
// budget.  All byte sums are 64-bit integers, so the result does not depend
// on summation order.  Each pass's cut is found at the start of the next
// pass's histogram kernel, by every work-group from the finished histogram
// (one launch per pass, plus one for the last cut).  Steps whose p equals
// the selected key are then taken in (position desc, head asc, step asc)
// order by a tiled prefix scan.
#include "ada_internal.h"

namespace ada {
namespace {

__device__ inline void set_status(int32_t *status, int code) { atomicCAS(status, 0, code); }

// steps item i may take
__device__ inline int item_steps(const RdrLaunch &a, int64_t i) {
    return a.cap ? min(a.n_steps, (int)a.cap[i]) : a.n_steps;
}

// radix-select state of sequence b after v passes (see RdrLaunch)
struct SelState {
    unsigned long long prefix;   // the chosen key bytes
    long long above;             // bytes of the steps above them
    int all_fit;                 // every step fits: nothing to select
};

__device__ inline SelState load_state(const RdrLaunch &a, int v, int b) {
    const size_t k = (size_t)v * a.B + b;
    return SelState{a.prefix[k], a.above[k], a.all_fit[k]};
}

__device__ inline void store_state(const RdrLaunch &a, int v, int b, const SelState &st) {
    const size_t k = (size_t)v * a.B + b;
    a.prefix[k] = st.prefix;
    a.above[k] = st.above;
    a.all_fit[k] = st.all_fit;
}

__device__ inline unsigned long long prio_key(float w, double c) {
    double p = (double)w * c;
    unsigned long long u;
    __builtin_memcpy(&u, &p, 8);
    return u & 0x7FFFFFFFFFFFFFFFull;   // -0.0 (utility -0.0) orders as +0.0
}

__global__ __launch_bounds__(256) void rdr_validate_kernel(RdrLaunch a) {
    const int64_t total = (int64_t)a.B * a.Hkv * a.stride;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t t = i % a.stride;
        const int b = (int)(i / ((int64_t)a.Hkv * a.stride));
        a.tie_sel[i] = 0;
        if (t >= a.ctx_len_dev[b]) continue;
        const float w = a.utility[i];
        if (!(isfinite(w) && w >= 0.f)) set_status(a.status, ADA_EINVAL);
    }
    if (blockIdx.x == 0) {
        for (int k = threadIdx.x; k < kRdrPasses * a.B * 256; k += 256) a.hist[k] = 0ull;
        for (int b = threadIdx.x; b < a.B; b += 256) store_state(a, 0, b, SelState{0ull, 0, 0});
    }
}

// The cut digit of pass `pass` for sequence b, from that pass's finished
// histogram: walking bins from the highest, the first whose bytes no longer
// fit beside those above it.  Bins' suffix sums grow as the digit falls, so
// the chosen bin is the highest digit whose inclusive suffix overshoots.
// Run by a whole work-group of 256 threads; every thread gets the state
// after the pass.
__device__ SelState select_digit(const RdrLaunch &a, int pass, int b, long long (&suf)[256], int &n_over) {
    const SelState s0 = load_state(a, pass, b);
    const int v = threadIdx.x;
    const bool active = s0.all_fit == 0 && *a.status == 0;
    suf[v] = (long long)a.hist[((size_t)pass * a.B + b) * 256 + v];
    if (v == 0) n_over = 0;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {   // suf[v] = sum of bins >= v
        const long long u = v + off < 256 ? suf[v + off] : 0;
        __syncthreads();
        suf[v] += u;
        __syncthreads();
    }
    if (s0.above + suf[v] > a.budget_dev[b]) atomicAdd(&n_over, 1);
    __syncthreads();
    const int chosen = n_over - 1;   // bins 0..chosen overshoot
    SelState s1 = s0;
    if (active) {
        if (chosen < 0) {
            s1.all_fit = 1;   // every remaining step fits (possible on the first pass only)
        } else {
            s1.above = s0.above + (chosen < 255 ? suf[chosen + 1] : 0);
            s1.prefix = (s0.prefix << 8) | (unsigned long long)chosen;
        }
    }
    __syncthreads();   // suf and n_over are free again
    return s1;
}

// histogram of step bytes per next digit, for steps matching the prefix
__global__ __launch_bounds__(256) void rdr_hist_kernel(RdrLaunch a, int pass) {
    __shared__ unsigned long long h[256];
    __shared__ long long suf[256];
    __shared__ int n_over;
    const int b = blockIdx.y;
    // the state before this pass: the previous pass's cut, found here from
    // its histogram by every work-group alike; one of them records it
    SelState st;
    if (pass == 0) {
        st = load_state(a, 0, b);
    } else {
        st = select_digit(a, pass - 1, b, suf, n_over);
        if (blockIdx.x == 0 && threadIdx.x == 0) store_state(a, pass, b, st);
    }
    h[threadIdx.x] = 0ull;
    __syncthreads();
    const int ctx = a.ctx_len_dev[b];
    const bool skip = st.all_fit != 0 || *a.status != 0;
    const unsigned long long pre = st.prefix;
    const int shift_hi = 64 - 8 * pass, shift_dig = 56 - 8 * pass;
    if (!skip) {
        // Wavefront-uniform loop.  When every taking lane of a step falls
        // into one bin (usual in the first pass, where the digit is the
        // exponent's top bits) one LDS atomic adds them all.
        const int lane = threadIdx.x & 63;
        const int64_t items = (int64_t)a.Hkv * ctx;
        const int64_t stride = (int64_t)gridDim.x * 256;
        for (int64_t base = (int64_t)blockIdx.x * 256 + (threadIdx.x & ~63); base < items; base += stride) {
            const int64_t it = base + lane;
            float w = 0.f;
            int nk = 0;
            if (it < items) {
                const int h_ = (int)(it / ctx);
                const int t = (int)(it % ctx);
                const int64_t i = ((int64_t)b * a.Hkv + h_) * a.stride + t;
                w = a.utility[i];
                nk = item_steps(a, i);
            }
            for (int k = 0; k < a.n_steps; ++k) {
                const unsigned long long key = prio_key(w, a.c[k]);
                const bool take = k < nk && (pass == 0 || (key >> shift_hi) == pre);
                const int bin = (int)((key >> shift_dig) & 255ull);
                const unsigned long long act = __ballot(take);
                if (act == 0ull) continue;
                const int leader = __ffsll((long long)act) - 1;
                const int lb = __shfl(bin, leader);
                const unsigned long long same = __ballot(take && bin == lb);
                if (same == act) {
                    if (lane == leader)
                        atomicAdd(&h[lb], (unsigned long long)__popcll(same) * (unsigned long long)a.dR[k]);
                } else if (take) {
                    atomicAdd(&h[bin], (unsigned long long)a.dR[k]);
                }
            }
        }
    }
    __syncthreads();
    if (!skip && h[threadIdx.x]) atomicAdd(&a.hist[((size_t)pass * a.B + b) * 256 + threadIdx.x], h[threadIdx.x]);
}

// The last pass's cut: the state after every pass (v = kRdrPasses).
__global__ __launch_bounds__(256) void rdr_select_kernel(RdrLaunch a) {
    __shared__ long long suf[256];
    __shared__ int n_over;
    const int b = blockIdx.x;
    const SelState st = select_digit(a, kRdrPasses - 1, b, suf, n_over);
    if (threadIdx.x == 0) store_state(a, kRdrPasses, b, st);
}

// Steps whose key equals the selected key, taken in (position desc, head
// asc, step asc) order: the longest prefix of that order fitting the budget
// left after the steps above the key.  Tie order index ii runs over
// (t = ctx - 1 - ii / Hkv, h = ii % Hkv); tiles of kRdrTieTile indices, four
// consecutive indices per thread.  Three passes: tie bytes per tile, an
// exclusive prefix over the tiles of a sequence, then each tile scans its own
// items from its prefix.
__device__ inline long long tie_bytes(const RdrLaunch &a, int b, int ctx, int64_t ii, unsigned long long T,
                                      float *w_out, int *nk_out, int64_t *i_out) {
    const int t = ctx - 1 - (int)(ii / a.Hkv), h_ = (int)(ii % a.Hkv);
    const int64_t i = ((int64_t)b * a.Hkv + h_) * a.stride + t;
    const float w = a.utility[i];
    const int nk = item_steps(a, i);
    long long bytes = 0;
    for (int k = 0; k < nk; ++k)
        if (prio_key(w, a.c[k]) == T) bytes += a.dR[k];
    *w_out = w;
    *nk_out = nk;
    *i_out = i;
    return bytes;
}

// the selection after every pass
__device__ inline SelState final_state(const RdrLaunch &a, int b) { return load_state(a, kRdrPasses, b); }
__device__ inline bool tie_active(const RdrLaunch &a, int b) { return final_state(a, b).all_fit == 0 && *a.status == 0; }

__global__ __launch_bounds__(256) void rdr_tie_sum_kernel(RdrLaunch a, int64_t tiles_per_seq) {
    __shared__ long long red[4];
    const int b = blockIdx.y;
    const int64_t tile = blockIdx.x;
    if (!tie_active(a, b)) return;
    const int ctx = a.ctx_len_dev[b];
    const int64_t items = (int64_t)a.Hkv * ctx;
    if (tile * kRdrTieTile >= items) return;
    const unsigned long long T = final_state(a, b).prefix;
    long long sum = 0;
    for (int k = 0; k < 4; ++k) {
        const int64_t ii = tile * kRdrTieTile + threadIdx.x * 4 + k;
        float w;
        int nk;
        int64_t i;
        if (ii < items) sum += tie_bytes(a, b, ctx, ii, T, &w, &nk, &i);
    }
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sum;
    __syncthreads();
    if (threadIdx.x == 0) a.tie_tile[b * tiles_per_seq + tile] = red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(1024) void rdr_tie_scan_kernel(RdrLaunch a, int64_t tiles_per_seq) {
    __shared__ long long sc[1024];
    __shared__ long long carry;
    const int b = blockIdx.x;
    if (!tie_active(a, b)) return;
    const int64_t tiles = rdr_tie_tiles((int64_t)a.Hkv * a.ctx_len_dev[b]);
    long long *tt = a.tie_tile + b * tiles_per_seq;
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    for (int64_t base = 0; base < tiles; base += 1024) {
        const int64_t j = base + threadIdx.x;
        const long long v = j < tiles ? tt[j] : 0;
        sc[threadIdx.x] = v;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const long long u = threadIdx.x >= off ? sc[threadIdx.x - off] : 0;
            __syncthreads();
            sc[threadIdx.x] += u;
            __syncthreads();
        }
        if (j < tiles) tt[j] = carry + sc[threadIdx.x] - v;
        __syncthreads();
        if (threadIdx.x == 0) carry += sc[1023];
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void rdr_tie_apply_kernel(RdrLaunch a, int64_t tiles_per_seq) {
    __shared__ long long sc[256];
    const int b = blockIdx.y;
    const int64_t tile = blockIdx.x;
    if (!tie_active(a, b)) return;
    const int ctx = a.ctx_len_dev[b];
    const int64_t items = (int64_t)a.Hkv * ctx;
    if (tile * kRdrTieTile >= items) return;
    const long long rem = a.budget_dev[b] - final_state(a, b).above;
    const long long off = a.tie_tile[b * tiles_per_seq + tile];
    if (off >= rem) return;   // every step costs at least one byte: nothing of this tile fits
    const unsigned long long T = final_state(a, b).prefix;
    float w[4];
    int nk[4];
    int64_t idx[4];
    long long bytes[4], mine = 0;
    for (int k = 0; k < 4; ++k) {
        const int64_t ii = tile * kRdrTieTile + threadIdx.x * 4 + k;
        bytes[k] = ii < items ? tie_bytes(a, b, ctx, ii, T, &w[k], &nk[k], &idx[k]) : 0;
        mine += bytes[k];
    }
    sc[threadIdx.x] = mine;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        const long long u = threadIdx.x >= o ? sc[threadIdx.x - o] : 0;
        __syncthreads();
        sc[threadIdx.x] += u;
        __syncthreads();
    }
    long long cum = off + sc[threadIdx.x] - mine;
    for (int k = 0; k < 4; ++k) {
        if (bytes[k] == 0) continue;
        long long c = cum;
        int taken = 0;
        for (int j = 0; j < nk[k]; ++j) {
            if (prio_key(w[k], a.c[j]) != T) continue;
            if (c + a.dR[j] > rem) break;
            c += a.dR[j];
            ++taken;
        }
        a.tie_sel[idx[k]] = (uint8_t)taken;
        cum += bytes[k];
    }
}

__global__ __launch_bounds__(256) void rdr_final_kernel(RdrLaunch a) {
    const int64_t total = (int64_t)a.B * a.Hkv * a.stride;
    if (*a.status != 0) return;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t t = i % a.stride;
        const int b = (int)(i / ((int64_t)a.Hkv * a.stride));
        int8_t out = -1;
        if (t < a.ctx_len_dev[b]) {
            int n;
            const int nk = item_steps(a, i);
            const SelState st = final_state(a, b);
            if (st.all_fit) {
                n = nk;
            } else {
                const unsigned long long T = st.prefix;
                const float w = a.utility[i];
                n = a.tie_sel[i];
                for (int k = 0; k < nk; ++k) n += prio_key(w, a.c[k]) > T ? 1 : 0;
            }
            out = n ? (int8_t)a.step_tier[n - 1] : (int8_t)-1;
        }
        a.tier_out[i] = out;
    }
}

__global__ __launch_bounds__(256) void repack_items_kernel(RepackItemsLaunch a) {
    const int64_t S = (int64_t)a.src_maxp * a.P;
    const int64_t n = (int64_t)a.B * a.Hkv * S;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t row = i / S, t = i % S;
        const int ip = (int)(t / a.P), slot = (int)(t % a.P);
        float u = 0.f;
        int8_t cap = 0;
        if (ip < a.num_pages[row]) {
            const int page = a.page_table[row * a.src_maxp + ip];
            const ada_page_meta_t m = a.page_meta[page];
            if (slot < m.count) {
                u = a.util[(size_t)page * a.P + slot];
                cap = a.level_of_tier[m.tier];
            }
        }
        a.util_v[i] = u;
        a.cap_v[i] = cap;
        if (i < a.B) a.ctx_v[i] = (int32_t)S;
    }
}

}  // namespace

hipError_t launch_repack_items(const RepackItemsLaunch &a, hipStream_t s) {
    const int64_t n = (int64_t)a.B * a.Hkv * a.src_maxp * a.P;
    int g = (int)((n + 255) / 256);
    g = g < 1 ? 1 : (g > 8192 ? 8192 : g);
    hipLaunchKernelGGL(repack_items_kernel, dim3(g), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_rdr(const RdrLaunch &a, hipStream_t s) {
    const int64_t total = (int64_t)a.B * a.Hkv * a.stride;
    int g = (int)((total + 255) / 256);
    g = g < 1 ? 1 : (g > 8192 ? 8192 : g);
    hipLaunchKernelGGL(rdr_validate_kernel, dim3(g), dim3(256), 0, s, a);
    const int64_t per_seq = (int64_t)a.Hkv * a.stride;
    // about eight items per thread, at most ~4096 work-groups in all: every
    // work-group adds its non-empty bins to the global histogram atomically
    const int64_t gcap = 4096 / a.B > 1 ? 4096 / a.B : 1;
    int64_t gx64 = (per_seq + 2047) / 2048;
    const int gx = (int)(gx64 < 1 ? 1 : (gx64 > gcap ? gcap : gx64));
    for (int pass = 0; pass < kRdrPasses; ++pass)
        hipLaunchKernelGGL(rdr_hist_kernel, dim3(gx, a.B), dim3(256), 0, s, a, pass);
    hipLaunchKernelGGL(rdr_select_kernel, dim3(a.B), dim3(256), 0, s, a);
    const int64_t tiles = rdr_tie_tiles(per_seq);
    hipLaunchKernelGGL(rdr_tie_sum_kernel, dim3((unsigned)tiles, a.B), dim3(256), 0, s, a, tiles);
    hipLaunchKernelGGL(rdr_tie_scan_kernel, dim3(a.B), dim3(1024), 0, s, a, tiles);
    hipLaunchKernelGGL(rdr_tie_apply_kernel, dim3((unsigned)tiles, a.B), dim3(256), 0, s, a, tiles);
    hipLaunchKernelGGL(rdr_final_kernel, dim3(g), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace ada
