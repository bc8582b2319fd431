// rdr.hip -- Rate-Distortion Retention: keep/drop and tier per (KV head,
// position) under a per-sequence byte budget, on gfx950.
//
// Method: "SPHERICAL KV" (arXiv 2605.18856), Abstract: RDR jointly chooses
// keep/drop decisions and precision tiers per token and head under a fixed
// budget.  Rate / distortion model and order (this library's reading):
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
// on summation order.  Steps whose p equals the selected key are then taken
// in (position desc, head asc, step asc) order by a single work-group scan.
#include "ada_internal.h"

namespace ada {
namespace {

__device__ inline void set_status(int32_t *status, int code) { atomicCAS(status, 0, code); }

// steps item i may take
__device__ inline int item_steps(const RdrLaunch &a, int64_t i) {
    return a.cap ? min(a.n_steps, (int)a.cap[i]) : a.n_steps;
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
        for (int k = threadIdx.x; k < a.B * 256; k += 256) a.hist[k] = 0ull;
        for (int b = threadIdx.x; b < a.B; b += 256) {
            a.prefix[b] = 0ull;
            a.above[b] = 0;
            a.all_fit[b] = 0;
        }
    }
}

// histogram of step bytes per next digit, for steps matching the prefix
__global__ __launch_bounds__(256) void rdr_hist_kernel(RdrLaunch a, int pass) {
    __shared__ unsigned long long h[256];
    const int b = blockIdx.y;
    h[threadIdx.x] = 0ull;
    __syncthreads();
    const int ctx = a.ctx_len_dev[b];
    const bool skip = a.all_fit[b] != 0 || *a.status != 0;
    const unsigned long long pre = a.prefix[b];
    const int shift_hi = 64 - 8 * pass, shift_dig = 56 - 8 * pass;
    if (!skip) {
        const int64_t items = (int64_t)a.Hkv * ctx;
        for (int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x; it < items; it += (int64_t)gridDim.x * 256) {
            const int h_ = (int)(it / ctx);
            const int t = (int)(it % ctx);
            const int64_t i = ((int64_t)b * a.Hkv + h_) * a.stride + t;
            const float w = a.utility[i];
            const int nk = item_steps(a, i);
            for (int k = 0; k < nk; ++k) {
                const unsigned long long key = prio_key(w, a.c[k]);
                if (pass > 0 && (key >> shift_hi) != pre) continue;
                atomicAdd(&h[(key >> shift_dig) & 255ull], (unsigned long long)a.dR[k]);
            }
        }
    }
    __syncthreads();
    if (!skip && h[threadIdx.x]) atomicAdd(&a.hist[b * 256 + threadIdx.x], h[threadIdx.x]);
}

__global__ void rdr_select_kernel(RdrLaunch a, int pass) {
    const int b = blockIdx.x;
    if (threadIdx.x != 0) return;
    unsigned long long *hb = a.hist + b * 256;
    if (a.all_fit[b] == 0 && *a.status == 0) {
        const long long budget = a.budget_dev[b];
        long long above = a.above[b];
        int chosen = -1;
        for (int v = 255; v >= 0; --v) {
            const long long hv = (long long)hb[v];
            if (above + hv <= budget) {
                above += hv;
            } else {
                chosen = v;
                break;
            }
        }
        if (chosen < 0) {
            a.all_fit[b] = 1;   // every remaining step fits (possible on the first pass only)
        } else {
            a.above[b] = above;
            a.prefix[b] = (a.prefix[b] << 8) | (unsigned long long)chosen;
        }
    }
    for (int v = 0; v < 256; ++v) hb[v] = 0ull;
}

// steps whose key equals the selected key, in (position desc, head asc,
// step asc) order: longest prefix fitting the remaining budget
__global__ __launch_bounds__(1024) void rdr_tie_kernel(RdrLaunch a) {
    __shared__ long long sc[1024];
    __shared__ long long carry;
    __shared__ int stop;
    const int b = blockIdx.x;
    if (a.all_fit[b] != 0 || *a.status != 0) return;
    const unsigned long long T = a.prefix[b];
    const long long rem = a.budget_dev[b] - a.above[b];
    const int ctx = a.ctx_len_dev[b];
    const int64_t items = (int64_t)a.Hkv * ctx;
    if (threadIdx.x == 0) {
        carry = 0;
        stop = 0;
    }
    __syncthreads();
    for (int64_t base = 0; base < items; base += 1024) {
        const int64_t ii = base + threadIdx.x;
        int h_ = 0, t = 0;
        long long bytes = 0;
        float w = 0.f;
        int nk = 0;
        if (ii < items) {
            t = ctx - 1 - (int)(ii / a.Hkv);
            h_ = (int)(ii % a.Hkv);
            const int64_t i = ((int64_t)b * a.Hkv + h_) * a.stride + t;
            w = a.utility[i];
            nk = item_steps(a, i);
            for (int k = 0; k < nk; ++k)
                if (prio_key(w, a.c[k]) == T) bytes += a.dR[k];
        }
        sc[threadIdx.x] = bytes;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            long long v = threadIdx.x >= off ? sc[threadIdx.x - off] : 0;
            __syncthreads();
            sc[threadIdx.x] += v;
            __syncthreads();
        }
        if (ii < items && bytes > 0) {
            long long cum = carry + sc[threadIdx.x] - bytes;
            int taken = 0;
            for (int k = 0; k < nk; ++k) {
                if (prio_key(w, a.c[k]) != T) continue;
                if (cum + a.dR[k] > rem) break;
                cum += a.dR[k];
                ++taken;
            }
            a.tie_sel[((int64_t)b * a.Hkv + h_) * a.stride + t] = (uint8_t)taken;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            carry += sc[1023];
            if (carry > rem) stop = 1;
        }
        __syncthreads();
        if (stop) break;
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
            if (a.all_fit[b]) {
                n = nk;
            } else {
                const unsigned long long T = a.prefix[b];
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
    int gx = (int)((per_seq + 255) / 256);
    gx = gx < 1 ? 1 : (gx > 2048 ? 2048 : gx);
    for (int pass = 0; pass < 8; ++pass) {
        hipLaunchKernelGGL(rdr_hist_kernel, dim3(gx, a.B), dim3(256), 0, s, a, pass);
        hipLaunchKernelGGL(rdr_select_kernel, dim3(a.B), dim3(64), 0, s, a, pass);
    }
    hipLaunchKernelGGL(rdr_tie_kernel, dim3(a.B), dim3(1024), 0, s, a);
    hipLaunchKernelGGL(rdr_final_kernel, dim3(g), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace ada
