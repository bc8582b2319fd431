// dense.hip -- dense fp16 paged decode with the same split-K skeleton as the
// ADA decode: a same-box traffic and footprint reference (512 bytes per
// token-head against the ADA tiers' 298-386), not part of the method.
//
// Key pages: fp16 [16 dimension blocks][P tokens][8 dims] (token-minor
// 16-byte units, so lane = token reads are 128-bit and contiguous across the
// wavefront).  Value pages: the ADA value layout (8-token groups,
// dimension-major).  Softmax, value accumulation, split-K partials and the
// reduction pass are those of the ADA decode.
#include "ada_internal.h"

namespace ada {
namespace {

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
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
template <typename T>
__device__ __forceinline__ T ldg(const void *p) {
    return *reinterpret_cast<const T *>(p);
}

template <int G, int P, int NW, int WPE>
__global__ __launch_bounds__(NW * 64, WPE) void dense_partials_kernel(DenseLaunch a) {
    constexpr int TPG = 64 / P, KB = P / 8, NBLK = TPG * KB;
    constexpr int RED = NW * G * 130;
    __shared__ float qd[kD * G];            // [d][g]
    __shared__ float pbuf[NW][64 * G];
    __shared__ float red[RED];

    const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int row = b * a.Hkv + h;
    const int ctx = a.ctx_len[b];
    const int np = (ctx + P - 1) / P;
    const int p0 = chunk * a.chunk_pages;
    if (p0 >= np) return;
    const int p1 = min(p0 + a.chunk_pages, np);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    constexpr int NT = NW * 64;
    const float mul = a.scale * kLog2e;
    const float *qrow = a.q + ((size_t)b * a.Hq + (size_t)h * G) * kD;
    for (int i = tid; i < G * kD; i += NT) qd[(i & 127) * G + (i >> 7)] = qrow[i] * mul;
    __syncthreads();

    float m_run[G], l_run[G], acc0[G], acc1[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m_run[g] = -INFINITY;
        l_run[g] = 0.f;
        acc0[g] = 0.f;
        acc1[g] = 0.f;
    }
    const int n_groups = (p1 - p0 + TPG - 1) / TPG;
    const int pg = lane / P, slot = lane % P;
    const int32_t *ptab = a.page_table + (size_t)row * a.maxp;
    for (int grp = w; grp < n_groups; grp += NW) {
        asm volatile("" ::: "memory");
        const int pbase = p0 + grp * TPG;
        const int npg = __builtin_amdgcn_readfirstlane(min(TPG, p1 - pbase));
        const int nblk = npg * KB;
        const bool pvalid = pg < npg;
        const int pidx = pbase + pg;
        const int page = pvalid ? ptab[pidx] : 0;
        const int count = pvalid ? min(P, ctx - pidx * P) : 0;
        const bool valid = pvalid && slot < count;
        int pk[TPG];
#pragma unroll
        for (int k = 0; k < TPG; ++k) pk[k] = __builtin_amdgcn_readlane(page, k * P);
        auto vaddr = [&](int blk) -> const uint16_t * {
            return a.v_pool + (size_t)pk[blk / KB] * P * kD + (blk % KB) * 1024 + lane * 8;
        };
        uint4 vb0[2], vb1[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            vb0[i] = make_uint4(0u, 0u, 0u, 0u);
            vb1[i] = vb0[i];
            if (i < nblk) {
                vb0[i] = ldg<uint4>(vaddr(i));
                vb1[i] = ldg<uint4>(vaddr(i) + 64 * 8);
            }
        }
        float lg[G];
#pragma unroll
        for (int g = 0; g < G; ++g) lg[g] = 0.f;
        if (valid) {
            const uint16_t *kp = a.k_pool + (size_t)page * P * kD + slot * 8;
#pragma unroll 2
            for (int db = 0; db < 16; ++db) {
                const uint4 kv = ldg<uint4>(kp + db * P * 8);
                const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float kf = h2f((i & 1) ? (kw[i >> 1] >> 16) : (kw[i >> 1] & 0xFFFFu));
                    const float *qq = qd + (db * 8 + i) * G;
#pragma unroll
                    for (int g = 0; g < G; ++g) lg[g] = fmaf(kf, qq[g], lg[g]);
                }
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mx = wave_max(valid ? lg[g] : -INFINITY);
            const float mnew = fmaxf(m_run[g], mx);
            const float alpha = (m_run[g] == -INFINITY) ? 0.f : exp2f(m_run[g] - mnew);
            const float p = valid ? exp2f(lg[g] - mnew) : 0.f;
            l_run[g] = l_run[g] * alpha + p;
            acc0[g] *= alpha;
            acc1[g] *= alpha;
            m_run[g] = mnew;
            pbuf[w][lane * G + g] = p;
        }
        wave_lds_sync();
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk) {
            if (blk >= nblk) break;
            const uint4 x0 = vb0[blk & 1], x1 = vb1[blk & 1];
            if (blk + 2 < nblk) {
                vb0[blk & 1] = ldg<uint4>(vaddr(blk + 2));
                vb1[blk & 1] = ldg<uint4>(vaddr(blk + 2) + 64 * 8);
            }
            const uint32_t a0[4] = {x0.x, x0.y, x0.z, x0.w};
            const uint32_t a1[4] = {x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int tok = blk * 8 + i;
                const float f0 = h2f((i & 1) ? (a0[i >> 1] >> 16) : (a0[i >> 1] & 0xFFFFu));
                const float f1 = h2f((i & 1) ? (a1[i >> 1] >> 16) : (a1[i >> 1] & 0xFFFFu));
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const float p = pbuf[w][tok * G + g];
                    acc0[g] = fmaf(p, f0, acc0[g]);
                    acc1[g] = fmaf(p, f1, acc1[g]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        wave_lds_sync();
    }
#pragma unroll
    for (int g = 0; g < G; ++g) l_run[g] = wave_sum(l_run[g]);
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float *rr = red + (w * G + g) * 130;
        if (lane == 0) {
            rr[0] = m_run[g];
            rr[1] = l_run[g];
        }
        rr[2 + lane] = acc0[g];
        rr[2 + 64 + lane] = acc1[g];
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

__global__ __launch_bounds__(128) void dense_reduce_kernel(DenseLaunch a) {
    const int bq = blockIdx.x;
    const int b = bq / a.Hq;
    const int np = (a.ctx_len[b] + a.P - 1) / a.P;
    const int nc = (np + a.chunk_pages - 1) / a.chunk_pages;
    const int d = threadIdx.x;
    const size_t base = (size_t)bq * a.S;
    float M = -INFINITY;
    for (int c = 0; c < nc; ++c) M = fmaxf(M, a.pm[base + c]);
    if (nc == 0 || M == -INFINITY) {
        a.out[(size_t)bq * kD + d] = 0.f;
        if (a.lse && d == 0) a.lse[bq] = -INFINITY;
        return;
    }
    float L = 0.f, o = 0.f;
    for (int c = 0; c < nc; ++c) {
        const float f = exp2f(a.pm[base + c] - M);
        L = fmaf(a.pl[base + c], f, L);
        o = fmaf(a.pacc[(base + c) * kD + d], f, o);
    }
    a.out[(size_t)bq * kD + d] = o / L;
    if (a.lse && d == 0) a.lse[bq] = (M + log2f(L)) * 0.69314718055994531f;
}

template <int G, int P>
hipError_t launch_gp(const DenseLaunch &a, hipStream_t s) {
    constexpr int NW = 4;
    constexpr int WPE = (G >= 8) ? 2 : 4;
    hipLaunchKernelGGL((dense_partials_kernel<G, P, NW, WPE>), dim3(a.S, a.Hkv, a.B), dim3(NW * 64), 0, s, a);
    return hipGetLastError();
}
template <int G>
hipError_t launch_g(const DenseLaunch &a, hipStream_t s) {
    return a.P == 16 ? launch_gp<G, 16>(a, s) : launch_gp<G, 32>(a, s);
}

// streaming copy, 16 bytes per lane per step
__global__ __launch_bounds__(256) void probe_copy_kernel(const uint4 *src, uint4 *dst, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) dst[i] = src[i];
}

}  // namespace

hipError_t launch_dense_partials(const DenseLaunch &a, hipStream_t s) {
    switch (a.Hq / a.Hkv) {
        case 1: return launch_g<1>(a, s);
        case 2: return launch_g<2>(a, s);
        case 4: return launch_g<4>(a, s);
        case 8: return launch_g<8>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dense_reduce(const DenseLaunch &a, hipStream_t s) {
    hipLaunchKernelGGL(dense_reduce_kernel, dim3(a.B * a.Hq), dim3(128), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_probe_copy(const void *src, void *dst, size_t bytes, hipStream_t s) {
    const int64_t n = (int64_t)(bytes / 16);
    hipLaunchKernelGGL(probe_copy_kernel, dim3(256 * 8), dim3(256), 0, s, (const uint4 *)src, (uint4 *)dst, n);
    return hipGetLastError();
}

}  // namespace ada
