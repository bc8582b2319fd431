// decode.hip -- ADA paged decode for gfx950: angle-LUT staging, tier-specialised
// logits from codes, wavefront online softmax, fp16 value accumulation,
// split-K partials over context chunks and the reduction pass.
//
// Method: "SPHERICAL KV" (arXiv 2605.18856), Abstract: logits come straight
// from the radius + angle codes (no dense key is rebuilt) on a paged,
// block-local decode path that streams tier-homogeneous pages.
//
// Work decomposition: one work-group per (context chunk, KV head, sequence).
// The G = Hq/Hkv query heads of a KV head share every code and value read.
// A wavefront takes 64 tokens at a time (4 pages of 16 or 2 pages of 32):
//   logits:  lane = token; the token's 16-byte code units are read with one
//            128-bit load per unit (units are token-minor, so the 64 lanes
//            read contiguous memory); per pair j the lane gathers
//            LUT_g[j][theta_code] from LDS for every head g and accumulates
//            s_code * entry.  T8 uses the factorised form
//            s (cos th, sin th) . (q[2j], q[2j+1]) with a 256-entry cos/sin
//            table in LDS instead of a 64 KB-per-head table.
//   softmax: per head, running max over the wavefront (butterfly), exp2 of
//            the base-2 scaled logits, per-lane running sums.
//   values:  lane = head dimension (lane and lane+64); each 128-bit load
//            brings 8 consecutive tokens of one dimension (value pages are
//            stored in 8-token groups, dimension-major), fp32 accumulation.
// There is no matrix-core work in the logit path: it is a gather-reduce over
// small per-pair tables, not a dense contraction.
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

// LDS writes by one lane become visible to other lanes of the same wave.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T>
__device__ __forceinline__ T ldg(const void *p) {
    return *reinterpret_cast<const T *>(p);
}

// ---- logits per tier (lane = token) --------------------------------------
// Each returns base-2 scaled logits: scale * log2(e) * r * sum_j s_j LUT[j][c].

template <int G, int P>
__device__ __forceinline__ void logits_t4(const uint8_t *blk, int slot, const float *lut4, float mul,
                                          float (&lg)[G]) {
    const float r = h2f(ldg<uint16_t>(blk + 2 * slot));
    const uint8_t *tb = blk + 2 * P + slot * 16;
    const uint8_t *sbp = blk + 2 * P + 32 * P + slot * 16;
    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.f;
    // one 16-byte unit = 32 pairs of 4-bit angle and magnitude codes
#pragma unroll 1
    for (int u = 0; u < 2; ++u) {
        const uint4 t = ldg<uint4>(tb + u * 16 * P);
        const uint4 sv = ldg<uint4>(sbp + u * 16 * P);
        const uint32_t tw[4] = {t.x, t.y, t.z, t.w};
        const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
        const float *lu = lut4 + u * 32 * G * 16;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const uint32_t c = (tw[j >> 3] >> ((j & 7) * 4)) & 15u;
            const float s = (float)((sw[j >> 3] >> ((j & 7) * 4)) & 15u);
            const float *e = lu + j * G * 16 + c;
#pragma unroll
            for (int g = 0; g < G; ++g) acc[g] = fmaf(s, e[g * 16], acc[g]);
        }
    }
    const float m = r * mul * (1.0f / 15.0f);
#pragma unroll
    for (int g = 0; g < G; ++g) lg[g] = acc[g] * m;
}

template <int G, int P>
__device__ __forceinline__ void logits_t2(const uint8_t *blk, int slot, const float *lut2, float mul,
                                          float (&lg)[G]) {
    const float r = h2f(ldg<uint16_t>(blk + 2 * slot));
    const uint8_t *tb = blk + 2 * P;
    const uint8_t *sbp = tb + 16 * P;
    const uint4 t0 = ldg<uint4>(tb + slot * 16);
    const uint4 s0 = ldg<uint4>(sbp + slot * 16);
    const uint2 s1 = ldg<uint2>(sbp + 16 * P + slot * 8);
    // half h covers pairs 32h..32h+31: angle words 2h, 2h+1 (2-bit codes),
    // magnitude words 3h..3h+2 (3-bit codes, 96 bits)
    uint32_t tw[4] = {t0.x, t0.y, t0.z, t0.w};
    uint32_t sw[6] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y};
    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.f;
    const float *lu = lut2;
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const uint32_t c = (tw[j >> 4] >> ((j & 15) * 2)) & 3u;
            const int bit = 3 * j, wd = bit >> 5, sh = bit & 31;
            uint32_t sv;
            if (sh <= 29)
                sv = (sw[wd] >> sh) & 7u;
            else   // the code straddles two words
                sv = ((sw[wd] >> sh) | (sw[wd + 1] << (32 - sh))) & 7u;
            const float s = (float)sv;
            const float *e = lu + j * G * 4 + c;
#pragma unroll
            for (int g = 0; g < G; ++g) acc[g] = fmaf(s, e[g * 4], acc[g]);
        }
        tw[0] = tw[2];
        tw[1] = tw[3];
        sw[0] = sw[3];
        sw[1] = sw[4];
        sw[2] = sw[5];
        lu += 32 * G * 4;
    }
    const float m = r * mul * (1.0f / 7.0f);
#pragma unroll
    for (int g = 0; g < G; ++g) lg[g] = acc[g] * m;
}

template <int G, int P>
__device__ __forceinline__ void logits_t8(const uint8_t *blk, int slot, const float2 *cs8, const float *q8,
                                          float mul, float (&lg)[G]) {
    const float r = h2f(ldg<uint16_t>(blk + 2 * slot));
    const uint8_t *tb = blk + 2 * P + slot * 16;
    const uint8_t *sbp = blk + 2 * P + 64 * P + slot * 16;
    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.f;
    // one 16-byte unit = 16 pairs of 8-bit codes
#pragma unroll 1
    for (int u = 0; u < 4; ++u) {
        const uint4 t = ldg<uint4>(tb + u * 16 * P);
        const uint4 sv = ldg<uint4>(sbp + u * 16 * P);
        const uint32_t tw[4] = {t.x, t.y, t.z, t.w};
        const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
        const float *qu = q8 + u * 16 * G * 2;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t c = (tw[j >> 2] >> ((j & 3) * 8)) & 255u;
            const float s = (float)((sw[j >> 2] >> ((j & 3) * 8)) & 255u);
            const float2 cs = cs8[c];
            const float ux = s * cs.x, uy = s * cs.y;
            const float *qq = qu + j * G * 2;
#pragma unroll
            for (int g = 0; g < G; ++g) acc[g] = fmaf(ux, qq[2 * g], fmaf(uy, qq[2 * g + 1], acc[g]));
        }
    }
    const float m = r * mul * (1.0f / 255.0f);
#pragma unroll
    for (int g = 0; g < G; ++g) lg[g] = acc[g] * m;
}

// ---- split-K pass ----------------------------------------------------------
template <int G, int P, int NW, int WPE>
__global__ __launch_bounds__(NW * 64, WPE) void decode_partials_kernel(DecodeLaunch a) {
    constexpr int TPG = 64 / P;       // pages per 64-token group
    constexpr int KB = P / 8;         // 8-token value blocks per page
    constexpr int NBLK = TPG * KB;    // value blocks per group (8)
    constexpr int RED = NW * G * 130;
    constexpr int LUTF = 64 * G * 16 + 64 * G * 4;
    __shared__ float lut[(LUTF > RED) ? LUTF : RED];   // T4 then T2 tables; reused for the wave merge
    __shared__ float2 cs8[256];
    __shared__ float q8[64 * G * 2];                     // [j][g][x|y]
    __shared__ float pbuf[NW][64 * G];                   // [wave][token][g]
    float *lut4 = lut;
    float *lut2 = lut + 64 * G * 16;

    const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int row = b * a.Hkv + h;
    const int np = a.num_pages[row];
    const int p0 = chunk * a.chunk_pages;
    if (p0 >= np) return;
    const int p1 = min(p0 + a.chunk_pages, np);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    constexpr int NT = NW * 64;

    // -- stage the angle LUTs of the G query heads --------------------------
    const float *qrow = a.q + ((size_t)b * a.Hq + (size_t)h * G) * kD;
    for (int i = tid; i < G * kD; i += NT) {
        const int g = i >> 7, d = i & 127;
        q8[((d >> 1) * G + g) * 2 + (d & 1)] = qrow[i];
    }
    for (int c = tid; c < 256; c += NT) cs8[c] = grid_dir(c);
    __syncthreads();
    for (int i = tid; i < 64 * G * 16; i += NT) {
        const int c = i & 15, jg = i >> 4;
        lut4[i] = lut_entry(q8[jg * 2], q8[jg * 2 + 1], cs8[c * 16]);
    }
    for (int i = tid; i < 64 * G * 4; i += NT) {
        const int c = i & 3, jg = i >> 2;
        lut2[i] = lut_entry(q8[jg * 2], q8[jg * 2 + 1], cs8[c * 64]);
    }
    __syncthreads();

    const float mul = a.scale * kLog2e;
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
        // Opaque to the optimiser: keeps loop-invariant LDS reads (query
        // pairs, tables) inside the loop instead of hoisting them into
        // registers for the whole loop.
        asm volatile("" ::: "memory");
        const int pbase = p0 + grp * TPG;
        const int npg = __builtin_amdgcn_readfirstlane(min(TPG, p1 - pbase));   // pages in this group
        const int nblk = npg * KB;
        const bool pvalid = pg < npg;
        const int page = pvalid ? ptab[pbase + pg] : 0;
        int pk[TPG];
#pragma unroll
        for (int k = 0; k < TPG; ++k) pk[k] = __builtin_amdgcn_readlane(page, k * P);

        // value block `blk` (8 tokens): dimension `lane` and `lane + 64`
        auto vaddr = [&](int blk) -> const uint16_t * {
            return a.value_pool + (size_t)pk[blk / KB] * P * kD + (blk % KB) * 1024 + lane * 8;
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

        uint2 meta = make_uint2(0u, 0u);
        if (pvalid) meta = ldg<uint2>(a.page_meta + page);
        const int tier = meta.x & 0xFF;
        const int count = (meta.x >> 8) & 0xFF;
        const bool valid = pvalid && slot < count;

        float lg[G];
#pragma unroll
        for (int g = 0; g < G; ++g) lg[g] = -INFINITY;
        const uint8_t *blkp = a.arena + (size_t)meta.y * 16;
        if (__any(valid && tier == ADA_TIER_T4)) {
            if (valid && tier == ADA_TIER_T4) logits_t4<G, P>(blkp, slot, lut4, mul, lg);
        }
        if (__any(valid && tier == ADA_TIER_T2)) {
            if (valid && tier == ADA_TIER_T2) logits_t2<G, P>(blkp, slot, lut2, mul, lg);
        }
        if (__any(valid && tier == ADA_TIER_T8)) {
            if (valid && tier == ADA_TIER_T8) logits_t8<G, P>(blkp, slot, cs8, q8, mul, lg);
        }

        // online softmax (base 2)
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

        // value accumulation, two blocks in flight
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

    // -- merge the waves of the work-group, write the chunk's partial --------
#pragma unroll
    for (int g = 0; g < G; ++g) l_run[g] = wave_sum(l_run[g]);
    __syncthreads();
    float *red = lut;   // [w][g][130]: m, l, acc[128]
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

// ---- reduction pass: merge the chunks of every (sequence, query head) -------
__global__ __launch_bounds__(128) void decode_reduce_kernel(DecodeLaunch a) {
    const int bq = blockIdx.x;
    const int b = bq / a.Hq, hq = bq % a.Hq;
    const int G = a.Hq / a.Hkv;
    const int np = a.num_pages[b * a.Hkv + hq / G];
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

// ---- stand-alone LUT builder --------------------------------------------
__global__ __launch_bounds__(256) void build_lut_kernel(const float *q, float *lut) {
    __shared__ float2 cs8[256];
    __shared__ float qs[kD];
    const int rowq = blockIdx.x, tid = threadIdx.x;
    cs8[tid] = grid_dir(tid);
    if (tid < kD) qs[tid] = q[(size_t)rowq * kD + tid];
    __syncthreads();
    float *out = lut + (size_t)rowq * (64 * (256 + 16 + 4));
    for (int i = tid; i < 64 * 256; i += 256) {
        const int j = i >> 8, c = i & 255;
        out[i] = lut_entry(qs[2 * j], qs[2 * j + 1], cs8[c]);
    }
    out += 64 * 256;
    for (int i = tid; i < 64 * 16; i += 256) {
        const int j = i >> 4, c = i & 15;
        out[i] = lut_entry(qs[2 * j], qs[2 * j + 1], cs8[c * 16]);
    }
    out += 64 * 16;
    for (int i = tid; i < 64 * 4; i += 256) {
        const int j = i >> 2, c = i & 3;
        out[i] = lut_entry(qs[2 * j], qs[2 * j + 1], cs8[c * 64]);
    }
}

template <int G, int P>
hipError_t launch_gp(const DecodeLaunch &a, hipStream_t s) {
    constexpr int NW = 4;
    constexpr int WPE = (G >= 8) ? 2 : 4;
    dim3 grid(a.S, a.Hkv, a.B);
    hipLaunchKernelGGL((decode_partials_kernel<G, P, NW, WPE>), grid, dim3(NW * 64), 0, s, a);
    return hipGetLastError();
}

template <int G>
hipError_t launch_g(const DecodeLaunch &a, hipStream_t s) {
    return a.P == 16 ? launch_gp<G, 16>(a, s) : launch_gp<G, 32>(a, s);
}

}  // namespace

hipError_t launch_decode_partials(const DecodeLaunch &a, hipStream_t s) {
    switch (a.Hq / a.Hkv) {
        case 1: return launch_g<1>(a, s);
        case 2: return launch_g<2>(a, s);
        case 4: return launch_g<4>(a, s);
        case 8: return launch_g<8>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_reduce(const DecodeLaunch &a, hipStream_t s) {
    hipLaunchKernelGGL(decode_reduce_kernel, dim3(a.B * a.Hq), dim3(128), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_build_lut(const float *q, int32_t rows, float *lut, hipStream_t s) {
    hipLaunchKernelGGL(build_lut_kernel, dim3(rows), dim3(256), 0, s, q, lut);
    return hipGetLastError();
}

}  // namespace ada
