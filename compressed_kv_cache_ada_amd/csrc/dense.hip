// dense.hip -- dense fp16 paged decode with the same split-K skeleton as the
// ADA decode: a same-box traffic and footprint reference (512 bytes per
// token-head against the ADA tiers' 298-386), not part of the method.
//
// Key pages: fp16 [16 dimension blocks][P tokens][8 dims] (token-minor
// 16-byte units, so lane = token reads are 128-bit and contiguous across the
// wavefront).  Value pages: the ADA value layout (8-token groups,
// dimension-major).  Page staging, softmax, value accumulation on the matrix
// cores, split-K partials and the reduction pass are the ADA decode's
// (decode_core.h); only the logits differ.
#include "decode_core.h"

namespace ada {
namespace {

using core::floatx4_t;
using core::half8_t;
using core::ldg;

// Logits at eight heads on the matrix cores: for each 16-token tile of the group, the
// 16 x 128 fp16 keys times the 128 x 16 queries (columns = heads, G used),
// in four K steps of 32 dimensions.  The queries (times scale * log2 e) go
// in as fp16 hi + lo, so the products carry about 22 bits of the fp32
// query; the keys are fp16 numbers exactly; the sums are fp32.
template <int G, int P, int NW>
struct DensePolicy {
    static constexpr bool kStaged = false;
    static constexpr bool kEarlyStage = false;
    static constexpr bool kValueTiers = false;   // fp16 values only
    struct Smem {
        float qd[kD * G];              // [d][g], pre-multiplied by scale * log2(e)
        // eight heads: MFMA B operands [hi|lo][K step][lane], and each
        // wavefront's logits [head][token]
        half8_t qb[G >= 8 ? 2 : 1][4][G >= 8 ? 64 : 1];
        float lg[NW][G][G >= 8 ? 64 : 1];
    };
    const int32_t *ctx_len;
    const uint16_t *k_pool, *v_pool;
    const float *q;
    int32_t Hq;
    float mul;

    __device__ int num_pages(int, int b) const { return (ctx_len[b] + P - 1) / P; }
    __device__ int num_pages_lane(int, int b, uint32_t z) const { return (ctx_len[b + z] + P - 1) / P; }
    __device__ uint2 meta(int, int idx, int b) const {
        const int count = min(P, ctx_len[b] - idx * P);
        return make_uint2((uint32_t)count << 8, 0u);
    }
    __device__ const uint8_t *value_part(int page, uint2) const {
        return reinterpret_cast<const uint8_t *>(v_pool + (size_t)page * P * kD);
    }
    __device__ void prologue(Smem &s, int b, int h, int tid, int nt) const {
        const float *qrow = q + ((size_t)b * Hq + (size_t)h * G) * kD;
        for (int i = tid; i < G * kD; i += nt) s.qd[(i & 127) * G + (i >> 7)] = qrow[i] * mul;
    }
    // B operand of K step ks for lane l: head l % 16 (zero past G),
    // dimensions 32 ks + 8 (l / 16) .. + 7
    __device__ void build(Smem &s, int tid, int nt) const {
        if constexpr (G < 8) return;
        for (int i = tid; i < 4 * 64; i += nt) {
            const int ks = i >> 6, l = i & 63, n = l & 15, d0 = 32 * ks + 8 * (l >> 4);
            half8_t hi, lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = n < G ? s.qd[(d0 + e) * G + (n < G ? n : 0)] : 0.f;
                const _Float16 vh = (_Float16)v;
                hi[e] = vh;
                lo[e] = (_Float16)(v - (float)vh);
            }
            s.qb[0][ks][l] = hi;
            s.qb[1][ks][l] = lo;
        }
    }
    __device__ bool after_pages(Smem &, const int *, int, int, int, int) const { return false; }
    // the lane's token's key base; the loads are issued inside the logits
    struct Codes {
        const uint16_t *kp;
    };
    __device__ Codes fetch(int page, uint2, int slot, bool) const {
        return Codes{k_pool + (size_t)page * P * kD + slot * 8};
    }
    // called by every lane of the wavefront (lane = token of the group).
    // Eight heads: the matrix cores; fewer: fp32 FMAs per lane, which
    // measure faster there (the 16 MFMA columns are mostly empty)
    __device__ void logits(const Smem &s, const Codes &c, uint2, bool valid, float (&lg)[G]) const {
        if constexpr (G >= 8) logits_mfma(s, c, valid, lg);
        else logits_fma(s, c, valid, lg);
    }
    __device__ void logits_fma(const Smem &s, const Codes &c, bool valid, float (&lg)[G]) const {
        if (!valid) return;
        float acc[G];
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g] = 0.f;
        const uint16_t *kp = c.kp;
#pragma unroll 2
        for (int db = 0; db < 16; ++db) {
            const uint4 kv = ldg<uint4>(kp + db * P * 8);
            const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float kf = h2f((i & 1) ? (kw[i >> 1] >> 16) : (kw[i >> 1] & 0xFFFFu));
                const float *qq = s.qd + (db * 8 + i) * G;
#pragma unroll
                for (int g = 0; g < G; ++g) acc[g] = fmaf(kf, qq[g], acc[g]);
            }
            asm volatile("" ::: "memory");
        }
#pragma unroll
        for (int g = 0; g < G; ++g) lg[g] = acc[g];
    }
    __device__ void logits_mfma(const Smem &s, const Codes &c, bool valid, float (&lg)[G]) const {
        const int lane = threadIdx.x & 63;
        const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        float *buf = const_cast<float *>(&s.lg[w][0][0]);
        const uintptr_t kp = reinterpret_cast<uintptr_t>(c.kp);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            // token 16 mt + l % 16 of the group: its key base, from the lane holding it
            const int src = 16 * mt + (lane & 15);
            const uint32_t lo32 = (uint32_t)__shfl((int)(uint32_t)kp, src, 64);
            const uint32_t hi32 = (uint32_t)__shfl((int)(uint32_t)(kp >> 32), src, 64);
            const uint16_t *tk = reinterpret_cast<const uint16_t *>(((uintptr_t)hi32 << 32) | lo32);
            uint4 a[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) a[ks] = ldg<uint4>(tk + (4 * ks + (lane >> 4)) * P * 8);
            floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const half8_t av = __builtin_bit_cast(half8_t, a[ks]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, s.qb[0][ks][lane], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, s.qb[1][ks][lane], acc, 0, 0, 0);
            }
            // C: row = token 16 mt + 4 (l / 16) + i, column = head l % 16
            if ((lane & 15) < G) {
#pragma unroll
                for (int i = 0; i < 4; ++i) buf[(lane & 15) * 64 + 16 * mt + 4 * (lane >> 4) + i] = acc[i];
            }
        }
        core::wave_lds_sync();
        if (valid) {
#pragma unroll
            for (int g = 0; g < G; ++g) lg[g] = buf[g * 64 + lane];
        }
        core::wave_lds_sync();   // read before the next group's logits overwrite it
    }
};

template <int G, int P, int NW, int WPE>
__global__ __launch_bounds__(NW * 64, WPE) void dense_partials_kernel(DenseLaunch a) {
    using Pol = DensePolicy<G, P, NW>;
    constexpr size_t RED = (size_t)NW * G * 130 * sizeof(float);
    constexpr size_t RAW = sizeof(typename Pol::Smem) > RED ? sizeof(typename Pol::Smem) : RED;
    __shared__ __align__(16) unsigned char raw[RAW];
    __shared__ core::CoreSmem<G, NW> cs;
    Pol pol;
    pol.ctx_len = a.ctx_len;
    pol.k_pool = a.k_pool;
    pol.v_pool = a.v_pool;
    pol.q = a.q;
    pol.Hq = a.Hq;
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
    c.logit_buf = nullptr;
    c.gv = G;
    c.voff = 0;
    core::split_k<G, P, NW, false>(c, pol, *reinterpret_cast<typename Pol::Smem *>(raw), cs,
                            reinterpret_cast<float *>(raw), blockIdx.x, blockIdx.y, blockIdx.z);
}

__global__ __launch_bounds__(core::kReduceThreads) void dense_reduce_kernel(DenseLaunch a) {
    const int bq = blockIdx.x;
    const int b = bq / a.Hq;
    const int np = (a.ctx_len[b] + a.P - 1) / a.P;
    core::reduce_chunks(a.pm, a.pl, a.pacc, a.S, core::chunks_with_data(np, 64 / a.P, a.S), bq, bq, threadIdx.x,
                        a.out, a.lse);
}

template <int G, int P>
hipError_t launch_gp(const DenseLaunch &a, hipStream_t s) {
    constexpr int NW = 4;
    constexpr int WPE = decode_waves_per_simd(G);
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

// streaming read: U loads of 16 bytes in flight per lane, optionally with the
// non-temporal hint; the xor-fold only keeps the loads alive
template <int U, bool NT>
__global__ __launch_bounds__(256) void probe_read_kernel(const uint4 *src, int64_t n, uint32_t *out) {
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + (U - 1) * stride < n; i += U * stride) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) { const uint4 *q = src + i + u * stride; if (NT) { v[u].x = __builtin_nontemporal_load(&q->x); v[u].y = __builtin_nontemporal_load(&q->y); v[u].z = __builtin_nontemporal_load(&q->z); v[u].w = __builtin_nontemporal_load(&q->w); } else { v[u] = *q; } }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n; i += stride) acc ^= src[i].x;
    if (acc == 0x9E3779B9u) out[0] = acc;
}

// each work-group streams its own contiguous region (many distant streams)
__global__ __launch_bounds__(256) void probe_read_blocked_kernel(const uint4 *src, int64_t n, uint32_t *out) {
    const int64_t per = (n + gridDim.x - 1) / gridDim.x;
    const int64_t lo = (int64_t)blockIdx.x * per, hi = min(lo + per, n);
    uint32_t acc = 0;
    for (int64_t i = lo + threadIdx.x; i < hi; i += 256) acc ^= src[i].x ^ src[i].y ^ src[i].z ^ src[i].w;
    if (acc == 0x9E3779B9u) out[0] = acc;
}

// Random 16 KB chunks: each wavefront reads whole 16 KB chunks (sixteen
// 16-byte loads per lane in flight, then their fold), the chunks in a
// scrambled order (chunk c of a power-of-two count n is c * 0x9E3779B1 mod
// n, a bijection): the access pattern of the split-K decode's value reads,
// 64-token groups of about 20 KB spread over the arena.  The dynamic LDS
// only caps residency at three work-groups per compute unit, as the decode.
constexpr int kChunkProbeLds = 48 * 1024;
__global__ __launch_bounds__(256) void probe_read_chunks_kernel(const uint4 *src, int64_t nchunks, uint32_t *out) {
    extern __shared__ uint32_t cap[];
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nw = (int64_t)gridDim.x * 4;
    uint32_t acc = 0;
    for (int64_t c = wave; c < nchunks; c += nw) {
        const int64_t pc = (int64_t)(((uint64_t)c * 0x9E3779B1ull) & (uint64_t)(nchunks - 1));
        const uint4 *base = src + pc * 1024;
        uint4 v[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) v[t] = base[t * 64 + lane];
#pragma unroll
        for (int t = 0; t < 16; ++t) acc ^= v[t].x ^ v[t].y ^ v[t].z ^ v[t].w;
    }
    if (acc == 0x9E3779B9u) {
        cap[0] = acc;
        out[0] = cap[0];
    }
}

}  // namespace

hipError_t launch_probe_read(const void *src, size_t bytes, int variant, uint32_t *out, hipStream_t s) {
    const int64_t n = (int64_t)(bytes / 16);
    const dim3 grid(256 * 8), block(256);
    const uint4 *p = (const uint4 *)src;
    switch (variant) {
        case 0: hipLaunchKernelGGL((probe_read_kernel<1, false>), grid, block, 0, s, p, n, out); break;
        case 1: hipLaunchKernelGGL((probe_read_kernel<4, false>), grid, block, 0, s, p, n, out); break;
        case 2: hipLaunchKernelGGL((probe_read_kernel<4, true>), grid, block, 0, s, p, n, out); break;
        case 3: hipLaunchKernelGGL((probe_read_kernel<8, true>), grid, block, 0, s, p, n, out); break;
        case 5: {
            int64_t nc = 1;   // the largest power of two of 16 KB chunks within `bytes`
            while (nc * 2 * 1024 <= n) nc *= 2;
            if (n < 1024) return hipSuccess;
            hipLaunchKernelGGL(probe_read_chunks_kernel, dim3(768), block, kChunkProbeLds, s, p, nc, out);
            break;
        }
        default: hipLaunchKernelGGL(probe_read_blocked_kernel, grid, block, 0, s, p, n, out); break;
    }
    return hipGetLastError();
}

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
    hipLaunchKernelGGL(dense_reduce_kernel, dim3(a.B * a.Hq), dim3(kD * core::reduce_groups(a.S)), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_probe_copy(const void *src, void *dst, size_t bytes, hipStream_t s) {
    const int64_t n = (int64_t)(bytes / 16);
    hipLaunchKernelGGL(probe_copy_kernel, dim3(256 * 8), dim3(256), 0, s, (const uint4 *)src, (uint4 *)dst, n);
    return hipGetLastError();
}

}  // namespace ada
