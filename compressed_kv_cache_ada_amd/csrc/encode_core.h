// encode_core.h -- the exact key encoder shared by the page writers
// (encode.hip) and the fused append + decode kernel (decode.hip).
//
// Method: "SPHERICAL KV" (arXiv 2605.18856), Abstract: keys are stored as a
// scalar radius plus compact angle codes.  Code decisions are exact: a code
// is the nearest grid point of the real-valued angle / magnitude, not of a
// rounded estimate.
//
// Encoder (one wavefront per key, lane j = pair j):
//   e_j = x_j^2 + y_j^2 (squares of fp32 values are exact in fp64),
//   R2  = pairwise tree over the wavefront, strides 32,16,...,1,
//   r   = sqrt(R2) (correctly rounded fp64), stored as fp16 (RNE, saturating),
//   magnitude code: exact test 4 L^2 e >= (2m+1)^2 R2 with TwoProduct (fma)
//                   around an fp64 estimate,
//   angle code:     fp64 atan2 estimate accepted outside a 2^-30 band around a
//                   rounding boundary; inside it the side of the boundary
//                   direction beta is decided by the sign of
//                   y cos(beta) - x sin(beta) in double-double arithmetic
//                   (cos/sin of beta from a double-double Taylor series);
//                   2-bit codes use exact comparisons on the diagonals.
// Every rounding below is the one written: each function turns off the
// contraction of multiplies and adds into fused multiply-adds (only the
// explicit ones remain), whatever the including file's settings.
#pragma once

#include "ada_internal.h"

namespace ada {
namespace enc {

// ---------------------------------------------------------------- fp16
__host__ __device__ inline uint16_t f64_to_f16_rne_sat(double x) {
    uint64_t u;
    __builtin_memcpy(&u, &x, 8);
    const uint16_t sign = (uint16_t)((u >> 63) << 15);
    u &= 0x7FFFFFFFFFFFFFFFull;
    if (u == 0) return sign;
    if (u >= 0x7FF0000000000000ull) return (uint16_t)(sign | 0x7BFF);   // inf / nan: saturate
    const int e = (int)(u >> 52) - 1023;                               // x in [2^e, 2^(e+1))
    if (e > 15) return (uint16_t)(sign | 0x7BFF);
    if (e < -25) return sign;                                          // below half the smallest subnormal
    const uint64_t m = (u & ((1ull << 52) - 1)) | (1ull << 52);       // x = m 2^(e-52)
    const int qexp = (e >= -14) ? e - 10 : -24;                        // fp16 spacing 2^qexp
    const int shift = 52 + qexp - e;                                   // 42..53
    uint64_t n = m >> shift;
    const uint64_t rem = m & ((1ull << shift) - 1), half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (n & 1))) ++n;
    if (e >= -14) {
        int ee = e;
        if (n == 2048) { n = 1024; ++ee; }
        if (ee > 15) return (uint16_t)(sign | 0x7BFF);
        return (uint16_t)(sign | ((ee + 15) << 10) | (uint16_t)(n - 1024));
    }
    return (uint16_t)(sign | (uint16_t)n);   // subnormal (n == 1024 is the smallest normal)
}

// ------------------------------------------------------- double-double
struct dd {
    double hi, lo;
};
__device__ inline dd two_sum(double a, double b) {
    #pragma clang fp contract(off)
    const double s = a + b;
    const double bb = s - a;
    return {s, (a - (s - bb)) + (b - bb)};
}
__device__ inline dd quick_two_sum(double a, double b) {
    #pragma clang fp contract(off)
    const double s = a + b;
    return {s, b - (s - a)};
}
__device__ inline dd two_prod(double a, double b) {
    #pragma clang fp contract(off)
    const double p = a * b;
    return {p, __builtin_fma(a, b, -p)};
}
__device__ inline dd dd_add(dd a, dd b) {
    #pragma clang fp contract(off)
    dd s = two_sum(a.hi, b.hi);
    const dd t = two_sum(a.lo, b.lo);
    s.lo += t.hi;
    s = quick_two_sum(s.hi, s.lo);
    s.lo += t.lo;
    return quick_two_sum(s.hi, s.lo);
}
__device__ inline dd dd_mul(dd a, dd b) {
    #pragma clang fp contract(off)
    dd p = two_prod(a.hi, b.hi);
    p.lo += a.hi * b.lo + a.lo * b.hi;
    return quick_two_sum(p.hi, p.lo);
}
__device__ inline dd dd_mul_d(dd a, double b) {
    #pragma clang fp contract(off)
    dd p = two_prod(a.hi, b);
    p.lo += a.lo * b;
    return quick_two_sum(p.hi, p.lo);
}
__device__ inline dd dd_div_d(dd a, double b) {
    #pragma clang fp contract(off)
    const double q1 = a.hi / b;
    const dd p = two_prod(q1, b);
    const double r = ((a.hi - p.hi) - p.lo) + a.lo;
    return quick_two_sum(q1, r / b);
}
__device__ inline dd dd_neg(dd a) { return {-a.hi, -a.lo}; }

// sin and cos of pi * n / N for 0 <= n <= N/4 (angle in [0, pi/4]) by Taylor
// series in double-double; 16 terms leave a truncation error below 2^-110.
__device__ inline void dd_sincos_pi_frac(int n, int N, dd *s_out, dd *c_out) {
    #pragma clang fp contract(off)
    const dd pi = {3.141592653589793116e+00, 1.224646799147353207e-16};
    dd x = dd_mul_d(pi, (double)n);
    x.hi = ldexp(x.hi, -__builtin_ctz((unsigned)N));
    x.lo = ldexp(x.lo, -__builtin_ctz((unsigned)N));
    const dd x2n = dd_neg(dd_mul(x, x));
    dd ts = x, ss = x;
    dd tc = {1.0, 0.0}, sc = {1.0, 0.0};
    for (int k = 1; k <= 16; ++k) {
        ts = dd_div_d(dd_mul(ts, x2n), (double)((2 * k) * (2 * k + 1)));
        ss = dd_add(ss, ts);
        tc = dd_div_d(dd_mul(tc, x2n), (double)((2 * k - 1) * (2 * k)));
        sc = dd_add(sc, tc);
    }
    *s_out = ss;
    *c_out = sc;
}

// direction of the boundary between angle codes m and m+1 (N = 2^tb):
// beta = -pi + (m + 1/2) 2pi / N = pi (2m + 1 - N) / N
__device__ inline void boundary_dir(int m, int N, dd *c, dd *s) {
    #pragma clang fp contract(off)
    int n = 2 * m + 1 - N;
    const double sgn_s = n < 0 ? -1.0 : 1.0;
    int an = n < 0 ? -n : n;          // angle pi*an/N in (0, pi)
    double sgn_c = 1.0;
    if (2 * an > N) {                 // beyond pi/2: reflect to pi - a
        an = N - an;
        sgn_c = -1.0;
    }
    bool swap = false;
    if (4 * an > N) {                 // beyond pi/4: use pi/2 - a
        an = N / 2 - an;
        swap = true;
    }
    dd s0, c0;
    dd_sincos_pi_frac(an, N, &s0, &c0);
    dd cc = swap ? s0 : c0, ss = swap ? c0 : s0;
    cc.hi *= sgn_c; cc.lo *= sgn_c;
    ss.hi *= sgn_s; ss.lo *= sgn_s;
    *c = cc;
    *s = ss;
}

__device__ inline int angle_code(double x, double y, int tb, int *undecidable) {
    #pragma clang fp contract(off)
    const int N = 1 << tb;
    if (x == 0.0 && y == 0.0) return N / 2;
    const double pi = 3.141592653589793116e+00;
    const double t = (atan2(y, x) + pi) / (2.0 * pi) * (double)N;
    const double fl = floor(t);
    if (fabs((t - fl) - 0.5) > 0x1p-30) {
        const int c = (int)floor(t + 0.5);
        return ((c % N) + N) % N;
    }
    const int m = (int)fl;   // boundary between codes m and m+1
    int c;
    if (tb == 2) {
        // boundary directions are the diagonals: decide with exact sums
        double v;
        switch (m & 3) {
            case 0: v = x - y; break;     // beta = -3pi/4
            case 1: v = x + y; break;     // beta = -pi/4
            case 2: v = y - x; break;     // beta =  pi/4
            default: v = -x - y; break;   // beta =  3pi/4
        }
        c = (v >= 0.0) ? m + 1 : m;       // exact tie: half up
    } else {
        dd cb, sb;
        boundary_dir(m, N, &cb, &sb);
        const dd v = dd_add(dd_mul_d(cb, y), dd_neg(dd_mul_d(sb, x)));
        if (fabs(v.hi) <= 0x1p-90 * (fabs(x) + fabs(y))) *undecidable = 1;
        c = (v.hi > 0.0) ? m + 1 : m;
    }
    return ((c % N) + N) % N;
}

// exact: 4 L^2 e >= (2m+1)^2 R2
__device__ inline bool magnitude_reaches(double e, double R2, int L, int m) {
    #pragma clang fp contract(off)
    const double A = 4.0 * (double)L * (double)L;
    const double Bc = (double)(2 * m + 1) * (double)(2 * m + 1);
    const dd p1 = two_prod(A, e), p2 = two_prod(Bc, R2);
    return (p1.hi > p2.hi) || (p1.hi == p2.hi && p1.lo >= p2.lo);
}

__device__ inline int magnitude_code(double e, double R2, int sb) {
    #pragma clang fp contract(off)
    const int L = (1 << sb) - 1;
    if (R2 == 0.0) return 0;
    int c = (int)floor((double)L * sqrt(e / R2) + 0.5);
    c = c < 0 ? 0 : (c > L ? L : c);
    while (c > 0 && !magnitude_reaches(e, R2, L, c - 1)) --c;
    while (c < L && magnitude_reaches(e, R2, L, c)) ++c;
    return c;
}

__device__ inline void set_status(int32_t *status, int code) { atomicCAS(status, 0, code); }

__device__ inline int read_status(const int32_t *status) {
    return __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------- V8 values
// V8 value codec (tiers 3-5): blocks of 32 dimensions share the exponent
// e = floor(log2 max|v|), at least -18; code = round-half-even(v 2^(6-e))
// clamped to [-127, 127]; decoded value code * 2^(e-6), an fp16 number.

// the shared exponent from the largest magnitude's fp16 bits (finite)
__device__ inline int v8_exponent(uint32_t amax_bits) {
    if (amax_bits == 0) return -18;
    const int E = (int)(amax_bits >> 10);
    const int e = E > 0 ? E - 15 : (31 - __builtin_clz(amax_bits)) - 24;   // subnormal: bits * 2^-24
    return e < -18 ? -18 : e;
}

// code of the fp16 value with bits h under exponent e (the scaling is exact)
__device__ inline int v8_code(uint32_t h, int e) {
    const float c = rintf(ldexpf(h2f(h & 0xFFFFu), 6 - e));
    return (int)fminf(fmaxf(c, -127.f), 127.f);
}

// fp16 bits of the decoded value code * 2^(scale_byte - 133) (exact)
__device__ inline uint32_t v8_value_bits(int code, int scale_byte) {
    return __builtin_bit_cast(uint16_t, (_Float16)ldexpf((float)code, scale_byte - 133));
}

// --------------------------------------------------- write one token
// Called by all 64 lanes of one wavefront, lane j holding pair j's angle code
// tc and magnitude code sc and the token's value dims 2j, 2j+1 (fp16 bits):
// packs the two bit strings (LSB first) in the wavefront's LDS scratch and
// writes radius r16, codes and values into slot `slot` of the page whose
// metadata is meta (tier, and the block at meta.y * 16: key part, then value
// part; values as fp16, or V8-encoded for tiers 3-5: the 16 lanes of a row
// hold one 32-dimension block).
__device__ inline void write_token(uint32_t tc, uint32_t sc, uint16_t r16, uint32_t v2, int slot, uint2 meta,
                                   uint8_t *arena, int P, uint32_t (&words)[2][16]) {
    const int lane = threadIdx.x & 63;
    const int tier = meta.x & 0xFF;
    const int tb = tier_tb(tier), sb = tier_sb(tier);
    uint32_t *wt = words[0], *ws = words[1];
    if (lane < 16) {
        wt[lane] = 0u;
        ws[lane] = 0u;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    {
        const int bit = lane * tb;
        atomicOr(&wt[bit >> 5], tc << (bit & 31));
        const int bs = lane * sb, sh = bs & 31;
        atomicOr(&ws[bs >> 5], sc << sh);
        if (sh + sb > 32) atomicOr(&ws[(bs >> 5) + 1], sc >> (32 - sh));
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    uint8_t *blk = arena + (size_t)meta.y * 16;
    const int nwt = 2 * tb, nws = 2 * sb;             // 32-bit words per component
    if (lane < nwt) {
        const int w = lane;
        uint8_t *dst = blk + 2 * P + (w >> 2) * 16 * P + slot * 16 + (w & 3) * 4;
        *reinterpret_cast<uint32_t *>(dst) = wt[w];
    } else if (lane >= 32 && lane < 32 + nws) {
        const int w = lane - 32;
        const int nfull = (8 * sb) / 16;
        uint8_t *sbase = blk + 2 * P + 8 * tb * P;
        uint8_t *dst = (w >> 2) < nfull ? sbase + (w >> 2) * 16 * P + slot * 16 + (w & 3) * 4
                                        : sbase + nfull * 16 * P + slot * 8 + (w - 4 * nfull) * 4;
        *reinterpret_cast<uint32_t *>(dst) = ws[w];
    }
    if (lane == 0) *reinterpret_cast<uint16_t *>(blk + 2 * slot) = r16;
    uint8_t *vpart = blk + key16(tier, P) * 16;
    if (tier_v8(tier)) {
        int m = (int)max(v2 & 0x7FFFu, (v2 >> 16) & 0x7FFFu);
        m = max(m, __shfl_xor(m, 1, 64));
        m = max(m, __shfl_xor(m, 2, 64));
        m = max(m, __shfl_xor(m, 4, 64));
        m = max(m, __shfl_xor(m, 8, 64));
        const int e = v8_exponent((uint32_t)m);
        uint8_t *vb = vpart + (slot >> 4) * kV8Group;
        vb[kV8Codes + (2 * lane) * 16 + (slot & 15)] = (uint8_t)(v8_code(v2, e) + 128);
        vb[kV8Codes + (2 * lane + 1) * 16 + (slot & 15)] = (uint8_t)(v8_code(v2 >> 16, e) + 128);
        if ((lane & 15) == 0) vb[(slot & 15) * 4 + (lane >> 4)] = (uint8_t)(e + 127);
    } else {
        uint16_t *vp = reinterpret_cast<uint16_t *>(vpart) + (slot >> 3) * 1024 + (slot & 7);
        vp[(2 * lane) * 8] = (uint16_t)(v2 & 0xFFFF);
        vp[(2 * lane + 1) * 8] = (uint16_t)(v2 >> 16);
    }
    __builtin_amdgcn_wave_barrier();
}

// ------------------------------------------------ encode + write one key
// Called by all 64 lanes of one wavefront: encodes key[128] (fp32; lane j
// takes pair j, (key[2j], key[2j+1]) or with half_pairs (key[j], key[j+64])) at the
// page's tier and writes its radius, codes and value (fp16 bits) into slot
// `slot` of the page whose metadata is meta (block at meta.y * 16).  words is the
// wavefront's LDS scratch for packing the bit strings.  An undecidable code
// (never expected) sets ADA_EINTERNAL and writes nothing.
__device__ inline void encode_write_one(const float *key, const uint16_t *value, int slot, uint2 meta,
                                        uint8_t *arena, int P, int32_t *status, uint32_t (&words)[2][16],
                                        bool half_pairs) {
    #pragma clang fp contract(off)
    const int lane = threadIdx.x & 63;
    const int tier = meta.x & 0xFF;
    const int tb = tier_tb(tier), sb = tier_sb(tier);
    float2 kk;
    if (half_pairs) kk = make_float2(key[lane], key[lane + 64]);
    else kk = *reinterpret_cast<const float2 *>(key + 2 * lane);
    const double x = kk.x, y = kk.y;
    const double xx = x * x;
    const double yy = y * y;
    const double e = xx + yy;
    double t = e;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
        const double o = __shfl_down(t, s, 64);
        if (lane < s) t = t + o;
    }
    const double R2 = __shfl(t, 0, 64);
    const double r = sqrt(R2);
    int und = 0;
    const uint32_t sc = (uint32_t)magnitude_code(e, R2, sb);
    const uint32_t tc = (uint32_t)angle_code(x, y, tb, &und);
    if (__any(und)) {
        if (lane == 0) set_status(status, ADA_EINTERNAL);
        return;
    }
    const uint32_t v2 = *reinterpret_cast<const uint32_t *>(value + 2 * lane);
    write_token(tc, sc, f64_to_f16_rne_sat(r), v2, slot, meta, arena, P, words);
}

}  // namespace enc
}  // namespace ada

