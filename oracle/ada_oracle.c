/*
 * ada_oracle.c -- plain CPU oracle for Spherical KV's Angle-Domain Attention
 * (ADA) paged decode and its Rate-Distortion Retention (RDR) packer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant
 * generator with the HIP library; each side implements the same written
 * specification on its own.
 *
 * Source of the method: "SPHERICAL KV: Angle-Domain Attention and
 * Rate-Distortion Retention for Efficient Long-Context Inference"
 * (arXiv 2605.18856), Abstract, as printed on the newx.sg paper page, the
 * Semantic-Scholar-style page and the searcharxiv.org abstract page.  The
 * abstract says keys are stored as a scalar radius plus compact angle codes,
 * that attention logits are computed from the codes without rebuilding dense
 * keys, and that RDR picks keep/drop and a precision tier per token and head
 * under a fixed budget, producing tier-homogeneous pages.  It gives no bit
 * layout, formula or rounding rule; the readings used below (pairing of
 * dimensions, codebooks, rounding, tie rules, page byte layout, the rate and
 * distortion model of the packer) are this library's specification and are
 * listed one by one in the design notes that ship with the repository.
 *
 * Arithmetic: fp64 throughout.  The two integer decisions that depend on real
 * numbers (nearest angle code, nearest magnitude code) are taken *exactly*:
 * the magnitude code by exact products in binary128 (every product fits in
 * 71 bits), the angle code by an fp64 estimate that is accepted only outside
 * a 2^-30 guard band around a rounding boundary and is otherwise recomputed
 * in binary128 (libquadmath), where an exact tie can only arise for 2-bit
 * angle codes on the diagonals |x| = |y| and is resolved by comparing |x| and
 * |y| directly.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared ... -lquadmath -lm -lpthread
 */
#include <math.h>
#include <pthread.h>
#include <quadmath.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Status codes returned by the oracle (same meaning as the library's).      */
enum { ORC_OK = 0, ORC_EINVAL = 1, ORC_ENOSPC = 2, ORC_EUNSUPPORTED = 3,
       ORC_EUNDECIDABLE = 99 };

#define ORC_D 128          /* head dimension                      */
#define ORC_NP 64          /* pairs per key: head dimension / 2   */

/* Fixed tier table (id order).  Keys: T8 = 8-bit angle / 8-bit magnitude,
 * T4 = 4 / 4, T2 = 2-bit angle / 3-bit magnitude.  Values: fp16 for ids 0-2
 * (T8, T4, T2); the block-scaled 8-bit value codec V8 (below) for ids 3-5
 * (T8V8, T4V8, T2V8), whose keys are those of ids 0-2.
 * Rate per token and head: 2 (radius) + 8 (tb + sb) (codes) + 256 (fp16
 * values) or 132 (V8 values).  Distortion: 2^-(tb + sb), plus 2^-14 for V8
 * values (the squared relative step of a 7-bit magnitude); a dropped token
 * has distortion 1 and rate 0. */
#define ORC_NT 6
static const int TIER_TB[ORC_NT] = {8, 4, 2, 8, 4, 2};
static const int TIER_SB[ORC_NT] = {8, 4, 3, 8, 4, 3};
static const int TIER_VB[ORC_NT] = {16, 16, 16, 8, 8, 8};

static int64_t tier_rate(int t) { return 2 + 8 * (TIER_TB[t] + TIER_SB[t]) + (TIER_VB[t] == 16 ? 256 : 132); }
static double tier_dist(int t)
{
    return ldexp(1.0, -(TIER_TB[t] + TIER_SB[t])) + (TIER_VB[t] == 16 ? 0.0 : ldexp(1.0, -14));
}

int orc_tier_theta_bits(int tier) { return (tier >= 0 && tier < ORC_NT) ? TIER_TB[tier] : -1; }
int orc_tier_s_bits(int tier) { return (tier >= 0 && tier < ORC_NT) ? TIER_SB[tier] : -1; }
int orc_tier_value_bits(int tier) { return (tier >= 0 && tier < ORC_NT) ? TIER_VB[tier] : -1; }
int64_t orc_tier_rate(int tier) { return (tier >= 0 && tier < ORC_NT) ? tier_rate(tier) : -1; }

/* ------------------------------------------------------------------------ */
/* fp16 conversion: round to nearest, ties to even, straight from fp64 (no
 * intermediate fp32).  Values that would round to infinity saturate to the
 * largest finite half, 65504.  Only non-negative finite inputs occur for a
 * radius, but the sign is handled for completeness. */
uint16_t orc_f64_to_f16(double x)
{
    uint16_t sign = 0;
    if (signbit(x)) { sign = 0x8000; x = -x; }
    if (x == 0.0) return sign;
    int e;                       /* x = f * 2^e, f in [0.5, 1) */
    frexp(x, &e);
    int E = e - 1;               /* x in [2^E, 2^(E+1)) */
    double quantum;
    if (E < -14) quantum = ldexp(1.0, -24);      /* subnormal spacing */
    else quantum = ldexp(1.0, E - 10);           /* 10 fraction bits */
    double n = x / quantum;                      /* exact: power-of-two scale */
    double r = nearbyint(n);                     /* default mode: ties to even */
    double v = r * quantum;
    if (v > 65504.0) return (uint16_t)(sign | 0x7BFF);   /* saturate */
    if (v < ldexp(1.0, -14)) {                   /* stays subnormal */
        return (uint16_t)(sign | (uint16_t)r);
    }
    /* normal: recompute exponent of the rounded value */
    int e2;
    frexp(v, &e2);
    int E2 = e2 - 1;
    double mant = v / ldexp(1.0, E2 - 10) - 1024.0;   /* 0..1023, exact */
    return (uint16_t)(sign | (uint16_t)((E2 + 15) << 10) | (uint16_t)mant);
}

double orc_f16_to_f64(uint16_t h)
{
    int s = (h >> 15) & 1, ex = (h >> 10) & 31, m = h & 1023;
    double v;
    if (ex == 0) v = ldexp((double)m, -24);
    else if (ex == 31) v = m ? NAN : INFINITY;
    else v = ldexp(1024.0 + m, ex - 25);
    return s ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* Encoder.  Key k (fp32, exact in fp64) -> radius r16 (fp16 bits), 64 angle
 * codes, 64 magnitude codes, for angle bits tb and magnitude bits sb.
 *   pairs:    (x_j, y_j) = (k[2j], k[2j+1]) in the adjacent layout, or
 *             (k[j], k[j+64]) in the half-split layout (the rotate-half
 *             form of rotary position embeddings pairs these components)
 *   energies: e_j = x_j^2 + y_j^2 (each square exact in fp64)
 *   norm^2:   R2 = fixed pairwise tree over e (strides 32,16,...,1)
 *   radius:   r = sqrt(R2) correctly rounded, r16 = fp16(r)
 *   magnitude code: nearest integer to L*sqrt(e_j/R2), ties up, L = 2^sb - 1
 *   angle code:     nearest integer to (atan2(y,x)+pi)/(2pi/2^tb), ties up,
 *                   taken mod 2^tb; the zero pair gets code 2^(tb-1).       */

/* exact test of  4 L^2 e >= (2m+1)^2 R2, i.e. L*sqrt(e/R2) >= m + 1/2 */
static int s_reaches(double e, double R2, int L, int m)
{
    __float128 lhs = (__float128)(4.0 * (double)L * (double)L) * (__float128)e;
    __float128 rhs = (__float128)((double)(2 * m + 1) * (double)(2 * m + 1)) * (__float128)R2;
    return lhs >= rhs;
}

static int magnitude_code(double e, double R2, int sb)
{
    int L = (1 << sb) - 1;
    if (R2 == 0.0) return 0;
    double v = (double)L * sqrt(e / R2);
    int c = (int)floor(v + 0.5);
    if (c < 0) c = 0;
    if (c > L) c = L;
    while (c > 0 && !s_reaches(e, R2, L, c - 1)) c--;
    while (c < L && s_reaches(e, R2, L, c)) c++;
    return c;
}

static int angle_code(double x, double y, int tb, int *undecidable)
{
    int N = 1 << tb;
    if (x == 0.0 && y == 0.0) return N / 2;
    double t = (atan2(y, x) + M_PI) / (2.0 * M_PI) * (double)N;
    double fr = t - floor(t);
    if (fabs(fr - 0.5) > ldexp(1.0, -30)) {
        long c = (long)floor(t + 0.5);
        return (int)(((c % N) + N) % N);
    }
    /* near a rounding boundary: redo in binary128 */
    __float128 tq = (atan2q((__float128)y, (__float128)x) + M_PIq) / (2 * M_PIq) * (__float128)N;
    __float128 m = floorq(tq);
    __float128 dq = tq - (m + 0.5Q);
    long c;
    if (fabsq(dq) > 0x1p-100Q) {
        c = (long)m + (dq > 0 ? 1 : 0);
    } else if (tb == 2 && fabs(x) == fabs(y)) {
        c = (long)m + 1;                 /* exact tie on a diagonal: half up */
    } else {
        *undecidable = 1;
        c = (long)m;
    }
    return (int)(((c % N) + N) % N);
}

/* Components of key (or query) vector forming pair j, for pair layout
 * 0 (adjacent) or 1 (half-split). */
static int pair_x(int layout, int j) { return layout ? j : 2 * j; }
static int pair_y(int layout, int j) { return layout ? j + ORC_NP : 2 * j + 1; }

/* Returns ORC_OK, ORC_EINVAL (non-finite key) or ORC_EUNDECIDABLE. */
int orc_encode_key(const float *k, int tb, int sb, uint16_t *r16,
                   uint16_t *theta, uint16_t *s, double *r_out, int layout)
{
    double x[ORC_NP], y[ORC_NP], e[ORC_NP], t[ORC_NP];
    for (int j = 0; j < ORC_NP; j++) {
        x[j] = (double)k[pair_x(layout, j)];
        y[j] = (double)k[pair_y(layout, j)];
        if (!isfinite(x[j]) || !isfinite(y[j])) return ORC_EINVAL;
        double xx = x[j] * x[j];
        double yy = y[j] * y[j];
        e[j] = xx + yy;
        t[j] = e[j];
    }
    for (int stride = ORC_NP / 2; stride >= 1; stride /= 2)
        for (int j = 0; j < stride; j++) t[j] = t[j] + t[j + stride];
    double R2 = t[0];
    double r = sqrt(R2);
    if (r_out) *r_out = r;
    *r16 = orc_f64_to_f16(r);
    int und = 0;
    for (int j = 0; j < ORC_NP; j++) {
        s[j] = (uint16_t)magnitude_code(e[j], R2, sb);
        theta[j] = (uint16_t)angle_code(x[j], y[j], tb, &und);
    }
    return und ? ORC_EUNDECIDABLE : ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Bit strings: code j of width b occupies bits [j*b, (j+1)*b) of a
 * little-endian bit string; bit i lives in bit (i mod 8) of byte i/8. */
void orc_bits_put(uint8_t *dst, int b, const uint16_t *codes, int n)
{
    memset(dst, 0, (size_t)(n * b + 7) / 8);
    for (int j = 0; j < n; j++)
        for (int q = 0; q < b; q++)
            if ((codes[j] >> q) & 1) {
                int i = j * b + q;
                dst[i / 8] |= (uint8_t)(1u << (i % 8));
            }
}

void orc_bits_get(const uint8_t *src, int b, uint16_t *codes, int n)
{
    for (int j = 0; j < n; j++) {
        int c = 0;
        for (int q = 0; q < b; q++) {
            int i = j * b + q;
            if ((src[i / 8] >> (i % 8)) & 1) c |= 1 << q;
        }
        codes[j] = (uint16_t)c;
    }
}

/* ------------------------------------------------------------------------ */
/* Page layout.
 * Block of a page (tier tau, page size P), 16-byte aligned at
 * arena + 16*code_off16: the key part, then the value part.
 * Key part: [radius: P x u16] [angle component] [magnitude component].
 * A component with Bc = 8*b bytes per token is cut into floor(Bc/16) units of
 * 16 bytes, plus one unit of 8 bytes when Bc mod 16 == 8.  Unit u of all P
 * tokens is stored contiguously (token-minor), units in order.
 * Value part of an fp16 tier (256 bytes per token): u16 element (slot, d) at
 *     (slot/8)*1024 + d*8 + slot%8   (8-token groups, dimension-major).
 * Value part of a V8 tier (132 bytes per token): see v8_scale_off below.
 * Page metadata (8 bytes): tier (u8), count (u8), reserved (u16, zero),
 * code_off16 (u32), little-endian. */

static int comp_bytes(int b) { return 8 * b; }           /* per token */

/* bytes of a page's key part and value part */
static int64_t key_bytes(int tier, int P) { return (int64_t)P * (2 + comp_bytes(TIER_TB[tier]) + comp_bytes(TIER_SB[tier])); }
static int64_t value_bytes(int tier, int P) { return (int64_t)P * (TIER_VB[tier] == 16 ? 256 : 132); }

int64_t orc_block_bytes(int tier, int P) { return key_bytes(tier, P) + value_bytes(tier, P); }

/* byte address (relative to the component start) of byte `byte` of the
 * component bit string of token `slot` */
static int64_t comp_addr(int Bc, int P, int slot, int byte)
{
    int u = byte / 16, within = byte % 16;
    int nfull = Bc / 16;
    if (u < nfull) return (int64_t)u * 16 * P + (int64_t)slot * 16 + within;
    return (int64_t)nfull * 16 * P + (int64_t)slot * 8 + within;   /* 8-byte unit */
}

static void write_token_codes(uint8_t *block, int tier, int P, int slot,
                              uint16_t r16, const uint16_t *th, const uint16_t *sc)
{
    int tb = TIER_TB[tier], sb = TIER_SB[tier];
    int Bt = comp_bytes(tb), Bs = comp_bytes(sb);
    uint8_t bt[64], bs[64];
    orc_bits_put(bt, tb, th, ORC_NP);
    orc_bits_put(bs, sb, sc, ORC_NP);
    block[2 * slot] = (uint8_t)(r16 & 0xFF);
    block[2 * slot + 1] = (uint8_t)(r16 >> 8);
    uint8_t *ct = block + 2 * P;
    uint8_t *cs = ct + (int64_t)P * Bt;
    for (int i = 0; i < Bt; i++) ct[comp_addr(Bt, P, slot, i)] = bt[i];
    for (int i = 0; i < Bs; i++) cs[comp_addr(Bs, P, slot, i)] = bs[i];
}

static void read_token_codes(const uint8_t *block, int tier, int P, int slot,
                             uint16_t *r16, uint16_t *th, uint16_t *sc)
{
    int tb = TIER_TB[tier], sb = TIER_SB[tier];
    int Bt = comp_bytes(tb), Bs = comp_bytes(sb);
    uint8_t bt[64], bs[64];
    const uint8_t *ct = block + 2 * P;
    const uint8_t *cs = ct + (int64_t)P * Bt;
    for (int i = 0; i < Bt; i++) bt[i] = ct[comp_addr(Bt, P, slot, i)];
    for (int i = 0; i < Bs; i++) bs[i] = cs[comp_addr(Bs, P, slot, i)];
    *r16 = (uint16_t)(block[2 * slot] | (block[2 * slot + 1] << 8));
    orc_bits_get(bt, tb, th, ORC_NP);
    orc_bits_get(bs, sb, sc, ORC_NP);
}

/* u16 index of fp16 value (slot, d) inside a value part */
static int64_t value_index(int slot, int d) { return (int64_t)(slot / 8) * 1024 + (int64_t)d * 8 + slot % 8; }

/* ------------------------------------------------------------------------ */
/* V8 value codec (value tiers 3-5).  The abstract speaks of precision tiers
 * per token and head without naming a value format; this one follows the
 * pattern of the OCP Microscaling formats: blocks of 32 consecutive
 * dimensions share a power-of-two scale, elements are 8-bit integers with 6
 * fraction bits.  For block k of a token-head's fp16 values v (exact in
 * fp64):
 *   amax = max |v_d|;  e = floor(log2 amax), raised to at least -18
 *   (e = -18 when amax = 0);
 *   c_d = clamp(round_half_even(v_d * 2^(6 - e)), -127, 127)   (the product
 *   is exact);  stored: the byte e + 127 and the int8 codes.
 *   Decoded value: c_d * 2^(e - 6), exactly an fp16 number (|c| <= 127,
 *   e - 6 >= -24).
 * A non-finite value cannot be encoded (EINVAL). */
int orc_v8_encode(const uint16_t *v, uint8_t *scale_byte, int8_t *codes)
{
    for (int k = 0; k < 4; k++) {
        double amax = 0.0;
        for (int d = 32 * k; d < 32 * k + 32; d++) {
            double x = fabs(orc_f16_to_f64(v[d]));
            if (!isfinite(x)) return ORC_EINVAL;
            if (x > amax) amax = x;
        }
        int e = -18;
        if (amax > 0) {
            int ex;
            frexp(amax, &ex);           /* amax = m 2^ex, m in [0.5, 1) */
            if (ex - 1 > e) e = ex - 1;
        }
        scale_byte[k] = (uint8_t)(e + 127);
        for (int d = 32 * k; d < 32 * k + 32; d++) {
            double c = nearbyint(ldexp(orc_f16_to_f64(v[d]), 6 - e));   /* round half to even */
            if (c > 127) c = 127;
            if (c < -127) c = -127;
            codes[d] = (int8_t)c;
        }
    }
    return ORC_OK;
}

void orc_v8_decode(const uint8_t *scale_byte, const int8_t *codes, double *v)
{
    for (int d = 0; d < ORC_D; d++) v[d] = ldexp((double)codes[d], (int)scale_byte[d / 32] - 127 - 6);
}

/* V8 value part: per 16-token group g, at byte 2112 g, [16 tokens][4
 * dimension blocks] scale bytes (64 bytes: a token's four scales are one
 * 4-byte word), then at 2112 g + 64, [128 dims][16 tokens] code bytes c + 128
 * (offset binary; 2048 bytes).  Empty slots are zero. */
static int64_t v8_scale_off(int slot, int k) { return (int64_t)(slot / 16) * 2112 + (slot % 16) * 4 + k; }
static int64_t v8_code_off(int slot, int d) { return (int64_t)(slot / 16) * 2112 + 64 + (int64_t)d * 16 + slot % 16; }

/* write token `slot`'s values (fp16 bits) into the value part of `block` in
 * the tier's format; returns EINVAL for a V8 tier and a non-finite value */
static int value_write(uint8_t *block, int tier, int P, int slot, const uint16_t *v)
{
    uint8_t *vb = block + key_bytes(tier, P);
    if (TIER_VB[tier] == 16) {
        for (int d = 0; d < ORC_D; d++) {
            int64_t i = 2 * value_index(slot, d);
            vb[i] = (uint8_t)(v[d] & 0xFF);
            vb[i + 1] = (uint8_t)(v[d] >> 8);
        }
        return ORC_OK;
    }
    uint8_t sb[4];
    int8_t c[ORC_D];
    if (orc_v8_encode(v, sb, c) != ORC_OK) return ORC_EINVAL;
    for (int k = 0; k < 4; k++) vb[v8_scale_off(slot, k)] = sb[k];
    for (int d = 0; d < ORC_D; d++) vb[v8_code_off(slot, d)] = (uint8_t)(c[d] + 128);
    return ORC_OK;
}

/* token `slot`'s decoded values from the value part of `block`, exact in fp64 */
static void value_read(const uint8_t *block, int tier, int P, int slot, double *v)
{
    const uint8_t *vb = block + key_bytes(tier, P);
    if (TIER_VB[tier] == 16) {
        for (int d = 0; d < ORC_D; d++) {
            int64_t i = 2 * value_index(slot, d);
            v[d] = orc_f16_to_f64((uint16_t)(vb[i] | (vb[i + 1] << 8)));
        }
        return;
    }
    uint8_t sb[4];
    int8_t c[ORC_D];
    for (int k = 0; k < 4; k++) sb[k] = vb[v8_scale_off(slot, k)];
    for (int d = 0; d < ORC_D; d++) c[d] = (int8_t)((int)vb[v8_code_off(slot, d)] - 128);
    orc_v8_decode(sb, c, v);
}

/* values of a token for an encoder: finite fp16 for V8 tiers */
static int values_ok(int tier, const uint16_t *v)
{
    if (TIER_VB[tier] == 16) return 1;
    for (int d = 0; d < ORC_D; d++)
        if (!isfinite(orc_f16_to_f64(v[d]))) return 0;
    return 1;
}

static void meta_write(uint8_t *meta, int64_t page, int tier, int count, uint32_t off16)
{
    uint8_t *m = meta + 8 * page;
    m[0] = (uint8_t)tier;
    m[1] = (uint8_t)count;
    m[2] = 0; m[3] = 0;
    m[4] = (uint8_t)(off16 & 0xFF);
    m[5] = (uint8_t)((off16 >> 8) & 0xFF);
    m[6] = (uint8_t)((off16 >> 16) & 0xFF);
    m[7] = (uint8_t)((off16 >> 24) & 0xFF);
}

static void meta_read(const uint8_t *meta, int64_t page, int *tier, int *count, uint32_t *off16)
{
    const uint8_t *m = meta + 8 * page;
    *tier = m[0];
    *count = m[1];
    *off16 = (uint32_t)m[4] | ((uint32_t)m[5] << 8) | ((uint32_t)m[6] << 16) | ((uint32_t)m[7] << 24);
}

/* ------------------------------------------------------------------------ */
/* Bulk pack (prefill).  For each sequence b < B, head h, tier id ascending,
 * the kept tokens of that (b,h,tier) in ascending position are cut into pages
 * of P; pages get consecutive ids from alloc[0] and consecutive code blocks
 * from alloc[1] (16-byte units).  The page-table row of (b,h) lists its pages
 * in that order; open_page[(b,h)][tier] is the last page of that tier when it
 * is not full, else -1.  Rows of sequences < B are (re)initialised.
 *
 * tiers: int8 [B][Hkv][ctx_stride], -1 = drop, else tier id.
 * keys:  fp32 [B][Hkv][ctx_stride][128]; values: fp16 bits, same shape.
 * All-or-nothing: on EINVAL / ENOSPC nothing is written.
 * Encoding each kept key is a pure function of that key, so it is done first
 * on `nthreads` threads; the page layout pass that follows is sequential. */
typedef struct {
    const int8_t *tiers;
    const float *keys;
    int64_t n_pos;
    uint16_t *r16;
    uint8_t *th, *sc;       /* [n_pos][64] each, codes <= 8 bits */
    int64_t next;
    int worst;
    int layout;
    pthread_mutex_t mu;
} encode_job_t;

static void *encode_worker(void *arg)
{
    encode_job_t *J = arg;
    const int64_t grain = 1024;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t lo = J->next;
        J->next += grain;
        pthread_mutex_unlock(&J->mu);
        if (lo >= J->n_pos) break;
        int64_t hi = lo + grain < J->n_pos ? lo + grain : J->n_pos;
        int worst = ORC_OK;
        for (int64_t i = lo; i < hi; i++) {
            int tau = J->tiers[i];
            if (tau < 0) continue;
            uint16_t th[ORC_NP], sc[ORC_NP];
            int st = orc_encode_key(J->keys + i * ORC_D, TIER_TB[tau], TIER_SB[tau], &J->r16[i], th, sc, NULL,
                                    J->layout);
            if (st > worst) worst = st;
            for (int j = 0; j < ORC_NP; j++) {
                J->th[i * ORC_NP + j] = (uint8_t)th[j];
                J->sc[i * ORC_NP + j] = (uint8_t)sc[j];
            }
        }
        pthread_mutex_lock(&J->mu);
        if (worst > J->worst) J->worst = worst;
        pthread_mutex_unlock(&J->mu);
    }
    return NULL;
}

/* Layout pass of a pack: for each (b, h), tier ascending, the items of
 * that tier in ascending position are written into consecutive new pages
 * (item idx carries its radius r16[idx], codes th/sc[idx][64] and value row
 * values[idx][128]). */
static void pack_layout(int P, int Hkv, int B, const int32_t *ctx_len, int64_t ctx_stride, const int8_t *tiers,
                        const uint16_t *r16, const uint8_t *th_codes, const uint8_t *sc_codes,
                        const uint16_t *values, int32_t max_pages_per_head, int32_t *page_table,
                        int32_t *num_pages, int32_t *open_page, uint8_t *page_meta, uint8_t *arena,
                        int64_t *alloc)
{
    for (int b = 0; b < B; b++) {
        for (int h = 0; h < Hkv; h++) {
            int64_t row = (int64_t)b * Hkv + h;
            int32_t np_row = 0;
            for (int tau = 0; tau < ORC_NT; tau++) {
                open_page[row * ORC_NT + tau] = -1;
                int64_t page = -1;
                int slot = P;
                uint8_t *block = NULL;
                uint32_t off16 = 0;
                for (int t = 0; t < ctx_len[b]; t++) {
                    int64_t idx = row * ctx_stride + t;
                    if (tiers[idx] != tau) continue;
                    if (slot == P) {          /* start a new page */
                        page = alloc[0]++;
                        off16 = (uint32_t)alloc[1];
                        int64_t bb = orc_block_bytes(tau, P);
                        alloc[1] += bb / 16;
                        block = arena + (int64_t)off16 * 16;
                        memset(block, 0, (size_t)bb);
                        page_table[row * max_pages_per_head + np_row] = (int32_t)page;
                        np_row++;
                        slot = 0;
                    }
                    uint16_t th[ORC_NP], sc[ORC_NP];
                    for (int j = 0; j < ORC_NP; j++) {
                        th[j] = th_codes[idx * ORC_NP + j];
                        sc[j] = sc_codes[idx * ORC_NP + j];
                    }
                    write_token_codes(block, tau, P, slot, r16[idx], th, sc);
                    value_write(block, tau, P, slot, values + idx * ORC_D);   /* checked before */
                    slot++;
                    meta_write(page_meta, page, tau, slot, off16);
                }
                if (page >= 0 && slot < P) open_page[row * ORC_NT + tau] = (int32_t)page;
            }
            num_pages[row] = np_row;
        }
    }
}

int orc_pack(int P, int Hkv, int B, const int32_t *ctx_len, int64_t ctx_stride,
             const int8_t *tiers, const float *keys, const uint16_t *values,
             int32_t max_pages_per_head, int64_t page_capacity, int64_t arena_capacity16,
             int32_t *page_table, int32_t *num_pages, int32_t *open_page,
             uint8_t *page_meta, uint8_t *arena, int64_t *alloc,
             int nthreads, int layout)
{
    if (P != 16 && P != 32) return ORC_EINVAL;
    /* validation pass */
    int64_t need_pages = 0, need16 = 0;
    for (int b = 0; b < B; b++) {
        if (ctx_len[b] < 0 || ctx_len[b] > ctx_stride) return ORC_EINVAL;
        for (int h = 0; h < Hkv; h++) {
            int64_t row_pages = 0;
            int64_t n_tier[ORC_NT] = {0};
            for (int t = 0; t < ctx_len[b]; t++) {
                int64_t idx = ((int64_t)b * Hkv + h) * ctx_stride + t;
                int tv = tiers[idx];
                if (tv < -1 || tv >= ORC_NT) return ORC_EINVAL;
                if (tv < 0) continue;
                const float *k = keys + idx * ORC_D;
                for (int d = 0; d < ORC_D; d++)
                    if (!isfinite(k[d])) return ORC_EINVAL;
                if (!values_ok(tv, values + idx * ORC_D)) return ORC_EINVAL;
                n_tier[tv]++;
            }
            for (int tau = 0; tau < ORC_NT; tau++) {
                int64_t pages = (n_tier[tau] + P - 1) / P;
                row_pages += pages;
                need_pages += pages;
                need16 += pages * (orc_block_bytes(tau, P) / 16);
            }
            if (row_pages > max_pages_per_head) return ORC_ENOSPC;
        }
    }
    if (alloc[0] + need_pages > page_capacity) return ORC_ENOSPC;
    if (alloc[1] + need16 > arena_capacity16) return ORC_ENOSPC;

    /* encode every kept key (positions beyond ctx_len are treated as dropped) */
    int64_t n_pos = (int64_t)B * Hkv * ctx_stride;
    int8_t *tiers_used = malloc((size_t)(n_pos > 0 ? n_pos : 1));
    for (int b = 0; b < B; b++)
        for (int h = 0; h < Hkv; h++)
            for (int64_t t = 0; t < ctx_stride; t++) {
                int64_t idx = ((int64_t)b * Hkv + h) * ctx_stride + t;
                tiers_used[idx] = t < ctx_len[b] ? tiers[idx] : -1;
            }
    encode_job_t E;
    E.tiers = tiers_used; E.keys = keys; E.n_pos = n_pos;
    E.r16 = malloc(sizeof(uint16_t) * (n_pos > 0 ? n_pos : 1));
    E.th = malloc((size_t)(n_pos > 0 ? n_pos : 1) * ORC_NP);
    E.sc = malloc((size_t)(n_pos > 0 ? n_pos : 1) * ORC_NP);
    E.next = 0; E.worst = ORC_OK; E.layout = layout;
    pthread_mutex_init(&E.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    pthread_t *thr = malloc(sizeof(pthread_t) * nthreads);
    for (int i = 0; i < nthreads; i++) pthread_create(&thr[i], NULL, encode_worker, &E);
    for (int i = 0; i < nthreads; i++) pthread_join(thr[i], NULL);
    free(thr);
    pthread_mutex_destroy(&E.mu);
    int status = E.worst;
    if (status == ORC_OK)
        pack_layout(P, Hkv, B, ctx_len, ctx_stride, tiers, E.r16, E.th, E.sc, values, max_pages_per_head,
                    page_table, num_pages, open_page, page_meta, arena, alloc);
    free(tiers_used); free(E.r16); free(E.th); free(E.sc);
    return status;
}

/* ------------------------------------------------------------------------ */
/* Append, with sequential semantics in request order: a request for
 * (seq, head, tier) fills the open page of that (seq, head, tier) at slot
 * `count`; when there is none it takes page alloc[0] and the next code block,
 * appends that page to the (seq, head) row and leaves it open unless it is
 * full.  If any request would exceed the page capacity, the arena capacity or
 * the row length, the call returns ENOSPC and writes nothing; a request with
 * an out-of-range seq/head/tier or a non-finite key gives EINVAL and nothing
 * is written. */
int orc_append(int P, int Hkv, int32_t num_seqs, int32_t max_pages_per_head,
               int64_t page_capacity, int64_t arena_capacity16, int n,
               const int32_t *seq, const int32_t *head, const uint8_t *tier,
               const float *keys, const uint16_t *values,
               int32_t *page_table, int32_t *num_pages, int32_t *open_page,
               uint8_t *page_meta, uint8_t *arena, int64_t *alloc, int layout)
{
    if (P != 16 && P != 32) return ORC_EINVAL;
    for (int i = 0; i < n; i++) {
        if (seq[i] < 0 || seq[i] >= num_seqs || head[i] < 0 || head[i] >= Hkv || tier[i] >= ORC_NT)
            return ORC_EINVAL;
        for (int d = 0; d < ORC_D; d++)
            if (!isfinite(keys[(int64_t)i * ORC_D + d])) return ORC_EINVAL;
        if (!values_ok(tier[i], values + (int64_t)i * ORC_D)) return ORC_EINVAL;
    }
    /* dry run on copies of the small state */
    int64_t rows = (int64_t)num_seqs * Hkv;
    int32_t *np_copy = malloc(sizeof(int32_t) * rows);
    int32_t *open_copy = malloc(sizeof(int32_t) * rows * ORC_NT);
    int32_t *cnt_open = malloc(sizeof(int32_t) * rows * ORC_NT);
    memcpy(np_copy, num_pages, sizeof(int32_t) * rows);
    memcpy(open_copy, open_page, sizeof(int32_t) * rows * ORC_NT);
    for (int64_t i = 0; i < rows * ORC_NT; i++) {
        cnt_open[i] = 0;
        if (open_copy[i] >= 0) {
            int tr, c; uint32_t o;
            meta_read(page_meta, open_copy[i], &tr, &c, &o);
            cnt_open[i] = c;
        }
    }
    int64_t a0 = alloc[0], a1 = alloc[1];
    int status = ORC_OK;
    for (int i = 0; i < n && status == ORC_OK; i++) {
        int64_t row = (int64_t)seq[i] * Hkv + head[i];
        int64_t key = row * ORC_NT + tier[i];
        if (open_copy[key] < 0) {
            if (a0 + 1 > page_capacity) status = ORC_ENOSPC;
            else if (a1 + orc_block_bytes(tier[i], P) / 16 > arena_capacity16) status = ORC_ENOSPC;
            else if (np_copy[row] + 1 > max_pages_per_head) status = ORC_ENOSPC;
            if (status) break;
            open_copy[key] = (int32_t)a0;
            a0++;
            a1 += orc_block_bytes(tier[i], P) / 16;
            np_copy[row]++;
            cnt_open[key] = 0;
        }
        cnt_open[key]++;
        if (cnt_open[key] == P) open_copy[key] = -1;
    }
    free(np_copy); free(open_copy); free(cnt_open);
    if (status) return status;

    /* apply */
    for (int i = 0; i < n; i++) {
        int64_t row = (int64_t)seq[i] * Hkv + head[i];
        int tau = tier[i];
        int32_t *op = &open_page[row * ORC_NT + tau];
        int64_t page;
        int cnt;
        uint32_t off16;
        if (*op < 0) {
            page = alloc[0]++;
            off16 = (uint32_t)alloc[1];
            int64_t bb = orc_block_bytes(tau, P);
            alloc[1] += bb / 16;
            memset(arena + (int64_t)off16 * 16, 0, (size_t)bb);
            page_table[row * max_pages_per_head + num_pages[row]] = (int32_t)page;
            num_pages[row]++;
            cnt = 0;
            *op = (int32_t)page;
        } else {
            int tr;
            page = *op;
            meta_read(page_meta, page, &tr, &cnt, &off16);
        }
        uint16_t r16, th[ORC_NP], sc[ORC_NP];
        if (orc_encode_key(keys + (int64_t)i * ORC_D, TIER_TB[tau], TIER_SB[tau], &r16, th, sc, NULL, layout) !=
            ORC_OK)
            return ORC_EUNDECIDABLE;
        write_token_codes(arena + (int64_t)off16 * 16, tau, P, cnt, r16, th, sc);
        value_write(arena + (int64_t)off16 * 16, tau, P, cnt, values + (int64_t)i * ORC_D);   /* checked above */
        cnt++;
        meta_write(page_meta, page, tau, cnt, off16);
        if (cnt == P) *op = -1;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* RDR keep/drop and tier assignment under a byte budget.
 * Items are (head, position) pairs of one sequence; all heads of a sequence
 * share its budget.  Rate of tier tau: 2 + 8*(tb+sb) + 256 bytes (radius,
 * codes, fp16 value row); distortion 2^-(tb+sb); a dropped item has rate 0,
 * distortion 1.  Enabled tiers sorted by rate give upgrade steps
 * drop -> first -> second ...; step k costs dR_k bytes and saves dD_k, with
 * c_k = dD_k / dR_k, which must decrease strictly (else EUNSUPPORTED).
 * Priority of step k of an item with utility w: p = w * c_k (fp64).
 * Total order: p descending, then position descending, then head ascending,
 * then k ascending.  Steps are taken in that order while the running byte
 * total stays within the budget; the walk stops at the first step that does
 * not fit.  An item's tier is its highest step taken (none: dropped = -1). */
typedef struct { double p; int32_t t; int32_t h; int32_t k; } orc_step_t;

static int step_cmp(const void *a, const void *b)
{
    const orc_step_t *x = a, *y = b;
    if (x->p != y->p) return x->p > y->p ? -1 : 1;
    if (x->t != y->t) return x->t > y->t ? -1 : 1;
    if (x->h != y->h) return x->h < y->h ? -1 : 1;
    if (x->k != y->k) return x->k < y->k ? -1 : 1;
    return 0;
}

int orc_rdr_steps(uint32_t tier_mask, int *n_steps, int *step_tier, int64_t *dR, double *c)
{
    int ids[ORC_NT], n = 0;
    if (tier_mask >> ORC_NT) return ORC_EINVAL;
    for (int tau = 0; tau < ORC_NT; tau++)
        if (tier_mask & (1u << tau)) ids[n++] = tau;
    if (n == 0) return ORC_EINVAL;
    /* sort enabled tiers by rate ascending */
    for (int i = 0; i < n; i++)
        for (int j = i + 1; j < n; j++) {
            if (tier_rate(ids[j]) < tier_rate(ids[i])) { int tmp = ids[i]; ids[i] = ids[j]; ids[j] = tmp; }
        }
    int64_t prevR = 0;
    double prevD = 1.0;
    for (int i = 0; i < n; i++) {
        int tau = ids[i];
        int64_t R = tier_rate(tau);
        double D = tier_dist(tau);
        if (R <= prevR || D >= prevD) return ORC_EUNSUPPORTED;
        dR[i] = R - prevR;
        c[i] = (prevD - D) / (double)dR[i];
        if (i > 0 && !(c[i] < c[i - 1])) return ORC_EUNSUPPORTED;
        step_tier[i] = tau;
        prevR = R;
        prevD = D;
    }
    *n_steps = n;
    return ORC_OK;
}

/* cap_level (optional, int8 [B][Hkv][ctx_stride]): an item may take only its
 * first cap_level steps (0 = it must be dropped); NULL = no cap. */
int orc_rdr_assign(int Hkv, int B, const int32_t *ctx_len, int64_t ctx_stride,
                   const float *utility, const int64_t *budget, uint32_t tier_mask,
                   const int8_t *cap_level, int8_t *tier_out)
{
    int n_steps, step_tier[ORC_NT];
    int64_t dR[ORC_NT];
    double c[ORC_NT];
    int st = orc_rdr_steps(tier_mask, &n_steps, step_tier, dR, c);
    if (st) return st;
    for (int b = 0; b < B; b++) {
        if (ctx_len[b] < 0 || ctx_len[b] > ctx_stride || budget[b] < 0) return ORC_EINVAL;
        for (int h = 0; h < Hkv; h++)
            for (int t = 0; t < ctx_len[b]; t++) {
                float w = utility[((int64_t)b * Hkv + h) * ctx_stride + t];
                if (!isfinite(w) || w < 0) return ORC_EINVAL;
            }
    }
    for (int b = 0; b < B; b++) {
        int64_t ctx = ctx_len[b];
        int64_t ns = (int64_t)Hkv * ctx * n_steps;
        orc_step_t *steps = malloc(sizeof(orc_step_t) * (ns > 0 ? ns : 1));
        int64_t q = 0;
        for (int h = 0; h < Hkv; h++)
            for (int64_t t = 0; t < ctx; t++) {
                int64_t idx = ((int64_t)b * Hkv + h) * ctx_stride + t;
                double w = (double)utility[idx];
                int nk = cap_level && cap_level[idx] < n_steps ? cap_level[idx] : n_steps;
                for (int k = 0; k < nk; k++) {
                    steps[q].p = w * c[k];
                    steps[q].t = (int32_t)t;
                    steps[q].h = h;
                    steps[q].k = k;
                    q++;
                }
            }
        ns = q;
        qsort(steps, (size_t)ns, sizeof(orc_step_t), step_cmp);
        for (int h = 0; h < Hkv; h++)
            for (int64_t t = 0; t < ctx_stride; t++)
                tier_out[((int64_t)b * Hkv + h) * ctx_stride + t] = -1;
        int8_t *level = calloc((size_t)(Hkv * ctx > 0 ? Hkv * ctx : 1), 1);
        int64_t cum = 0;
        for (int64_t i = 0; i < ns; i++) {
            if (cum + dR[steps[i].k] > budget[b]) break;
            cum += dR[steps[i].k];
            level[(int64_t)steps[i].h * ctx + steps[i].t] = (int8_t)(steps[i].k + 1);
        }
        for (int h = 0; h < Hkv; h++)
            for (int64_t t = 0; t < ctx; t++) {
                int lv = level[(int64_t)h * ctx + t];
                tier_out[((int64_t)b * Hkv + h) * ctx_stride + t] = lv ? (int8_t)step_tier[lv - 1] : -1;
            }
        free(level);
        free(steps);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Transcoding a token's key codes to a tier of no more bits (tb and sb both
 * not larger), in code space:
 *   angle:     the grids are nested (grid point c of tb bits is grid point
 *              c * 2^(tb_old - tb) of tb_old bits), so the new code is the
 *              nearest new grid point, c_old / 2^d rounded half up, mod 2^tb
 *              (d = tb_old - tb): the tie rule of the encoder;
 *   magnitude: the nearest of the new levels c / L to c_old / L_old, i.e.
 *              round(c_old * L / L_old); for these tiers no exact tie exists;
 *   radius unchanged.
 * This is re-encoding the dequantised key, decided exactly.  Values are
 * re-encoded from their decoded fp16 numbers in the new tier's format (an
 * fp16 -> V8 move quantises them; V8 -> V8 reproduces the codes). */
void orc_transcode(int tier_old, int tier_new, const uint16_t *th_old, const uint16_t *s_old,
                   uint16_t *th_new, uint16_t *s_new)
{
    int d = TIER_TB[tier_old] - TIER_TB[tier_new];
    int N = 1 << TIER_TB[tier_new];
    int64_t L_old = (1 << TIER_SB[tier_old]) - 1, L = (1 << TIER_SB[tier_new]) - 1;
    for (int j = 0; j < ORC_NP; j++) {
        int c = d > 0 ? (th_old[j] + (1 << (d - 1))) >> d : th_old[j];
        th_new[j] = (uint16_t)(c % N);
        /* floor((2 c L + L_old) / (2 L_old)) = round half up of c L / L_old */
        s_new[j] = (uint16_t)((2 * (int64_t)s_old[j] * L + L_old) / (2 * L_old));
    }
}

/* Re-pack (RDR over the cache's own tokens, downgrade only).  The items of
 * sequence b are the kept tokens of its rows in the source cache: item
 * (h, t) is slot t % P of page-list entry t / P of row (b, h), so t orders
 * the row's tokens as its pages list them (t plays the part of the position
 * in the RDR order).  Each item's utility is util[page * P + slot]; it may
 * take only the steps up to its current tier (the codes hold no more), so
 * RDR assigns drop or a tier no larger than the current one under the
 * budget.  The kept items are transcoded (orc_transcode) and packed into the
 * destination cache exactly as orc_pack lays out a tier map over positions
 * 0 .. max_pages_per_head(src) * P - 1.
 * tier_v (optional, int8 [B][Hkv][max_pages_src * P]) receives the tier map.
 * Status: RDR's (EINVAL for a bad utility or budget), then ENOSPC if the
 * destination is too small (nothing written to it). */
int orc_repack(int P, int Hkv, int B, int32_t src_maxp, const int32_t *src_page_table,
               const int32_t *src_num_pages, const uint8_t *src_page_meta, const uint8_t *src_arena,
               const float *util, const int64_t *budget, uint32_t tier_mask,
               int32_t dst_maxp, int64_t dst_page_capacity, int64_t dst_arena_capacity16,
               int32_t *page_table, int32_t *num_pages, int32_t *open_page, uint8_t *page_meta,
               uint8_t *arena, int64_t *alloc, int8_t *tier_v_out)
{
    if (P != 16 && P != 32) return ORC_EINVAL;
    if (tier_mask == 0) tier_mask = 7;
    int n_steps, step_tier[ORC_NT];
    int64_t dR[ORC_NT];
    double c[ORC_NT];
    int st = orc_rdr_steps(tier_mask, &n_steps, step_tier, dR, c);
    if (st) return st;
    /* the codes hold nothing finer than they are: each step of the chain must
     * keep or refine angle, magnitude and value precision, so that the
     * tiers a token may move to form a prefix of the chain */
    for (int k = 1; k < n_steps; k++) {
        int a = step_tier[k - 1], b2 = step_tier[k];
        if (TIER_TB[a] > TIER_TB[b2] || TIER_SB[a] > TIER_SB[b2] || TIER_VB[a] > TIER_VB[b2])
            return ORC_EUNSUPPORTED;
    }
    int64_t S = (int64_t)src_maxp * P;
    int64_t n = (int64_t)B * Hkv * S;
    float *uv = calloc((size_t)(n > 0 ? n : 1), sizeof(float));
    int8_t *cap = calloc((size_t)(n > 0 ? n : 1), 1);
    int8_t *cur = malloc((size_t)(n > 0 ? n : 1));
    int8_t *tier_v = malloc((size_t)(n > 0 ? n : 1));
    int32_t *ctx = malloc(sizeof(int32_t) * (B > 0 ? B : 1));
    memset(cur, -1, (size_t)(n > 0 ? n : 1));
    for (int b = 0; b < B; b++) {
        ctx[b] = (int32_t)S;
        for (int h = 0; h < Hkv; h++) {
            int64_t row = (int64_t)b * Hkv + h;
            for (int i = 0; i < src_num_pages[row]; i++) {
                int64_t page = src_page_table[row * src_maxp + i];
                int tier, count; uint32_t off16;
                meta_read(src_page_meta, page, &tier, &count, &off16);
                int lv = 0;   /* the chain's tiers holding no more than the current one */
                while (lv < n_steps && TIER_TB[step_tier[lv]] <= TIER_TB[tier] &&
                       TIER_SB[step_tier[lv]] <= TIER_SB[tier] && TIER_VB[step_tier[lv]] <= TIER_VB[tier])
                    lv++;
                for (int slot = 0; slot < count; slot++) {
                    int64_t idx = row * S + (int64_t)i * P + slot;
                    uv[idx] = util[page * P + slot];
                    cap[idx] = (int8_t)lv;
                    cur[idx] = (int8_t)tier;
                }
            }
        }
    }
    st = orc_rdr_assign(Hkv, B, ctx, S, uv, budget, tier_mask, cap, tier_v);
    if (st == ORC_OK) {
        /* destination capacity (all-or-nothing) */
        int64_t need_pages = 0, need16 = 0;
        for (int64_t row = 0; row < (int64_t)B * Hkv && st == ORC_OK; row++) {
            int64_t cnt[ORC_NT] = {0}, rp = 0;
            for (int64_t t = 0; t < S; t++)
                if (tier_v[row * S + t] >= 0) cnt[tier_v[row * S + t]]++;
            for (int tau = 0; tau < ORC_NT; tau++) {
                int64_t pg = (cnt[tau] + P - 1) / P;
                rp += pg;
                need_pages += pg;
                need16 += pg * (orc_block_bytes(tau, P) / 16);
            }
            if (rp > dst_maxp) st = ORC_ENOSPC;
        }
        if (alloc[0] + need_pages > dst_page_capacity || alloc[1] + need16 > dst_arena_capacity16) st = ORC_ENOSPC;
    }
    if (st == ORC_OK) {
        uint16_t *r16 = calloc((size_t)(n > 0 ? n : 1), sizeof(uint16_t));
        uint8_t *th = calloc((size_t)(n > 0 ? n : 1) * ORC_NP, 1);
        uint8_t *sc = calloc((size_t)(n > 0 ? n : 1) * ORC_NP, 1);
        uint16_t *vals = calloc((size_t)(n > 0 ? n : 1) * ORC_D, sizeof(uint16_t));
        for (int64_t row = 0; row < (int64_t)B * Hkv; row++)
            for (int64_t t = 0; t < S; t++) {
                int64_t idx = row * S + t;
                if (tier_v[idx] < 0) continue;
                int64_t page = src_page_table[row * src_maxp + t / P];
                int slot = (int)(t % P), tier, count; uint32_t off16;
                meta_read(src_page_meta, page, &tier, &count, &off16);
                uint16_t th_o[ORC_NP], s_o[ORC_NP], th_n[ORC_NP], s_n[ORC_NP];
                read_token_codes(src_arena + (int64_t)off16 * 16, tier, P, slot, &r16[idx], th_o, s_o);
                orc_transcode(tier, tier_v[idx], th_o, s_o, th_n, s_n);
                for (int j = 0; j < ORC_NP; j++) {
                    th[idx * ORC_NP + j] = (uint8_t)th_n[j];
                    sc[idx * ORC_NP + j] = (uint8_t)s_n[j];
                }
                double v[ORC_D];   /* decoded values are fp16 numbers exactly */
                value_read(src_arena + (int64_t)off16 * 16, tier, P, slot, v);
                for (int dd = 0; dd < ORC_D; dd++) vals[idx * ORC_D + dd] = orc_f64_to_f16(v[dd]);
            }
        pack_layout(P, Hkv, B, ctx, S, tier_v, r16, th, sc, vals, dst_maxp, page_table, num_pages, open_page,
                    page_meta, arena, alloc);
        free(r16); free(th); free(sc); free(vals);
    }
    if (tier_v_out) memcpy(tier_v_out, tier_v, (size_t)n);
    free(uv); free(cap); free(cur); free(tier_v); free(ctx);
    return st;
}

/* ------------------------------------------------------------------------ */
/* Angle lookup table of one query head for angle bits tb:
 *   LUT[j][c] = qx_j cos(th_c) + qy_j sin(th_c),  th_c = -pi + c*2pi/2^tb,
 * with (qx_j, qy_j) the query's pair j in the same layout as the keys
 * (no softmax scale folded in). */
void orc_lut(const float *q, int tb, double *lut, int layout)
{
    int N = 1 << tb;
    for (int j = 0; j < ORC_NP; j++)
        for (int c = 0; c < N; c++) {
            double th = -M_PI + (double)c * (2.0 * M_PI / (double)N);
            lut[j * N + c] = (double)q[pair_x(layout, j)] * cos(th) + (double)q[pair_y(layout, j)] * sin(th);
        }
}

/* ------------------------------------------------------------------------ */
/* ADA paged decode, one query row (b, hq), KV head h = hq / G.
 *   logit_t = scale * r_t * sum_j (s_code/L) * LUT[j][theta_code]   (j order)
 *   over the kept tokens of (b,h) as they appear in the page-table row:
 *   m = max logit, w_t = exp(logit_t - m) / sum exp(logit - m),
 *   out = sum_t w_t v_t, lse = m + log(sum exp(logit - m)).
 *   No kept token: out = 0, lse = -inf. */
typedef struct {
    int P, Hq, Hkv, B;
    int32_t max_pages_per_head;
    const int32_t *page_table, *num_pages;
    const uint8_t *page_meta, *arena;
    const float *q;
    double scale;
    double *out, *lse;
    int64_t next_row, n_rows;
    int layout;
    pthread_mutex_t mu;
} decode_job_t;

static void decode_row(decode_job_t *J, int64_t row_q, double *lut8, double *lut4, double *lut2,
                       double *logit, int64_t cap)
{
    int b = (int)(row_q / J->Hq), hq = (int)(row_q % J->Hq);
    int G = J->Hq / J->Hkv;
    int h = hq / G;
    const float *q = J->q + row_q * ORC_D;
    orc_lut(q, 8, lut8, J->layout);
    orc_lut(q, 4, lut4, J->layout);
    orc_lut(q, 2, lut2, J->layout);
    int64_t row = (int64_t)b * J->Hkv + h;
    int np = J->num_pages[row];
    int64_t n = 0;
    double m = -INFINITY;
    /* pass 1: logits */
    for (int i = 0; i < np; i++) {
        int64_t page = J->page_table[row * J->max_pages_per_head + i];
        int tier, count; uint32_t off16;
        meta_read(J->page_meta, page, &tier, &count, &off16);
        const uint8_t *block = J->arena + (int64_t)off16 * 16;
        int tb = TIER_TB[tier], sb = TIER_SB[tier];
        int N = 1 << tb;
        double L = (double)((1 << sb) - 1);
        const double *lut = tb == 8 ? lut8 : (tb == 4 ? lut4 : lut2);
        for (int slot = 0; slot < count; slot++) {
            uint16_t r16, th[ORC_NP], sc[ORC_NP];
            read_token_codes(block, tier, J->P, slot, &r16, th, sc);
            double acc = 0.0;
            for (int j = 0; j < ORC_NP; j++)
                acc += ((double)sc[j] / L) * lut[j * N + th[j]];
            double lg = J->scale * orc_f16_to_f64(r16) * acc;
            if (n < cap) logit[n] = lg;
            n++;
            if (lg > m) m = lg;
        }
    }
    double *o = J->out + row_q * ORC_D;
    for (int d = 0; d < ORC_D; d++) o[d] = 0.0;
    if (n == 0) { J->lse[row_q] = -INFINITY; return; }
    double sum = 0.0;
    for (int64_t t = 0; t < n; t++) sum += exp(logit[t] - m);
    /* pass 2: weighted values */
    int64_t t = 0;
    for (int i = 0; i < np; i++) {
        int64_t page = J->page_table[row * J->max_pages_per_head + i];
        int tier, count; uint32_t off16;
        meta_read(J->page_meta, page, &tier, &count, &off16);
        for (int slot = 0; slot < count; slot++, t++) {
            double w = exp(logit[t] - m) / sum;
            double v[ORC_D];
            value_read(J->arena + (int64_t)off16 * 16, tier, J->P, slot, v);
            for (int d = 0; d < ORC_D; d++) o[d] += w * v[d];
        }
    }
    J->lse[row_q] = m + log(sum);
}

static void *decode_worker(void *arg)
{
    decode_job_t *J = arg;
    double *lut8 = malloc(sizeof(double) * ORC_NP * 256);
    double *lut4 = malloc(sizeof(double) * ORC_NP * 16);
    double *lut2 = malloc(sizeof(double) * ORC_NP * 4);
    int64_t cap = (int64_t)J->max_pages_per_head * J->P;
    double *logit = malloc(sizeof(double) * (cap > 0 ? cap : 1));
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t r = J->next_row++;
        pthread_mutex_unlock(&J->mu);
        if (r >= J->n_rows) break;
        decode_row(J, r, lut8, lut4, lut2, logit, cap);
    }
    free(lut8); free(lut4); free(lut2); free(logit);
    return NULL;
}

/* rows: optional list of (b*Hq + hq) rows to compute (n_rows entries); when
 * rows == NULL all B*Hq rows are computed.  out/lse are indexed by row. */
int orc_decode(int P, int Hq, int Hkv, int B, int32_t max_pages_per_head,
               const int32_t *page_table, const int32_t *num_pages,
               const uint8_t *page_meta, const uint8_t *arena,
               const float *q, double scale, double *out, double *lse, int nthreads, int layout)
{
    if (Hkv <= 0 || Hq % Hkv != 0 || (P != 16 && P != 32)) return ORC_EINVAL;
    decode_job_t J;
    J.P = P; J.Hq = Hq; J.Hkv = Hkv; J.B = B;
    J.max_pages_per_head = max_pages_per_head;
    J.page_table = page_table; J.num_pages = num_pages;
    J.page_meta = page_meta; J.arena = arena;
    J.q = q; J.scale = scale; J.out = out; J.lse = lse;
    J.next_row = 0; J.n_rows = (int64_t)B * Hq;
    J.layout = layout;
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads < 1) nthreads = 1;
    pthread_t *th = malloc(sizeof(pthread_t) * nthreads);
    for (int i = 0; i < nthreads; i++) pthread_create(&th[i], NULL, decode_worker, &J);
    for (int i = 0; i < nthreads; i++) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.mu);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Attention mass of every kept token in one decode step (the utility signal
 * the RDR packer consumes; the abstract names "estimated future utility"
 * without defining it, and this is the plain reading: the attention the
 * token receives now).  For KV row (b, h) and each of its G query heads hq,
 * the logits and lse are exactly those of orc_decode; the token's utility is
 *     u_t = sum_{hq of h} exp(logit_t(hq) - lse(hq)),
 * accumulated over hq in ascending order and written to
 * util[page * P + slot].  Other entries of util are left unchanged.  Over a
 * row with kept tokens the u_t sum to G.  Threaded over KV rows. */
typedef struct {
    decode_job_t d;          /* shared fields; d.out / d.lse unused */
    double *util;
    int64_t next_kv, n_kv;
} util_job_t;

static void *util_worker(void *arg)
{
    util_job_t *U = arg;
    decode_job_t *J = &U->d;
    int G = J->Hq / J->Hkv;
    double *lut8 = malloc(sizeof(double) * ORC_NP * 256);
    double *lut4 = malloc(sizeof(double) * ORC_NP * 16);
    double *lut2 = malloc(sizeof(double) * ORC_NP * 4);
    int64_t cap = (int64_t)J->max_pages_per_head * J->P;
    double *logit = malloc(sizeof(double) * (cap > 0 ? cap : 1));
    double *u = malloc(sizeof(double) * (cap > 0 ? cap : 1));
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t row = U->next_kv++;
        pthread_mutex_unlock(&J->mu);
        if (row >= U->n_kv) break;
        int b = (int)(row / J->Hkv), h = (int)(row % J->Hkv);
        int np = J->num_pages[row];
        int64_t n = 0;
        for (int g = 0; g < G; g++) {
            const float *q = J->q + ((int64_t)b * J->Hq + (int64_t)h * G + g) * ORC_D;
            orc_lut(q, 8, lut8, J->layout);
            orc_lut(q, 4, lut4, J->layout);
            orc_lut(q, 2, lut2, J->layout);
            double m = -INFINITY;
            n = 0;
            for (int i = 0; i < np; i++) {
                int64_t page = J->page_table[row * J->max_pages_per_head + i];
                int tier, count; uint32_t off16;
                meta_read(J->page_meta, page, &tier, &count, &off16);
                const uint8_t *block = J->arena + (int64_t)off16 * 16;
                int N = 1 << TIER_TB[tier];
                double L = (double)((1 << TIER_SB[tier]) - 1);
                const double *lut = TIER_TB[tier] == 8 ? lut8 : (TIER_TB[tier] == 4 ? lut4 : lut2);
                for (int slot = 0; slot < count; slot++) {
                    uint16_t r16, th[ORC_NP], sc[ORC_NP];
                    read_token_codes(block, tier, J->P, slot, &r16, th, sc);
                    double acc = 0.0;
                    for (int j = 0; j < ORC_NP; j++)
                        acc += ((double)sc[j] / L) * lut[j * N + th[j]];
                    double lg = J->scale * orc_f16_to_f64(r16) * acc;
                    logit[n++] = lg;
                    if (lg > m) m = lg;
                }
            }
            if (n == 0) break;
            double sum = 0.0;
            for (int64_t t = 0; t < n; t++) sum += exp(logit[t] - m);
            double lse = m + log(sum);
            for (int64_t t = 0; t < n; t++) {
                double w = exp(logit[t] - lse);
                u[t] = (g == 0) ? w : u[t] + w;
            }
        }
        int64_t t = 0;
        for (int i = 0; i < np && n > 0; i++) {
            int64_t page = J->page_table[row * J->max_pages_per_head + i];
            int tier, count; uint32_t off16;
            meta_read(J->page_meta, page, &tier, &count, &off16);
            for (int slot = 0; slot < count; slot++, t++) U->util[page * J->P + slot] = u[t];
        }
    }
    free(lut8); free(lut4); free(lut2); free(logit); free(u);
    return NULL;
}

int orc_decode_utility(int P, int Hq, int Hkv, int B, int32_t max_pages_per_head,
                       const int32_t *page_table, const int32_t *num_pages,
                       const uint8_t *page_meta, const uint8_t *arena,
                       const float *q, double scale, double *util, int nthreads, int layout)
{
    if (Hkv <= 0 || Hq % Hkv != 0 || (P != 16 && P != 32)) return ORC_EINVAL;
    util_job_t U;
    memset(&U, 0, sizeof(U));
    decode_job_t *J = &U.d;
    J->P = P; J->Hq = Hq; J->Hkv = Hkv; J->B = B;
    J->max_pages_per_head = max_pages_per_head;
    J->page_table = page_table; J->num_pages = num_pages;
    J->page_meta = page_meta; J->arena = arena;
    J->q = q; J->scale = scale;
    J->layout = layout;
    U.util = util;
    U.next_kv = 0; U.n_kv = (int64_t)B * Hkv;
    pthread_mutex_init(&J->mu, NULL);
    if (nthreads < 1) nthreads = 1;
    pthread_t *th = malloc(sizeof(pthread_t) * nthreads);
    for (int i = 0; i < nthreads; i++) pthread_create(&th[i], NULL, util_worker, &U);
    for (int i = 0; i < nthreads; i++) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J->mu);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Unquantised angle-domain logits (oracle only): r, s_j and theta_j kept as
 * exact fp64 reals, logit = r * sum_j s_j (qx_j cos th_j + qy_j sin th_j)
 * over the pairs of the given layout.  This equals the plain dot product q.k
 * up to rounding. */
void orc_identity_logits(const float *keys, int64_t n, const float *q, double *logits, int layout)
{
    for (int64_t i = 0; i < n; i++) {
        const float *k = keys + i * ORC_D;
        double e[ORC_NP], t[ORC_NP];
        for (int j = 0; j < ORC_NP; j++) {
            double x = k[pair_x(layout, j)], y = k[pair_y(layout, j)];
            e[j] = x * x + y * y;
            t[j] = e[j];
        }
        for (int stride = ORC_NP / 2; stride >= 1; stride /= 2)
            for (int j = 0; j < stride; j++) t[j] = t[j] + t[j + stride];
        double r = sqrt(t[0]);
        double acc = 0.0;
        if (r > 0)
            for (int j = 0; j < ORC_NP; j++) {
                double x = k[pair_x(layout, j)], y = k[pair_y(layout, j)];
                double s = sqrt(e[j]) / r;
                double th = atan2(y, x);
                acc += s * ((double)q[pair_x(layout, j)] * cos(th) + (double)q[pair_y(layout, j)] * sin(th));
            }
        logits[i] = r * acc;
    }
}

/* encode many keys at once (threads not needed; used by tests) */
int orc_encode_many(const float *keys, int64_t n, int tb, int sb, uint16_t *r16,
                    uint16_t *theta, uint16_t *s, int layout)
{
    int worst = ORC_OK;
    for (int64_t i = 0; i < n; i++) {
        int st = orc_encode_key(keys + i * ORC_D, tb, sb, r16 + i, theta + i * ORC_NP, s + i * ORC_NP, NULL, layout);
        if (st > worst) worst = st;
    }
    return worst;
}

int64_t orc_value_index(int slot, int d) { return value_index(slot, d); }
int64_t orc_key_bytes(int tier, int P) { return key_bytes(tier, P); }

void orc_read_token(const uint8_t *arena, const uint8_t *page_meta, int P, int64_t page, int slot,
                    uint16_t *r16, uint16_t *theta, uint16_t *s, int *tier_out)
{
    int tier, count; uint32_t off16;
    meta_read(page_meta, page, &tier, &count, &off16);
    read_token_codes(arena + (int64_t)off16 * 16, tier, P, slot, r16, theta, s);
    *tier_out = tier;
}

void orc_read_values(const uint8_t *arena, const uint8_t *page_meta, int P, int64_t page, int slot, double *v)
{
    int tier, count; uint32_t off16;
    meta_read(page_meta, page, &tier, &count, &off16);
    value_read(arena + (int64_t)off16 * 16, tier, P, slot, v);
}

void orc_f64_to_f16_many(const double *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = orc_f64_to_f16(x[i]);
}
