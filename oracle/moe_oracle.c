/*
 * moe_oracle.c -- plain CPU oracle for the batch-1 decode MoE FFN stage.
 *
 * TEST INFRASTRUCTURE ONLY (see moe_oracle.h).  Slow on purpose: scalar
 * loops, fp64 arithmetic, one explicit rounding per storage point.
 *
 * Source pages:
 *   [P273] "perf(qwen3.6): fused router GEMV+top-k + folded residual-norm (decode)"
 *   [P239] "perf(qwen3.6): fuse decode kernel launches -- shared-expert + GDN conv/L2-norm"
 *   [P359] "perf(qwen36): Q4_K shared-expert FFN kernels + Q8_0/Q5_K->Q4_K requant of the MoE FFN stage"
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* IEEE-754 conversions                                               */
/* ------------------------------------------------------------------ */

static uint32_t f32_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float bits_f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* bf16 keeps the top 16 bits of the fp32 pattern; the dropped 16 bits are
 * rounded to nearest, ties to the even kept pattern.  NaN stays NaN. */
uint16_t orc_f32_to_bf16(float x)
{
    uint32_t u = f32_bits(x);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1u; /* a carry into the exponent is the correct result, inf included */
    return (uint16_t)kept;
}

double orc_bf16_to_f64(uint16_t h) { return (double)bits_f32((uint32_t)h << 16); }

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
uint16_t orc_f32_to_f16(float x)
{
    uint32_t u = f32_bits(x);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t ex = (u >> 23) & 0xFFu;
    uint32_t fr = u & 0x007FFFFFu;
    if (ex == 0xFFu) /* inf or NaN */
        return (uint16_t)(sign | 0x7C00u | (fr ? (0x0200u | (fr >> 13)) : 0u));
    if (ex == 0u) /* fp32 zero or subnormal: below 2^-126, far under half the smallest binary16 */
        return sign;
    int e = (int)ex - 127;              /* value = sig * 2^(e-23), sig has 24 bits */
    uint32_t sig = fr | 0x00800000u;
    if (e > 15)
        return (uint16_t)(sign | 0x7C00u);
    if (e >= -14) {                     /* normal binary16: keep 11 significant bits */
        uint32_t kept = sig >> 13, dropped = sig & 0x1FFFu;
        if (dropped > 0x1000u || (dropped == 0x1000u && (kept & 1u)))
            kept += 1u;
        if (kept == 0x800u) { kept = 0x400u; e += 1; }
        if (e > 15)
            return (uint16_t)(sign | 0x7C00u);
        return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(kept & 0x3FFu));
    }
    /* subnormal binary16: units of 2^-24, so the count is sig * 2^(e+1) */
    int shift = -e - 1;                 /* >= 14 */
    if (shift > 24)
        return sign;                    /* below half the smallest subnormal */
    uint32_t kept = sig >> shift;
    uint32_t dropped = sig & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (dropped > half || (dropped == half && (kept & 1u)))
        kept += 1u;                     /* 0x400 becomes the smallest normal: same encoding */
    return (uint16_t)(sign | kept);
}

double orc_f16_to_f64(uint16_t h)
{
    int s = (h >> 15) & 1, ex = (h >> 10) & 0x1F, fr = h & 0x3FF;
    double v;
    if (ex == 0)
        v = ldexp((double)fr, -24);
    else if (ex == 31)
        v = fr ? NAN : INFINITY;
    else
        v = ldexp((double)(fr | 0x400), ex - 25);
    return s ? -v : v;
}

static double rd_f16(const uint8_t* p) { return orc_f16_to_f64((uint16_t)(p[0] | (p[1] << 8))); }

/* Rounding to the fp32 storage type, then (where stated) to bf16. */
static float st_f32(double v) { return (float)v; }
static uint16_t st_bf16(double v) { return orc_f32_to_bf16((float)v); }

/* Scratch allocation: the oracle has no way to continue without its
 * buffers, so running out of memory ends the process with a message. */
static void* must_alloc(size_t n)
{
    void* p = malloc(n ? n : 1);
    if (!p) {
        fputs("moe_oracle: out of memory\n", stderr);
        abort();
    }
    return p;
}

static void* must_zalloc(size_t n, size_t size)
{
    void* p = calloc(n ? n : 1, size);
    if (!p) {
        fputs("moe_oracle: out of memory\n", stderr);
        abort();
    }
    return p;
}


/* ------------------------------------------------------------------ */
/* Block formats.  The pages name Q4_K, Q5_K, Q8_0 (34 bytes per block) */
/* and Q8_1 ([P359] Summary) but print no bit layout.  Reading: the    */
/* GGUF layouts, since the models are GGUF files and type id 12 is     */
/* Q4_K there.                                                         */
/*   Q4_K (144 B): d f16 @0, dmin f16 @2, scales[12] @4, qs[128] @16.  */
/*   Q5_K (176 B): as Q4_K, then qh[32] @16, qs[128] @48.              */
/*   Q8_0 (34 B):  d f16 @0, q int8[32] @2.                            */
/*   Q8_1 (36 B):  d f16 @0, s f16 @2, q int8[32] @4.                  */
/* ------------------------------------------------------------------ */

/* 6-bit scale and min of the 8 sub-blocks.  Sub-blocks 0..3 keep them in
 * the low 6 bits of scales[j] and scales[j+4]; sub-blocks 4..7 keep the low
 * 4 bits in the two nibbles of scales[j+4] and the top 2 bits in the top
 * 2 bits of scales[j-4] (scale) and scales[j] (min). */
void orc_kquant_scales(const uint8_t* blk, int sc[8], int m[8])
{
    const uint8_t* s = blk + 4;
    for (int j = 0; j < 8; ++j) {
        if (j < 4) {
            sc[j] = s[j] & 63;
            m[j] = s[j + 4] & 63;
        } else {
            sc[j] = (s[j + 4] & 0x0F) | ((s[j - 4] >> 6) << 4);
            m[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
        }
    }
}

/* 4-bit codes: 32-byte group g (0..3) holds elements 64g+l in its low
 * nibbles and elements 64g+32+l in its high nibbles (l = 0..31). */
static void q4k_codes(const uint8_t* blk, int q[256])
{
    const uint8_t* qs = blk + 16;
    for (int g = 0; g < 4; ++g)
        for (int l = 0; l < 32; ++l) {
            q[64 * g + l] = qs[32 * g + l] & 0x0F;
            q[64 * g + 32 + l] = qs[32 * g + l] >> 4;
        }
}

/* 5-bit codes: the low 4 bits as in Q4_K (from qs @48); the fifth bit of
 * element 64g+l is bit 2g of qh[l], of element 64g+32+l bit 2g+1. */
static void q5k_codes(const uint8_t* blk, int q[256])
{
    const uint8_t* qh = blk + 16;
    const uint8_t* qs = blk + 48;
    for (int g = 0; g < 4; ++g)
        for (int l = 0; l < 32; ++l) {
            q[64 * g + l] = (qs[32 * g + l] & 0x0F) | (((qh[l] >> (2 * g)) & 1) << 4);
            q[64 * g + 32 + l] = (qs[32 * g + l] >> 4) | (((qh[l] >> (2 * g + 1)) & 1) << 4);
        }
}

/* Element i of sub-block j = i/32: w = d*sc_j*q_i - dmin*m_j. */
static void kquant_decode(const uint8_t* blk, const int q[256], double out[256])
{
    int sc[8], m[8];
    orc_kquant_scales(blk, sc, m);
    double d = rd_f16(blk), dmin = rd_f16(blk + 2);
    for (int i = 0; i < 256; ++i)
        out[i] = d * sc[i / 32] * q[i] - dmin * m[i / 32];
}

void orc_decode_q4k(const uint8_t* blk, double out[256])
{
    int q[256];
    q4k_codes(blk, q);
    kquant_decode(blk, q, out);
}

void orc_decode_q5k(const uint8_t* blk, double out[256])
{
    int q[256];
    q5k_codes(blk, q);
    kquant_decode(blk, q, out);
}

void orc_decode_q8_0(const uint8_t* blk, double out[32])
{
    double d = rd_f16(blk);
    for (int i = 0; i < 32; ++i)
        out[i] = d * (double)(int8_t)blk[2 + i];
}

void orc_decode_q8_1(const uint8_t* blk, double out[32], double* sum_out)
{
    double d = rd_f16(blk);
    for (int i = 0; i < 32; ++i)
        out[i] = d * (double)(int8_t)blk[4 + i];
    if (sum_out)
        *sum_out = rd_f16(blk + 2);
}

/* ------------------------------------------------------------------ */
/* Load-time requantisation to Q4_K ([P359] Summary: the shared expert */
/* stored as Q8_0 and the routed down projection stored as Q5_K are     */
/* re-quantised to Q4_K once, when the model is loaded).  The pages     */
/* name the step, not the quantiser.  Reading: the source values are    */
/* decoded exactly and rounded once to fp32; each 256-value superblock  */
/* is then quantised by a min/max rule with every step an fp32          */
/* operation rounded to nearest (ties to even):                         */
/*   per 32-value sub-block j: lo = min(0, min x), hi = max x,          */
/*     step_j = (hi - lo) / 15, off_j = -lo;                            */
/*   d = f16(max_j step_j / 63), dmin = f16(max_j off_j / 63);          */
/*   sc_j = clamp(rint(step_j / d), 0, 63) (0 when d = 0), and m_j the  */
/*     same from off_j and dmin;                                        */
/*   q = clamp(rint((x + dmin*m_j) / (d*sc_j)), 0, 15) (0 when d*sc_j   */
/*     = 0);                                                            */
/* then the GGUF Q4_K byte layout (6-bit scale/min packing, nibble      */
/* order of the decoder above).                                         */
/* ------------------------------------------------------------------ */
static float f16_f32(uint16_t h) { return (float)orc_f16_to_f64(h); }

void orc_quantize_q4k(const float x[256], uint8_t blk[144])
{
    float step[8], off[8], maxstep = 0.0f, maxoff = 0.0f;
    for (int j = 0; j < 8; ++j) {
        float mn = x[32 * j], mx = x[32 * j];
        for (int i = 1; i < 32; ++i) {
            if (x[32 * j + i] < mn) mn = x[32 * j + i];
            if (x[32 * j + i] > mx) mx = x[32 * j + i];
        }
        const float lo = mn < 0.0f ? mn : 0.0f;
        volatile float st = (mx - lo) / 15.0f;
        step[j] = st;
        off[j] = -lo;
        if (step[j] > maxstep) maxstep = step[j];
        if (off[j] > maxoff) maxoff = off[j];
    }
    volatile float dq = maxstep / 63.0f, mq = maxoff / 63.0f;
    const uint16_t d16 = orc_f32_to_f16(dq), m16 = orc_f32_to_f16(mq);
    const float d = f16_f32(d16), dmin = f16_f32(m16);
    int sc[8], m[8];
    for (int j = 0; j < 8; ++j) {
        volatile float a = d > 0.0f ? step[j] / d : 0.0f;
        volatile float b = dmin > 0.0f ? off[j] / dmin : 0.0f;
        float ra = rintf(a), rb = rintf(b);
        sc[j] = ra < 0.0f ? 0 : (ra > 63.0f ? 63 : (int)ra);
        m[j] = rb < 0.0f ? 0 : (rb > 63.0f ? 63 : (int)rb);
    }
    int q[256];
    for (int j = 0; j < 8; ++j) {
        volatile float es = d * (float)sc[j];
        volatile float eo = dmin * (float)m[j];
        for (int i = 0; i < 32; ++i) {
            int v = 0;
            if (es > 0.0f) {
                volatile float num = x[32 * j + i] + eo;
                volatile float t = num / es;
                const float r = rintf(t);
                v = r < 0.0f ? 0 : (r > 15.0f ? 15 : (int)r);
            }
            q[32 * j + i] = v;
        }
    }
    blk[0] = (uint8_t)(d16 & 0xFF);
    blk[1] = (uint8_t)(d16 >> 8);
    blk[2] = (uint8_t)(m16 & 0xFF);
    blk[3] = (uint8_t)(m16 >> 8);
    uint8_t* sb = blk + 4;
    for (int j = 0; j < 4; ++j) {
        sb[j] = (uint8_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
        sb[j + 4] = (uint8_t)((m[j] & 63) | ((m[j + 4] >> 4) << 6));
        sb[j + 8] = (uint8_t)((sc[j + 4] & 15) | ((m[j + 4] & 15) << 4));
    }
    for (int p = 0; p < 4; ++p)
        for (int l = 0; l < 32; ++l)
            blk[16 + 32 * p + l] = (uint8_t)(q[64 * p + l] | (q[64 * p + 32 + l] << 4));
}

/* rows of K source elements (Q8_0, Q5_K or Q4_K) -> rows of Q4_K       */
int orc_requant_q4k(const uint8_t* src, int src_type, int n_rows, int K, uint8_t* dst)
{
    if (K % 256)
        return -1;
    const long sb_src = (src_type == ORC_Q8_0) ? 8L * ORC_Q80_BYTES
                      : (src_type == ORC_Q5_K) ? ORC_Q5K_BYTES
                      : (src_type == ORC_Q4_K) ? ORC_Q4K_BYTES : -1;
    if (sb_src < 0)
        return -1;
    const int nsb = K / 256;
#pragma omp parallel for schedule(static)
    for (long t = 0; t < (long)n_rows * nsb; ++t) {
        const uint8_t* s = src + t * sb_src;
        double v[256];
        if (src_type == ORC_Q8_0)
            for (int b = 0; b < 8; ++b)
                orc_decode_q8_0(s + b * ORC_Q80_BYTES, v + 32 * b);
        else if (src_type == ORC_Q5_K)
            orc_decode_q5k(s, v);
        else
            orc_decode_q4k(s, v);
        float x[256];
        for (int i = 0; i < 256; ++i)
            x[i] = (float)v[i];
        orc_quantize_q4k(x, dst + t * ORC_Q4K_BYTES);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Q8_1 activation quantiser ([P359] Summary: the shared-expert path    */
/* quantises the normed activations and the SwiGLU output to Q8_1).    */
/* Reading: per 32 values, d = amax/127 in fp32, codes are the fp32     */
/* product x*(1/d) rounded half away from zero; d is stored as fp16;   */
/* s is the fp16 of d16 times the code sum (the value the codes        */
/* represent, reproducible from the block).  An all-zero block stores  */
/* zeros.  The code decision is taken in fp32 on purpose: a float      */
/* decides an integer, so the precision is fixed, not fp64.            */
/* ------------------------------------------------------------------ */
void orc_quantize_q8_1(const float* x, int n, uint8_t* out)
{
    for (int b = 0; b < n / 32; ++b) {
        const float* xb = x + 32 * b;
        uint8_t* ob = out + ORC_Q81_BYTES * b;
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i) {
            float a = fabsf(xb[i]);
            if (a > amax)
                amax = a;
        }
        memset(ob, 0, ORC_Q81_BYTES);
        if (amax == 0.0f)
            continue;
        volatile float d32 = amax / 127.0f;   /* fp32 division, correctly rounded */
        volatile float id = 1.0f / d32;
        int qsum = 0;
        for (int i = 0; i < 32; ++i) {
            volatile float t = xb[i] * id;    /* fp32 product */
            float r = roundf(t);              /* half away from zero */
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            int q = (int)r;
            ob[4 + i] = (uint8_t)(int8_t)q;
            qsum += q;
        }
        uint16_t d16 = orc_f32_to_f16(d32);
        /* d16 has 11 significant bits and |qsum| <= 4064, so this fp32 product is exact */
        float s = (float)orc_f16_to_f64(d16) * (float)qsum;
        uint16_t s16 = orc_f32_to_f16(s);
        ob[0] = (uint8_t)(d16 & 0xFF);
        ob[1] = (uint8_t)(d16 >> 8);
        ob[2] = (uint8_t)(s16 & 0xFF);
        ob[3] = (uint8_t)(s16 >> 8);
    }
}

/* ------------------------------------------------------------------ */
/* Quantised row x Q8_1 activations ([P359] Summary: the weight dot is  */
/* an int8 dot of the weight codes with the Q8_1 codes; sub-block j of  */
/* superblock b pairs with activation block 8b+j).                      */
/* ------------------------------------------------------------------ */
long orc_row_bytes(int type, int K)
{
    switch (type) {
    case ORC_Q4_K: return (K % 256) ? 0 : (long)(K / 256) * ORC_Q4K_BYTES;
    case ORC_Q5_K: return (K % 256) ? 0 : (long)(K / 256) * ORC_Q5K_BYTES;
    case ORC_Q8_0: return (K % 32) ? 0 : (long)(K / 32) * ORC_Q80_BYTES;
    default: return 0;
    }
}

int orc_pad_k(int type, int K)
{
    if (type == ORC_Q4_K || type == ORC_Q5_K)
        return (K + 255) / 256 * 256;
    return (K + 31) / 32 * 32;
}

int orc_subblock_dots(const uint8_t* row, int type, int K, const uint8_t* xq, int32_t* out)
{
    if (orc_row_bytes(type, K) == 0)
        return -1;
    if (type == ORC_Q8_0) {
        for (int j = 0; j < K / 32; ++j) {
            const uint8_t* w = row + ORC_Q80_BYTES * j;
            const uint8_t* a = xq + ORC_Q81_BYTES * j;
            int32_t D = 0;
            for (int i = 0; i < 32; ++i)
                D += (int32_t)(int8_t)w[2 + i] * (int32_t)(int8_t)a[4 + i];
            out[j] = D;
        }
        return 0;
    }
    int bytes = (type == ORC_Q4_K) ? ORC_Q4K_BYTES : ORC_Q5K_BYTES;
    for (int b = 0; b < K / 256; ++b) {
        int q[256];
        if (type == ORC_Q4_K)
            q4k_codes(row + (long)bytes * b, q);
        else
            q5k_codes(row + (long)bytes * b, q);
        for (int j = 0; j < 8; ++j) {
            const uint8_t* a = xq + ORC_Q81_BYTES * (8 * b + j);
            int32_t D = 0;
            for (int i = 0; i < 32; ++i)
                D += q[32 * j + i] * (int32_t)(int8_t)a[4 + i];
            out[8 * b + j] = D;
        }
    }
    return 0;
}

/* K-quant row: sum over superblocks b and sub-blocks j of
 *   d_b*sc_bj*d_a*D_bj - dmin_b*m_bj*s_a
 * (the min term uses the stored activation sum s_a).  Q8_0 row: sum over
 * blocks of d_w*d_a*D.  Every product is exact in fp64; only the running
 * sum rounds. */
double orc_row_dot(const uint8_t* row, int type, int K, const uint8_t* xq)
{
    int nsub = K / 32;
    int32_t D[ORC_MAX_K / 32];
    if (K > ORC_MAX_K || orc_subblock_dots(row, type, K, xq, D) != 0)
        return NAN;
    double acc = 0.0;
    if (type == ORC_Q8_0) {
        for (int j = 0; j < nsub; ++j)
            acc += rd_f16(row + ORC_Q80_BYTES * j) * rd_f16(xq + ORC_Q81_BYTES * j) * (double)D[j];
    } else {
        int bytes = (type == ORC_Q4_K) ? ORC_Q4K_BYTES : ORC_Q5K_BYTES;
        for (int b = 0; b < K / 256; ++b) {
            const uint8_t* blk = row + (long)bytes * b;
            int sc[8], m[8];
            orc_kquant_scales(blk, sc, m);
            double d = rd_f16(blk), dmin = rd_f16(blk + 2);
            for (int j = 0; j < 8; ++j) {
                const uint8_t* a = xq + ORC_Q81_BYTES * (8 * b + j);
                double da = rd_f16(a), sa = rd_f16(a + 2);
                acc += d * sc[j] * da * (double)D[8 * b + j] - dmin * m[j] * sa;
            }
        }
    }
    return acc;
}

/* ------------------------------------------------------------------ */
/* a1: residual add folded into RMSNorm ([P273] Summary item 2: the     */
/* routed+shared residual add is folded into a 3-input add_rmsnorm3,    */
/* bit-identical to the separate add followed by the 2-input norm).     */
/* Readings: t = bf16(routed+shared); u = bf16(residual+t) is stored     */
/* (out_sum) and the norm reads that bf16 sum back (the 3-input kernel   */
/* keeps the out_sum reload, [P273] Relation to open PRs); RMSNorm is    */
/* u*(1/sqrt(mean(u^2)+eps))*w with an fp32 weight; xn stays fp32 (the   */
/* router is an fp32 GEMV) and xq is its Q8_1.                          */
/* ------------------------------------------------------------------ */
void orc_add_rmsnorm(const uint16_t* residual, const uint16_t* routed, const uint16_t* shared,
                     const float* w, int H, float eps,
                     uint16_t* out_sum, float* xn, uint8_t* xq)
{
    double* u = (double*)must_alloc(sizeof(double) * (size_t)H);
    for (int i = 0; i < H; ++i) {
        double t;
        if (routed && shared)
            t = orc_bf16_to_f64(st_bf16(orc_bf16_to_f64(routed[i]) + orc_bf16_to_f64(shared[i])));
        else if (routed)
            t = orc_bf16_to_f64(routed[i]);
        else
            t = 0.0;
        uint16_t ub = st_bf16(orc_bf16_to_f64(residual[i]) + t);
        if (out_sum)
            out_sum[i] = ub;
        u[i] = orc_bf16_to_f64(ub);
    }
    double ss = 0.0;
    for (int i = 0; i < H; ++i)
        ss += u[i] * u[i];
    double r = 1.0 / sqrt(ss / (double)H + (double)eps);
    float* xf = (float*)must_alloc(sizeof(float) * (size_t)H);
    for (int i = 0; i < H; ++i)
        xf[i] = st_f32((u[i] * r) * (double)w[i]);
    if (xn)
        memcpy(xn, xf, sizeof(float) * (size_t)H);
    if (xq)
        orc_quantize_q8_1(xf, H, xq);
    free(xf);
    free(u);
}

/* ------------------------------------------------------------------ */
/* a2: fp32 router GEMV over the experts ([P273] Summary item 1: a       */
/* split-K fp32 GEMV writes the expert logits).  No bias is mentioned,   */
/* so none is added.                                                     */
/* ------------------------------------------------------------------ */
void orc_router(const float* xn, const float* W, int E, int H, float* logits)
{
    int e;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (e = 0; e < E; ++e) {
        double acc = 0.0;
        for (int i = 0; i < H; ++i)
            acc += (double)W[(long)e * H + i] * (double)xn[i];
        logits[e] = st_f32(acc);
    }
}

/* ------------------------------------------------------------------ */
/* a3: top-k ([P273] Summary item 1: selection by value descending,      */
/* ties to the lower expert index, the same as the O(E^2) rank scan).    */
/* rank_e = #{e' : l_e' > l_e} + #{e' < e : l_e' == l_e}; expert e takes */
/* output slot rank_e when rank_e < k.  Reading: IEEE comparison (so     */
/* -0 and +0 tie) and a NaN logit ranks as -inf.                         */
/* ------------------------------------------------------------------ */
static double rank_key(float v) { return isnan(v) ? -INFINITY : (double)v; }

void orc_topk(const float* logits, int E, int k, int32_t* ids)
{
    for (int e = 0; e < E; ++e) {
        double le = rank_key(logits[e]);
        int rank = 0;
        for (int f = 0; f < E; ++f) {
            double lf = rank_key(logits[f]);
            if (lf > le || (f < e && lf == le))
                ++rank;
        }
        if (rank < k)
            ids[rank] = e;
    }
}

/* Routing weights.  The pages never state them; reading: a softmax over
 * the k selected logits, shifted by the largest (slot 0), no extra
 * renormalisation, scale or bias. */
void orc_softmax_selected(const float* logits, const int32_t* ids, int k, float* w)
{
    double m = (double)logits[ids[0]];
    double* p = (double*)must_alloc(sizeof(double) * (size_t)k);
    double s = 0.0;
    for (int j = 0; j < k; ++j) {
        p[j] = exp((double)logits[ids[j]] - m);
        s += p[j];
    }
    for (int j = 0; j < k; ++j)
        w[j] = st_f32(p[j] / s);
    free(p);
}

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }
static double silu(double x) { return x / (1.0 + exp(-x)); }

void orc_router_topk(const orc_desc* d, const orc_weights* w, const float* xn,
                     float* logits, float* z, int32_t* ids, float* weights, float* shared_gate)
{
    orc_router(xn, w->router_w, d->E, d->H, logits);
    orc_topk(logits, d->E, d->k, ids);
    orc_softmax_selected(logits, ids, d->k, weights);
    /* Shared-expert gate: one more fp32 row dotted with xn, squashed by a
     * sigmoid (the shared gate is a GEMV with a sigmoid, [P273] Relation to
     * open PRs); the sigmoid value is stored as fp32. */
    if (d->Fs > 0 && w->shared_gate_w) {
        double acc = 0.0;
        for (int i = 0; i < d->H; ++i)
            acc += (double)w->shared_gate_w[i] * (double)xn[i];
        float zf = st_f32(acc);
        if (z) *z = zf;
        if (shared_gate) *shared_gate = st_f32(sigmoid((double)zf));
    } else {
        if (z) *z = 0.0f;
        if (shared_gate) *shared_gate = 0.0f;
    }
}

/* ------------------------------------------------------------------ */
/* a4..a6: expert FFN ([P359] Summary: Q8_1 activations -> gate/up with  */
/* SiLU -> Q8_1 of the product -> down; [P239] Summary item 1: gate and  */
/* up of the shared expert share one pass over the activations).         */
/* Readings: h = silu(g)*u with silu(x) = x/(1+e^-x) on the gate row,     */
/* h kept in fp32 and quantised to Q8_1 (no bf16 step on this path);      */
/* down rows longer than F are zero-padded to a whole superblock and the  */
/* padding activations are zero Q8_1 blocks; the routed outputs are       */
/* combined in slot order in fp64 and rounded once; the shared output is  */
/* scaled by the stored sigmoid gate before its one rounding.             */
/* ------------------------------------------------------------------ */

/* h (F values) -> Q8_1 blocks for a down row of Kp >= F elements. */
static void quantize_h_padded(const float* h, int F, int Kp, uint8_t* hq)
{
    memset(hq, 0, (size_t)(Kp / 32) * ORC_Q81_BYTES);
    orc_quantize_q8_1(h, F, hq);
}

static void ffn_gate_up(const uint8_t* gate, const uint8_t* up, int type, int H, int F,
                        const uint8_t* xq, float* h)
{
    long rb = orc_row_bytes(type, H);
    int f;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (f = 0; f < F; ++f) {
        float g = st_f32(orc_row_dot(gate + rb * f, type, H, xq));
        float u = st_f32(orc_row_dot(up + rb * f, type, H, xq));
        h[f] = st_f32(silu((double)g) * (double)u);
    }
}

static void ffn_down(const uint8_t* down, int type, int H, int Kp, const uint8_t* hq, float* y)
{
    long rb = orc_row_bytes(type, Kp);
    int i;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (i = 0; i < H; ++i)
        y[i] = st_f32(orc_row_dot(down + rb * i, type, Kp, hq));
}

void orc_expert_ffn(const orc_desc* d, const orc_weights* w, const uint8_t* xq,
                    const int32_t* ids, const float* weights, float shared_gate,
                    orc_layer_out* o)
{
    int H = d->H, F = d->F, k = d->k, Fs = d->Fs;
    int Kp = orc_pad_k(d->down_type, F);
    long gu_rb = orc_row_bytes(d->gate_up_type, H);
    long dn_rb = orc_row_bytes(d->down_type, Kp);
    float* h = (float*)must_alloc(sizeof(float) * (size_t)k * F);
    float* y = (float*)must_alloc(sizeof(float) * (size_t)k * H);
    uint8_t* hq = (uint8_t*)must_alloc((size_t)(Kp / 32) * ORC_Q81_BYTES);
    for (int s = 0; s < k; ++s) {
        long e = ids[s];
        ffn_gate_up(w->gate + e * F * gu_rb, w->up + e * F * gu_rb, d->gate_up_type, H, F, xq, h + (long)s * F);
        quantize_h_padded(h + (long)s * F, F, Kp, hq);
        ffn_down(w->down + e * H * dn_rb, d->down_type, H, Kp, hq, y + (long)s * H);
    }
    for (int i = 0; i < H; ++i) {
        double acc = 0.0;
        for (int s = 0; s < k; ++s)
            acc += (double)weights[s] * (double)y[(long)s * H + i];
        if (o->routed_exact) o->routed_exact[i] = acc;
        if (o->routed) o->routed[i] = st_bf16(acc);
    }
    if (o->h) memcpy(o->h, h, sizeof(float) * (size_t)k * F);
    if (o->y) memcpy(o->y, y, sizeof(float) * (size_t)k * H);
    free(hq);
    free(y);
    free(h);

    if (Fs > 0) {
        int Kps = orc_pad_k(d->shared_type, Fs);
        float* hs = (float*)must_alloc(sizeof(float) * (size_t)Fs);
        float* ys = (float*)must_alloc(sizeof(float) * (size_t)H);
        uint8_t* hqs = (uint8_t*)must_alloc((size_t)(Kps / 32) * ORC_Q81_BYTES);
        ffn_gate_up(w->sgate, w->sup, d->shared_type, H, Fs, xq, hs);
        quantize_h_padded(hs, Fs, Kps, hqs);
        ffn_down(w->sdown, d->shared_type, H, Kps, hqs, ys);
        for (int i = 0; i < H; ++i) {
            double v = (double)shared_gate * (double)ys[i];
            if (o->shared_exact) o->shared_exact[i] = v;
            if (o->shared) o->shared[i] = st_bf16(v);
        }
        if (o->hs) memcpy(o->hs, hs, sizeof(float) * (size_t)Fs);
        if (o->ys) memcpy(o->ys, ys, sizeof(float) * (size_t)H);
        free(hqs);
        free(ys);
        free(hs);
    } else {
        for (int i = 0; i < H; ++i) {
            if (o->shared_exact) o->shared_exact[i] = 0.0;
            if (o->shared) o->shared[i] = 0;
        }
    }
}

static int desc_ok(const orc_desc* d)
{
    if (d->H > ORC_MAX_K || d->F > ORC_MAX_K || d->Fs > ORC_MAX_K)
        return 0;
    if (d->H <= 0 || d->H % 256 || d->E <= 0 || d->k <= 0 || d->k > d->E || d->F <= 0 || d->F % 32)
        return 0;
    if (d->Fs < 0 || d->Fs % 32)
        return 0;
    if (d->gate_up_type != ORC_Q4_K)
        return 0;
    if (d->down_type != ORC_Q4_K && d->down_type != ORC_Q5_K)
        return 0;
    if (d->Fs > 0 && d->shared_type != ORC_Q4_K && d->shared_type != ORC_Q8_0)
        return 0;
    return 1;
}

/* One layer; ids_in == NULL takes the selection from the top-k, otherwise
 * ids_in[0..k) is the selection in slot order. */
static int moe_layer_impl(const orc_desc* d, const orc_weights* w,
                          const uint16_t* residual, const uint16_t* routed_prev, const uint16_t* shared_prev,
                          const float* x, const int32_t* ids_in, orc_layer_out* o)
{
    if (!desc_ok(d))
        return -1;
    if (ids_in) {
        for (int s = 0; s < d->k; ++s) {
            if (ids_in[s] < 0 || ids_in[s] >= d->E)
                return -1;
            for (int t = 0; t < s; ++t)
                if (ids_in[t] == ids_in[s])
                    return -1;
        }
    }
    int H = d->H, E = d->E, k = d->k;
    float* xn = (float*)must_alloc(sizeof(float) * (size_t)H);
    uint8_t* xq = (uint8_t*)must_alloc((size_t)(H / 32) * ORC_Q81_BYTES);
    float* logits = (float*)must_alloc(sizeof(float) * (size_t)E);
    int32_t* ids = (int32_t*)must_alloc(sizeof(int32_t) * (size_t)k);
    float* wts = (float*)must_alloc(sizeof(float) * (size_t)k);
    float z = 0.0f, sg = 0.0f;
    if (d->norm) {
        orc_add_rmsnorm(residual, routed_prev, shared_prev, w->norm_w, H, d->eps, o->out_sum, xn, xq);
    } else {
        memcpy(xn, x, sizeof(float) * (size_t)H);
        orc_quantize_q8_1(xn, H, xq);
    }
    orc_router_topk(d, w, xn, logits, &z, ids, wts, &sg);
    if (ids_in) {
        /* the given selection; its weights are the softmax over its logits */
        memcpy(ids, ids_in, sizeof(int32_t) * (size_t)k);
        orc_softmax_selected(logits, ids, k, wts);
    }
    orc_expert_ffn(d, w, xq, ids, wts, sg, o);
    if (o->xn) memcpy(o->xn, xn, sizeof(float) * (size_t)H);
    if (o->xq) memcpy(o->xq, xq, (size_t)(H / 32) * ORC_Q81_BYTES);
    if (o->logits) memcpy(o->logits, logits, sizeof(float) * (size_t)E);
    if (o->z) *o->z = z;
    if (o->shared_gate) *o->shared_gate = sg;
    if (o->ids) memcpy(o->ids, ids, sizeof(int32_t) * (size_t)k);
    if (o->weights) memcpy(o->weights, wts, sizeof(float) * (size_t)k);
    free(wts);
    free(ids);
    free(logits);
    free(xq);
    free(xn);
    return 0;
}

int orc_moe_layer(const orc_desc* d, const orc_weights* w,
                  const uint16_t* residual, const uint16_t* routed_prev, const uint16_t* shared_prev,
                  const float* x, orc_layer_out* o)
{
    return moe_layer_impl(d, w, residual, routed_prev, shared_prev, x, NULL, o);
}

/* Reading of the near-tie rule for chained comparisons: two implementations
 * whose inputs to a layer differ by rounding may order two almost equal
 * logits differently, and both selections are then correct.  The oracle can
 * continue such a comparison with the other side's selection: the layer is
 * computed as defined, except that the experts are the given ones (in the
 * given slot order) and the routing weights the softmax over their logits. */
int orc_moe_layer_sel(const orc_desc* d, const orc_weights* w,
                      const uint16_t* residual, const uint16_t* routed_prev, const uint16_t* shared_prev,
                      const float* x, const int32_t* ids_in, orc_layer_out* o)
{
    if (!ids_in)
        return -1;
    return moe_layer_impl(d, w, residual, routed_prev, shared_prev, x, ids_in, o);
}


/* ------------------------------------------------------------------ */
/* a8: several tokens at once, grouped by expert.  The pages cover batch 1 */
/* only; reading: the tokens whose top-k contains expert e form its group  */
/* and the shared expert is one group of all tokens; every member of a     */
/* group gets exactly what the batch-1 integer path (a4/a5) gives it, so   */
/* the result does not depend on the batch it runs in.  Norm, router,      */
/* top-k, weights and the combine are the single-token steps per token.    */
/* ------------------------------------------------------------------ */

/* Q8_1 integer path of one expert for one token (a4/a5). */
static void expert_int(const uint8_t* gate, const uint8_t* up, int gu_type, const uint8_t* down, int dn_type,
                       int H, int F, int Kp, const uint8_t* xq, float* h, float* y)
{
    uint8_t* hq = (uint8_t*)must_alloc((size_t)(Kp / 32) * ORC_Q81_BYTES);
    ffn_gate_up(gate, up, gu_type, H, F, xq, h);
    quantize_h_padded(h, F, Kp, hq);
    ffn_down(down, dn_type, H, Kp, hq, y);
    free(hq);
}

int orc_moe_layer_batch(const orc_desc* d, const orc_weights* w, int n_tok,
                        const uint16_t* residual, const uint16_t* routed_prev, const uint16_t* shared_prev,
                        const float* x, orc_batch_out* o)
{
    if (!desc_ok(d) || n_tok <= 0)
        return -1;
    int H = d->H, E = d->E, k = d->k, F = d->F, Fs = d->Fs;
    int Kp = orc_pad_k(d->down_type, F);
    int Kps = Fs > 0 ? orc_pad_k(d->shared_type, Fs) : 0;
    long gu_rb = orc_row_bytes(d->gate_up_type, H);
    long dn_rb = orc_row_bytes(d->down_type, Kp);
    float* xn = (float*)must_alloc(sizeof(float) * (size_t)n_tok * H);
    uint8_t* xq = (uint8_t*)must_alloc((size_t)n_tok * (H / 32) * ORC_Q81_BYTES);
    int32_t* ids = (int32_t*)must_alloc(sizeof(int32_t) * (size_t)n_tok * k);
    float* wts = (float*)must_alloc(sizeof(float) * (size_t)n_tok * k);
    float* sg = (float*)must_alloc(sizeof(float) * (size_t)n_tok);
    float* logits = (float*)must_alloc(sizeof(float) * (size_t)E);
    float* y = (float*)must_alloc(sizeof(float) * (size_t)n_tok * k * H);
    float* ys = (float*)must_alloc(sizeof(float) * (size_t)n_tok * H);
    int* cnt = (int*)must_zalloc((size_t)E, sizeof(int));
    int* toks = (int*)must_alloc(sizeof(int) * (size_t)n_tok);
    int* slot_of = (int*)must_alloc(sizeof(int) * (size_t)n_tok);

    /* a1..a3 per token */
    for (int t = 0; t < n_tok; ++t) {
        float* xt = xn + (long)t * H;
        uint8_t* qt = xq + (long)t * (H / 32) * ORC_Q81_BYTES;
        if (d->norm) {
            orc_add_rmsnorm(residual + (long)t * H, routed_prev ? routed_prev + (long)t * H : NULL,
                            shared_prev ? shared_prev + (long)t * H : NULL, w->norm_w, H, d->eps,
                            o->out_sum ? o->out_sum + (long)t * H : NULL, xt, qt);
        } else {
            memcpy(xt, x + (long)t * H, sizeof(float) * (size_t)H);
            orc_quantize_q8_1(xt, H, qt);
        }
        float z;
        orc_router_topk(d, w, xt, logits, &z, ids + (long)t * k, wts + (long)t * k, &sg[t]);
    }
    /* group sizes */
    for (int t = 0; t < n_tok; ++t)
        for (int s = 0; s < k; ++s)
            cnt[ids[(long)t * k + s]] += 1;
    /* routed experts, one group at a time, in expert order */
    for (int e = 0; e < E; ++e) {
        if (cnt[e] == 0) continue;
        int nt = 0;
        for (int t = 0; t < n_tok; ++t)
            for (int s = 0; s < k; ++s)
                if (ids[(long)t * k + s] == e) { toks[nt] = t; slot_of[nt] = s; ++nt; }
        const uint8_t* G = w->gate + (long)e * F * gu_rb;
        const uint8_t* U = w->up + (long)e * F * gu_rb;
        const uint8_t* D = w->down + (long)e * H * dn_rb;
        float* h = (float*)must_alloc(sizeof(float) * (size_t)nt * F);
        float* ye = (float*)must_alloc(sizeof(float) * (size_t)nt * H);
        for (int j = 0; j < nt; ++j)
            expert_int(G, U, d->gate_up_type, D, d->down_type, H, F, Kp,
                       xq + (long)toks[j] * (H / 32) * ORC_Q81_BYTES, h + (long)j * F, ye + (long)j * H);
        for (int j = 0; j < nt; ++j) {
            memcpy(y + ((long)toks[j] * k + slot_of[j]) * H, ye + (long)j * H, sizeof(float) * (size_t)H);
            if (o->h) memcpy(o->h + ((long)toks[j] * k + slot_of[j]) * F, h + (long)j * F, sizeof(float) * (size_t)F);
        }
        free(ye);
        free(h);
    }
    /* shared expert: one group of all tokens */
    if (Fs > 0) {
        float* hs = (float*)must_alloc(sizeof(float) * (size_t)n_tok * Fs);
        for (int t = 0; t < n_tok; ++t)
            expert_int(w->sgate, w->sup, d->shared_type, w->sdown, d->shared_type, H, Fs, Kps,
                       xq + (long)t * (H / 32) * ORC_Q81_BYTES, hs + (long)t * Fs, ys + (long)t * H);
        if (o->hs) memcpy(o->hs, hs, sizeof(float) * (size_t)n_tok * Fs);
        free(hs);
    }
    /* combine per token, slot order */
    for (int t = 0; t < n_tok; ++t) {
        for (int i = 0; i < H; ++i) {
            double acc = 0.0;
            for (int s = 0; s < k; ++s)
                acc += (double)wts[(long)t * k + s] * (double)y[((long)t * k + s) * H + i];
            if (o->routed_exact) o->routed_exact[(long)t * H + i] = acc;
            if (o->routed) o->routed[(long)t * H + i] = st_bf16(acc);
            double v = Fs > 0 ? (double)sg[t] * (double)ys[(long)t * H + i] : 0.0;
            if (o->shared_exact) o->shared_exact[(long)t * H + i] = v;
            if (o->shared) o->shared[(long)t * H + i] = Fs > 0 ? st_bf16(v) : 0;
        }
        for (int s = 0; s < k; ++s)
            if (o->group_size) o->group_size[(long)t * k + s] = cnt[ids[(long)t * k + s]];
    }
    if (o->xn) memcpy(o->xn, xn, sizeof(float) * (size_t)n_tok * H);
    if (o->xq) memcpy(o->xq, xq, (size_t)n_tok * (H / 32) * ORC_Q81_BYTES);
    if (o->ids) memcpy(o->ids, ids, sizeof(int32_t) * (size_t)n_tok * k);
    if (o->weights) memcpy(o->weights, wts, sizeof(float) * (size_t)n_tok * k);
    if (o->shared_gate) memcpy(o->shared_gate, sg, sizeof(float) * (size_t)n_tok);
    if (o->y) memcpy(o->y, y, sizeof(float) * (size_t)n_tok * k * H);
    if (o->ys) memcpy(o->ys, ys, sizeof(float) * (size_t)n_tok * H);
    free(slot_of);
    free(toks);
    free(cnt);
    free(ys);
    free(y);
    free(logits);
    free(sg);
    free(wts);
    free(ids);
    free(xq);
    free(xn);
    return 0;
}

/* Stack of L layers for one token.  Layer l reads the residual stream and
 * the previous layer's routed/shared outputs (zero before layer 0, so the
 * first norm sees the input itself); the stack output is the residual plus
 * the last layer's routed+shared, folded the same way the next norm would.
 * Requires norm = 1. */
int orc_moe_stack(const orc_desc* d, const orc_weights* layers, int L,
                  const uint16_t* input, const uint16_t* attn_per_layer, uint16_t* output,
                  int32_t* ids_per_layer, uint16_t* routed_per_layer,
                  uint16_t* shared_per_layer, uint16_t* resid_per_layer)
{
    if (!desc_ok(d) || !d->norm || L <= 0)
        return -1;
    int H = d->H;
    uint16_t* res = (uint16_t*)must_alloc(sizeof(uint16_t) * (size_t)H);
    uint16_t* routed = (uint16_t*)must_alloc(sizeof(uint16_t) * (size_t)H);
    uint16_t* shared = (uint16_t*)must_alloc(sizeof(uint16_t) * (size_t)H);
    uint16_t* nres = (uint16_t*)must_alloc(sizeof(uint16_t) * (size_t)H);
    memcpy(res, input, sizeof(uint16_t) * (size_t)H);
    memset(routed, 0, sizeof(uint16_t) * (size_t)H);
    memset(shared, 0, sizeof(uint16_t) * (size_t)H);
    int rc = 0;
    for (int l = 0; l < L && rc == 0; ++l) {
        orc_layer_out o;
        memset(&o, 0, sizeof(o));
        uint16_t* nrouted = (uint16_t*)must_alloc(sizeof(uint16_t) * (size_t)H);
        uint16_t* nshared = (uint16_t*)must_alloc(sizeof(uint16_t) * (size_t)H);
        o.out_sum = nres;
        o.routed = nrouted;
        o.shared = nshared;
        if (ids_per_layer) o.ids = ids_per_layer + (long)l * d->k;
        if (attn_per_layer) {
            /* Reading of the layer behind an attention block: the fold of the
             * previous outputs (the add that precedes the attention's input
             * norm) gives u1; the attention block is outside this stage, its
             * bf16 output is an input; the post-attention add-norm takes
             * bf16(u1 + attn) as the residual it normalises for the experts
             * ([P273] Relation to open PRs: add_rmsnorm2_q8 after the
             * attention, add_rmsnorm3 folding the expert outputs). */
            for (int i = 0; i < H; ++i) {
                double t = d->Fs > 0
                    ? orc_bf16_to_f64(st_bf16(orc_bf16_to_f64(routed[i]) + orc_bf16_to_f64(shared[i])))
                    : orc_bf16_to_f64(routed[i]);
                nres[i] = st_bf16(orc_bf16_to_f64(res[i]) + t);
            }
            rc = orc_moe_layer(d, &layers[l], nres, attn_per_layer + (long)l * H, NULL, NULL, &o);
        } else {
            rc = orc_moe_layer(d, &layers[l], res, routed, d->Fs > 0 ? shared : NULL, NULL, &o);
        }
        memcpy(res, nres, sizeof(uint16_t) * (size_t)H);
        memcpy(routed, nrouted, sizeof(uint16_t) * (size_t)H);
        memcpy(shared, nshared, sizeof(uint16_t) * (size_t)H);
        if (routed_per_layer) memcpy(routed_per_layer + (long)l * H, nrouted, sizeof(uint16_t) * (size_t)H);
        if (shared_per_layer) memcpy(shared_per_layer + (long)l * H, nshared, sizeof(uint16_t) * (size_t)H);
        if (resid_per_layer) memcpy(resid_per_layer + (long)l * H, nres, sizeof(uint16_t) * (size_t)H);
        free(nshared);
        free(nrouted);
    }
    if (rc == 0) {
        for (int i = 0; i < H; ++i) {
            double t = d->Fs > 0
                ? orc_bf16_to_f64(st_bf16(orc_bf16_to_f64(routed[i]) + orc_bf16_to_f64(shared[i])))
                : orc_bf16_to_f64(routed[i]);
            output[i] = st_bf16(orc_bf16_to_f64(res[i]) + t);
        }
    }
    free(nres);
    free(shared);
    free(routed);
    free(res);
    return rc;
}

void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
