/*
 * oracle.c -- plain, slow CPU reference for the quantized-weight matvec /
 * skinny GEMM  Y[M,N] = X[M,K] . dequant(Wq[N,K])^T  and its fused variants.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test-suite, the package smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code, header, table or
 * constant generator with the HIP library; both are written independently
 * from the same definitions.
 *
 * Build: gcc -O2 -ffp-contract=off (no -ffast-math, no FTZ/DAZ).  Every fp32
 * operation below is one IEEE-754 binary32 operation rounded to nearest-even;
 * nothing is contracted into an FMA unless written as fmaf().
 *
 * Sources (cited by page title and section):
 *  [A19]  "Gemma4 raw-Metal loop on A19 -- findings + the remaining (parked)
 *         levers", section "What moved the needle": int2 weights hold 16 codes
 *         per 32-bit word, a byte decodes to 4 values, the products x*c with
 *         c in {-2,-1,0,1} are exact and the fp32 accumulation follows code
 *         order, so the result is bit-exact; the residual-add RMSNorm is
 *         folded into the next matvec; the decode-side and verify-side tile
 *         must agree because the tile changes the fp32 strided-merge order.
 *         Section "The parked levers": argmax with the first-max tie-break.
 *  [PB]   "raw-Metal loop playbook", prefill route table: for M = 8/16 keep
 *         every output scalar's K-dot in the M = 1 accumulation order while
 *         the weights are shared across the M columns.  Next-target ranking
 *         table: an expert-gather matvec that reads the selected experts'
 *         weights in place (gpt-oss MoE).
 *  [GEM]  "Gemma 4 Optimization with Agentic Kernel Engineering", sections
 *         "A new chip, the same model" and "How much of the chip we use now":
 *         MXFP4 weights on MI355X.  The MXFP4 element and scale encodings are
 *         those of the OCP Microscaling Formats specification v1.0 (E2M1
 *         elements, E8M0 shared scale per 32 elements).
 *
 * The fixed order (FO) -- the pages require a frozen order but do not spell
 * one out; this is the plainest order they support (the per-lane sequential
 * partial sums merged by a fixed strided pattern of [A19]):
 *   segment = 16 consecutive bytes of a row's packed codes
 *             (int2: 64 codes, int4: 32 codes, MXFP4: 32 codes);
 *   t_j     = +0, then t_j = t_j (+) p_k for k ascending over segment j,
 *             p_k = value_k * x_k, exact in fp32;
 *   v_j     = t_j (int2) | fl32(s[n][j]) (*) t_j (int4) | t_j (*) 2^(E-127)
 *             (MXFP4);
 *   tree    : pad v to P2 = next power of two >= n_seg with +0, then for
 *             s = P2/2, ..., 1: v_p = v_p (+) v_{p+s} for every p < s;
 *   y       = fl32(s[n]) (*) v_0 (int2) | v_0 (int4, MXFP4).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* binary16 / bfloat16 <-> binary32, IEEE round-to-nearest-even.             */
/* ------------------------------------------------------------------------ */

ORC_API float orc_f16_to_f32(uint16_t h)
{
    unsigned s = (h >> 15) & 1u, e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? (double)NAN : (double)INFINITY;
    else
        v = ldexp((double)(m | 0x400u), (int)e - 25); /* (1024+m) * 2^(e-25) */
    return (float)(s ? -v : v);
}

ORC_API float orc_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;                /* bf16 = top half of f32 */
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round a double to a binary format with `p` significand bits (incl. the
 * hidden one), minimum normal exponent `emin`, maximum finite value given by
 * `emax`; returns the rounded value as a double (or +-inf).  Plain RNE via
 * nearbyint() in the default rounding mode. */
static double round_to_format(double v, int p, int emin, int emax)
{
    if (isnan(v) || isinf(v) || v == 0.0) return v;
    double a = fabs(v);
    int E;
    frexp(a, &E);                       /* a = f * 2^E, f in [0.5, 1) */
    int e = E - 1;                      /* a in [2^e, 2^(e+1)) */
    if (e < emin) e = emin;             /* subnormal range: fixed quantum */
    double q = ldexp(a, (p - 1) - e);   /* a / quantum, quantum = 2^(e-p+1) */
    double r = nearbyint(q);            /* ties to even */
    double out = ldexp(r, e - (p - 1));
    double maxfin = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
    if (out > maxfin) out = INFINITY;
    return v < 0 ? -out : out;
}

static uint16_t encode_small_float(double r, int p, int emin, int ebias, int ebits)
{
    /* r is already exactly representable (or inf/nan) in the target format */
    unsigned mbits = (unsigned)(p - 1);
    unsigned sign = signbit(r) ? 1u : 0u;
    unsigned expall = (1u << ebits) - 1u;
    unsigned bits;
    if (isnan(r)) {
        bits = (expall << mbits) | (1u << (mbits - 1));
    } else if (isinf(r)) {
        bits = expall << mbits;
    } else if (r == 0.0) {
        bits = 0;
    } else {
        double a = fabs(r);
        int E;
        frexp(a, &E);
        int e = E - 1;
        if (e < emin) { /* subnormal */
            bits = (unsigned)ldexp(a, (int)mbits - emin);
        } else {
            unsigned frac = (unsigned)(ldexp(a, (int)mbits - e) - ldexp(1.0, (int)mbits));
            bits = ((unsigned)(e + ebias) << mbits) | frac;
        }
    }
    return (uint16_t)((sign << (mbits + (unsigned)ebits)) | bits);
}

ORC_API uint16_t orc_f64_to_f16(double v)
{
    return encode_small_float(round_to_format(v, 11, -14, 15), 11, -14, 15, 5);
}

ORC_API uint16_t orc_f32_to_f16(float f) { return orc_f64_to_f16((double)f); }

ORC_API uint16_t orc_f64_to_bf16(double v)
{
    return encode_small_float(round_to_format(v, 8, -126, 127), 8, -126, 127, 8);
}

ORC_API uint16_t orc_f32_to_bf16(float f) { return orc_f64_to_bf16((double)f); }

/* ------------------------------------------------------------------------ */
/* Weight formats.                                                           */
/* ------------------------------------------------------------------------ */

/* int2: the 2-bit field read as a two's-complement integer (field 2 = -2,
 * field 3 = -1), so the values are {-2,-1,0,1}.  Code k = 16w + i of a row is
 * field i (bits 2i+1..2i) of word w; byte j of a word therefore holds the four
 * codes 4j..4j+3 of that word, low bits first. */
static const int INT2_VALUE[4] = {0, 1, -2, -1};

ORC_API int orc_int2_value(unsigned field) { return INT2_VALUE[field & 3u]; }

/* Byte -> 4 values through a 256-entry table composed from INT2_VALUE. */
static int8_t INT2_BYTE_LUT[256][4];
static int int2_lut_ready = 0;

ORC_API void orc_int2_decode_byte_lut(uint8_t b, int8_t out[4])
{
    if (!int2_lut_ready) {
        for (int v = 0; v < 256; ++v)
            for (int t = 0; t < 4; ++t)
                INT2_BYTE_LUT[v][t] = (int8_t)INT2_VALUE[(v >> (2 * t)) & 3];
        int2_lut_ready = 1;
    }
    memcpy(out, INT2_BYTE_LUT[b], 4);
}

/* Byte -> 4 values arithmetically: move the field to the top of a signed
 * byte and shift back (sign extension of a 2-bit two's-complement field). */
ORC_API void orc_int2_decode_byte_arith(uint8_t b, int8_t out[4])
{
    for (int t = 0; t < 4; ++t) {
        int8_t top = (int8_t)(uint8_t)(b << (6 - 2 * t));
        out[t] = (int8_t)(top >> 6);
    }
}

/* int4 symmetric: value = q - 8, q the 4-bit field; code k = 8w + i is field i
 * (bits 4i+3..4i) of word w.  Group scale s[n][k/32] (fp16). */
ORC_API int orc_int4_value(unsigned q) { return (int)(q & 15u) - 8; }

ORC_API void orc_int4_decode_byte_arith(uint8_t b, int8_t out[2])
{
    out[0] = (int8_t)((b & 15) - 8);
    out[1] = (int8_t)((b >> 4) - 8);
}

/* E2M1 (OCP MX v1.0): bit 3 sign, bits 2..1 exponent (bias 1), bit 0
 * mantissa.  Written out as the table of the eight magnitudes. */
static const float E2M1_MAG[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

ORC_API float orc_e2m1_value(unsigned nib)
{
    float m = E2M1_MAG[nib & 7u];
    return (nib & 8u) ? -m : m;
}

/* Ternary ([PB] next-target ranking table, BitCPM ternary row: ternary
 * unpack in the same family as the int2 byte decode).  Five base-3 digits per
 * byte: b = t0 + 3 t1 + 9 t2 + 27 t3 + 81 t4, t_i in {0,1,2}, weight value
 * t_i - 1.  Digit i is floor(b / 3^i) mod 3.  Bytes 243..255 are not codes. */
ORC_API int orc_ternary_value(unsigned b, int i)
{
    unsigned d = b & 255u;
    for (int s = 0; s < i; ++s) d /= 3u;
    return (int)(d % 3u) - 1;
}

/* Pack values v[N][K] in {-1,0,1} into rows of ceil(K/80) 16-byte segments:
 * element k is digit k mod 5 of byte k/5; digits past K are 1 (value 0). */
ORC_API void orc_pack_ternary(const int8_t *v, int64_t N, int64_t K, uint8_t *wq)
{
    int64_t rb = (K + 79) / 80 * 16;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t c = 0; c < rb; ++c) {
            unsigned b = 0, p = 1;
            for (int i = 0; i < 5; ++i, p *= 3u) {
                int64_t k = 5 * c + i;
                int t = k < K ? v[n * K + k] + 1 : 1;
                b += (unsigned)t * p;
            }
            wq[n * rb + c] = (uint8_t)b;
        }
}

/* E8M0 scale: 2^(E-127); E = 255 encodes NaN. */
ORC_API float orc_e8m0_value(uint8_t e)
{
    if (e == 255) return NAN;
    return ldexpf(1.0f, (int)e - 127);
}

/* Packing (used by tests to build inputs and for the round-trip pin). */
ORC_API void orc_pack_int2(const int8_t *vals, int64_t N, int64_t K, uint32_t *wq)
{
    int64_t W = K / 16;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t w = 0; w < W; ++w) {
            uint32_t word = 0;
            for (int i = 0; i < 16; ++i) {
                int v = vals[n * K + w * 16 + i];
                uint32_t field = (uint32_t)v & 3u; /* two's complement, 2 bits */
                word |= field << (2 * i);
            }
            wq[n * W + w] = word;
        }
}

ORC_API void orc_unpack_int2(const uint32_t *wq, int64_t N, int64_t K, int8_t *vals)
{
    int64_t W = K / 16;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            vals[n * K + k] = (int8_t)orc_int2_value(wq[n * W + k / 16] >> (2 * (k % 16)));
}

ORC_API void orc_pack_int4(const uint8_t *q, int64_t N, int64_t K, uint32_t *wq)
{
    int64_t W = K / 8;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t w = 0; w < W; ++w) {
            uint32_t word = 0;
            for (int i = 0; i < 8; ++i) word |= ((uint32_t)q[n * K + w * 8 + i] & 15u) << (4 * i);
            wq[n * W + w] = word;
        }
}

ORC_API void orc_unpack_int4(const uint32_t *wq, int64_t N, int64_t K, uint8_t *q)
{
    int64_t W = K / 8;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) q[n * K + k] = (uint8_t)((wq[n * W + k / 8] >> (4 * (k % 8))) & 15u);
}

/* MXFP4 elements: k = 2j in the low nibble of byte j, k = 2j+1 in the high. */
ORC_API void orc_pack_e2m1(const uint8_t *nib, int64_t N, int64_t K, uint8_t *wq)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 2; ++j)
            wq[n * (K / 2) + j] =
                (uint8_t)((nib[n * K + 2 * j] & 15u) | ((nib[n * K + 2 * j + 1] & 15u) << 4));
}

ORC_API void orc_unpack_e2m1(const uint8_t *wq, int64_t N, int64_t K, uint8_t *nib)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            uint8_t b = wq[n * (K / 2) + k / 2];
            nib[n * K + k] = (uint8_t)((k % 2 == 0) ? (b & 15u) : (b >> 4));
        }
}

/* ------------------------------------------------------------------------ */
/* Fixed-order pieces.                                                       */
/* ------------------------------------------------------------------------ */

/* Halving tree over v[0..nseg-1], padded with +0 up to a power of two.
 * v must have room for that power of two. */
static float fo_tree(float *v, int nseg)
{
    int p2 = 1;
    while (p2 < nseg) p2 <<= 1;
    for (int j = nseg; j < p2; ++j) v[j] = 0.0f;
    for (int s = p2 / 2; s >= 1; s /= 2)
        for (int p = 0; p < s; ++p) v[p] = v[p] + v[p + s];
    return v[0];
}

static int pow2_at_least(int n)
{
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

/* One output of the int2 FO matvec: row n against the fp32 copy xf[K]. */
static float fo_int2_row(const uint32_t *row, float scale, const float *xf, int64_t K, float *v)
{
    int nseg = (int)(K / 64);
    for (int j = 0; j < nseg; ++j) {
        float t = 0.0f;
        for (int64_t k = 64 * (int64_t)j; k < 64 * (int64_t)j + 64; ++k) {
            float c = (float)orc_int2_value(row[k / 16] >> (2 * (k % 16)));
            float p = c * xf[k]; /* exact */
            t = t + p;
        }
        v[j] = t;
    }
    float total = fo_tree(v, nseg);
    return scale * total;
}

static float fo_int4_row(const uint32_t *row, const uint16_t *srow, const float *xf, int64_t K, float *v)
{
    int nseg = (int)(K / 32);
    for (int j = 0; j < nseg; ++j) {
        float t = 0.0f;
        for (int64_t k = 32 * (int64_t)j; k < 32 * (int64_t)j + 32; ++k) {
            float c = (float)orc_int4_value(row[k / 8] >> (4 * (k % 8)));
            float p = c * xf[k]; /* exact */
            t = t + p;
        }
        v[j] = orc_f16_to_f32(srow[j]) * t;
    }
    return fo_tree(v, nseg);
}

static float fo_mxfp4_row(const uint8_t *row, const uint8_t *erow, const float *xf, int64_t K, float *v)
{
    int nseg = (int)(K / 32);
    for (int j = 0; j < nseg; ++j) {
        float t = 0.0f;
        for (int64_t k = 32 * (int64_t)j; k < 32 * (int64_t)j + 32; ++k) {
            uint8_t b = row[k / 2];
            float c = orc_e2m1_value((k % 2 == 0) ? (b & 15u) : (b >> 4));
            float p = c * xf[k]; /* exact */
            t = t + p;
        }
        v[j] = t * orc_e8m0_value(erow[j]);
    }
    return fo_tree(v, nseg);
}

/* Ternary: a row is ceil(K/80) 16-byte segments of 80 codes; only codes
 * k < K are summed (the last segment may hold fewer); fp16 row scale at the
 * end, as for int2. */
static float fo_ternary_row(const uint8_t *row, float scale, const float *xf, int64_t K, float *v)
{
    int nseg = (int)((K + 79) / 80);
    for (int j = 0; j < nseg; ++j) {
        float t = 0.0f;
        int64_t end = 80 * (int64_t)j + 80 < K ? 80 * (int64_t)j + 80 : K;
        for (int64_t k = 80 * (int64_t)j; k < end; ++k) {
            float c = (float)orc_ternary_value(row[k / 5], (int)(k % 5));
            float p = c * xf[k]; /* exact */
            t = t + p;
        }
        v[j] = t;
    }
    float total = fo_tree(v, nseg);
    return scale * total;
}

/* ------------------------------------------------------------------------ */
/* Row-parallel driver (rows are independent; the thread count never changes */
/* any bit of the result).                                                   */
/* ------------------------------------------------------------------------ */

typedef void (*row_fn)(void *ctx, int64_t n0, int64_t n1);
typedef struct { row_fn fn; void *ctx; int64_t n0, n1; } chunk_t;

static void *chunk_main(void *arg)
{
    chunk_t *c = (chunk_t *)arg;
    c->fn(c->ctx, c->n0, c->n1);
    return NULL;
}

static void parallel_rows(row_fn fn, void *ctx, int64_t N, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > N) nthreads = (int)(N > 0 ? N : 1);
    if (nthreads == 1) { fn(ctx, 0, N); return; }
    pthread_t th[256];
    chunk_t ch[256];
    for (int t = 0; t < nthreads; ++t) {
        ch[t].fn = fn; ch[t].ctx = ctx;
        ch[t].n0 = N * t / nthreads; ch[t].n1 = N * (t + 1) / nthreads;
        pthread_create(&th[t], NULL, chunk_main, &ch[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

typedef struct {
    const void *wq; const void *sc; const float *xf; float *y;
    int64_t M, N, K;
} mv_ctx;

static void int2_rows(void *p, int64_t n0, int64_t n1)
{
    mv_ctx *c = (mv_ctx *)p;
    float *v = (float *)malloc(sizeof(float) * (size_t)pow2_at_least((int)(c->K / 64)));
    const uint32_t *wq = (const uint32_t *)c->wq;
    const uint16_t *s = (const uint16_t *)c->sc;
    for (int64_t n = n0; n < n1; ++n)
        for (int64_t m = 0; m < c->M; ++m)
            c->y[m * c->N + n] = fo_int2_row(wq + n * (c->K / 16), orc_f16_to_f32(s[n]),
                                             c->xf + m * c->K, c->K, v);
    free(v);
}

static void int4_rows(void *p, int64_t n0, int64_t n1)
{
    mv_ctx *c = (mv_ctx *)p;
    float *v = (float *)malloc(sizeof(float) * (size_t)pow2_at_least((int)(c->K / 32)));
    const uint32_t *wq = (const uint32_t *)c->wq;
    const uint16_t *s = (const uint16_t *)c->sc;
    for (int64_t n = n0; n < n1; ++n)
        for (int64_t m = 0; m < c->M; ++m)
            c->y[m * c->N + n] = fo_int4_row(wq + n * (c->K / 8), s + n * (c->K / 32),
                                             c->xf + m * c->K, c->K, v);
    free(v);
}

static void mxfp4_rows(void *p, int64_t n0, int64_t n1)
{
    mv_ctx *c = (mv_ctx *)p;
    float *v = (float *)malloc(sizeof(float) * (size_t)pow2_at_least((int)(c->K / 32)));
    const uint8_t *wq = (const uint8_t *)c->wq;
    const uint8_t *e = (const uint8_t *)c->sc;
    for (int64_t n = n0; n < n1; ++n)
        for (int64_t m = 0; m < c->M; ++m)
            c->y[m * c->N + n] = fo_mxfp4_row(wq + n * (c->K / 2), e + n * (c->K / 32),
                                              c->xf + m * c->K, c->K, v);
    free(v);
}

static void ternary_rows(void *p, int64_t n0, int64_t n1)
{
    mv_ctx *c = (mv_ctx *)p;
    int64_t nseg = (c->K + 79) / 80;
    float *v = (float *)malloc(sizeof(float) * (size_t)pow2_at_least((int)nseg));
    const uint8_t *wq = (const uint8_t *)c->wq;
    const uint16_t *s = (const uint16_t *)c->sc;
    for (int64_t n = n0; n < n1; ++n)
        for (int64_t m = 0; m < c->M; ++m)
            c->y[m * c->N + n] = fo_ternary_row(wq + n * nseg * 16, orc_f16_to_f32(s[n]),
                                                c->xf + m * c->K, c->K, v);
    free(v);
}

static float *widen_f16(const uint16_t *x, int64_t cnt)
{
    float *xf = (float *)malloc(sizeof(float) * (size_t)(cnt > 0 ? cnt : 1));
    for (int64_t i = 0; i < cnt; ++i) xf[i] = orc_f16_to_f32(x[i]);
    return xf;
}

static float *widen_bf16(const uint16_t *x, int64_t cnt)
{
    float *xf = (float *)malloc(sizeof(float) * (size_t)(cnt > 0 ? cnt : 1));
    for (int64_t i = 0; i < cnt; ++i) xf[i] = orc_bf16_to_f32(x[i]);
    return xf;
}

/* y[M][N] (fp32) = FO int2 matvec.  wq [N][K/16], scale fp16 [N], x fp16 [M][K]. */
ORC_API void orc_qmv_int2(const uint32_t *wq, const uint16_t *scale, const uint16_t *x, float *y,
                          int64_t M, int64_t N, int64_t K, int nthreads)
{
    float *xf = widen_f16(x, M * K);
    mv_ctx c = {wq, scale, xf, y, M, N, K};
    parallel_rows(int2_rows, &c, N, nthreads);
    free(xf);
}

/* int4: wq [N][K/8], scales fp16 [N][K/32], x fp16 [M][K]. */
ORC_API void orc_qmv_int4(const uint32_t *wq, const uint16_t *scales, const uint16_t *x, float *y,
                          int64_t M, int64_t N, int64_t K, int nthreads)
{
    float *xf = widen_f16(x, M * K);
    mv_ctx c = {wq, scales, xf, y, M, N, K};
    parallel_rows(int4_rows, &c, N, nthreads);
    free(xf);
}

/* MXFP4: wq uint8 [N][K/2], e8m0 uint8 [N][K/32], x bf16 [M][K]. */
ORC_API void orc_qmm_mxfp4(const uint8_t *wq, const uint8_t *e8m0, const uint16_t *x, float *y,
                           int64_t M, int64_t N, int64_t K, int nthreads)
{
    float *xf = widen_bf16(x, M * K);
    mv_ctx c = {wq, e8m0, xf, y, M, N, K};
    parallel_rows(mxfp4_rows, &c, N, nthreads);
    free(xf);
}

/* Ternary: wq uint8 [N][ceil(K/80)*16], scale fp16 [N], x fp16 [M][K]. */
ORC_API void orc_qmv_ternary(const uint8_t *wq, const uint16_t *scale, const uint16_t *x, float *y,
                             int64_t M, int64_t N, int64_t K, int nthreads)
{
    float *xf = widen_f16(x, M * K);
    mv_ctx c = {wq, scale, xf, y, M, N, K};
    parallel_rows(ternary_rows, &c, N, nthreads);
    free(xf);
}

/* Expert-gather MXFP4 matvec ([PB], next-target ranking table, the gpt-oss MoE
 * row: close the gather_qmm frontier with a zero-materialisation expert-gather
 * matvec).  E experts' weights wq [E][N][K/2], e8m0 [E][N][K/32]; for activation
 * row m and slot j the expert e = idx[m][j] selects its weights in place (no
 * gathered copy) and y[m][j][N] = the FO MXFP4 matvec of expert e with x[m].
 * Every idx entry must lie in [0, E). */
ORC_API void orc_qmm_mxfp4_gather(const uint8_t *wq, const uint8_t *e8m0, const uint16_t *x,
                                  const int32_t *idx, float *y, int64_t E, int64_t topk, int64_t M,
                                  int64_t N, int64_t K, int nthreads)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t j = 0; j < topk; ++j) {
            const int64_t e = idx[m * topk + j];
            if (e < 0 || e >= E) abort();
            orc_qmm_mxfp4(wq + e * N * (K / 2), e8m0 + e * N * (K / 32), x + m * K,
                          y + (m * topk + j) * N, 1, N, K, nthreads);
        }
}

/* ------------------------------------------------------------------------ */
/* Exponential and GELU (tanh form) -- the library's own sequence.           */
/* ------------------------------------------------------------------------ */

/* e^z for z in [-87, 87]: Cody & Waite range reduction z = n ln2 + r with
 * ln2 split into a 15-significant-bit head (so n * head is exact for
 * |n| <= 127) and a tail, then the degree-7 Taylor polynomial of e^r with
 * coefficients 1/j! rounded to binary32, evaluated by Horner with fused
 * multiply-adds, then scaled by 2^n built from its exponent bits. */
#define ORC_LOG2E 0x1.715476p+0f
#define ORC_LN2_HI 0x1.62e4p-1f
#define ORC_LN2_LO 0x1.7f7d1cp-20f

ORC_API float orc_exp(float z)
{
    static const float C[8] = {0x1p+0f, 0x1p+0f, 0x1p-1f, 0x1.555556p-3f,
                               0x1.555556p-5f, 0x1.111112p-7f, 0x1.6c16c2p-10f, 0x1.a01a02p-13f};
    float t = z * ORC_LOG2E;
    float n = rintf(t);
    float r = fmaf(-n, ORC_LN2_HI, z);
    r = fmaf(-n, ORC_LN2_LO, r);
    float p = C[7];
    for (int j = 6; j >= 0; --j) p = fmaf(p, r, C[j]);
    int ni = (int)n;
    uint32_t bits = (uint32_t)(ni + 127) << 23;
    float two_n;
    memcpy(&two_n, &bits, 4);
    return p * two_n;
}

/* Build guard (no part of the method): a * b + c with the product and the
 * sum rounded separately, written as every unfused step of this file is.  A
 * build that contracts it into one fused multiply-add (for example
 * -ffp-contract=fast with FMA instructions available) rounds once instead;
 * the pins call it where the two differ, so such a build is rejected even
 * where no method output happens to change. */
ORC_API float orc_probe_mul_add(float a, float b, float c)
{
    float p = a * b;
    return p + c;
}

#define ORC_SQRT_2_OVER_PI 0x1.988454p-1f
#define ORC_GELU_C 0x1.6e4e26p-5f /* 0.044715 */

/* GELU, tanh form, through the identity (1 + tanh u)/2 = 1/(1 + e^(-2u)). */
ORC_API float orc_gelu(float g)
{
    float g2 = g * g;
    float g3 = g2 * g;
    float cg3 = ORC_GELU_C * g3;
    float inner = g + cg3;
    float u = ORC_SQRT_2_OVER_PI * inner;
    float z = -2.0f * u;
    if (z > 87.0f) z = 87.0f;
    if (z < -87.0f) z = -87.0f;
    float e = orc_exp(z);
    float den = 1.0f + e;
    return g / den;
}

/* ------------------------------------------------------------------------ */
/* Residual-add + RMSNorm prologue (folded into the next matvec, [A19]).     */
/* ------------------------------------------------------------------------ */

/* For one activation row: h = fl16(x + r) (single rounding; the exact sum is
 * formed in double), ss = sum of exact squares fl32(h)^2 in the FO shape with
 * 64-element segments, inv = 1 / sqrt(ss / K + eps) (correctly rounded
 * division and square root), xn = fl16((fl32(h) * inv) * fl32(gamma)).
 * Writes h (fp16) and xn (fp16); returns inv. */
ORC_API float orc_rmsnorm_prologue(const uint16_t *x, const uint16_t *r, const uint16_t *gamma,
                                   float eps, int64_t K, uint16_t *h_out, uint16_t *xn_out)
{
    int nseg = (int)(K / 64);
    float *v = (float *)malloc(sizeof(float) * (size_t)pow2_at_least(nseg));
    for (int64_t k = 0; k < K; ++k)
        h_out[k] = orc_f64_to_f16((double)orc_f16_to_f32(x[k]) + (double)orc_f16_to_f32(r[k]));
    for (int j = 0; j < nseg; ++j) {
        float t = 0.0f;
        for (int64_t k = 64 * (int64_t)j; k < 64 * (int64_t)j + 64; ++k) {
            float hf = orc_f16_to_f32(h_out[k]);
            float sq = hf * hf; /* exact */
            t = t + sq;
        }
        v[j] = t;
    }
    float ss = fo_tree(v, nseg);
    free(v);
    float ms = ss / (float)K;
    float rr = ms + eps;
    float root = sqrtf(rr);
    float inv = 1.0f / root;
    for (int64_t k = 0; k < K; ++k) {
        float a = orc_f16_to_f32(h_out[k]) * inv;
        float b = a * orc_f16_to_f32(gamma[k]);
        xn_out[k] = orc_f32_to_f16(b);
    }
    return inv;
}

/* Fused: residual add + RMSNorm prologue, dual int2 FO matvec (gate, up) on
 * the normalised activations, out = fl16(GELU(gate) * up).
 * x, residual: fp16 [M][K]; gamma fp16 [K]; residual_out fp16 [M][K] or NULL;
 * wq_gate/wq_up [N][K/16]; s_gate/s_up fp16 [N]; out fp16 [M][N].
 * gate_out/up_out (fp32 [M][N], may be NULL) expose the intermediate logits. */
ORC_API void orc_int2_rmsnorm_gateup_gelu(const uint16_t *x, const uint16_t *residual,
                                          uint16_t *residual_out, const uint16_t *gamma, float eps,
                                          const uint32_t *wq_gate, const uint16_t *s_gate,
                                          const uint32_t *wq_up, const uint16_t *s_up,
                                          uint16_t *out, float *gate_out, float *up_out,
                                          int64_t M, int64_t N, int64_t K, int nthreads)
{
    uint16_t *h = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(M * K));
    uint16_t *xn = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(M * K));
    float *g = (float *)malloc(sizeof(float) * (size_t)(M * N));
    float *u = (float *)malloc(sizeof(float) * (size_t)(M * N));
    for (int64_t m = 0; m < M; ++m)
        orc_rmsnorm_prologue(x + m * K, residual + m * K, gamma, eps, K, h + m * K, xn + m * K);
    orc_qmv_int2(wq_gate, s_gate, xn, g, M, N, K, nthreads);
    orc_qmv_int2(wq_up, s_up, xn, u, M, N, K, nthreads);
    for (int64_t i = 0; i < M * N; ++i) {
        float ge = orc_gelu(g[i]);
        float o = ge * u[i];
        out[i] = orc_f32_to_f16(o);
    }
    if (residual_out) memcpy(residual_out, h, sizeof(uint16_t) * (size_t)(M * K));
    if (gate_out) memcpy(gate_out, g, sizeof(float) * (size_t)(M * N));
    if (up_out) memcpy(up_out, u, sizeof(float) * (size_t)(M * N));
    free(h); free(xn); free(g); free(u);
}

/* MXFP4 quantisation of one 32-value block (OCP Microscaling Formats v1.0,
 * conversion to an MX format): the shared exponent is floor(log2(max |v|))
 * minus 2, the exponent of E2M1's largest value; the E8M0 byte is that plus
 * 127; each element is v / 2^shared rounded to the nearest E2M1 value, ties
 * to the even code (mantissa bit 0), which also clamps everything from 5 up
 * to 6.  The sign bit is v's (a value rounding to zero keeps it).  An
 * all-zero block takes the E8M0 byte 0.  Inputs are fp16, finite.  Code k
 * goes to the low nibble of byte k/2 for even k, the high nibble for odd k. */
ORC_API void orc_quant_mxfp4_block(const uint16_t *v, uint8_t *codes, uint8_t *e8m0)
{
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) {
        double a = fabs((double)orc_f16_to_f32(v[i]));
        if (a > amax) amax = a;
    }
    int shared = -127;
    if (amax > 0.0) {
        int ex;
        frexp(amax, &ex);   /* amax = f * 2^ex, f in [0.5, 1): floor(log2) = ex - 1 */
        shared = ex - 1 - 2;
    }
    *e8m0 = (uint8_t)(shared + 127);
    for (int i = 0; i < 32; i += 2) codes[i / 2] = 0;
    for (int i = 0; i < 32; ++i) {
        double x = (double)orc_f16_to_f32(v[i]);
        double mag = ldexp(fabs(x), -shared); /* exact */
        int best = 0;
        for (int c = 1; c < 8; ++c) {
            double dc = fabs(mag - (double)E2M1_MAG[c]), db = fabs(mag - (double)E2M1_MAG[best]);
            if (dc < db || (dc == db && (c % 2) == 0)) best = c;
        }
        unsigned code = (unsigned)best | (signbit(x) ? 8u : 0u);
        codes[i / 2] |= (uint8_t)(i % 2 == 0 ? code : code << 4);
    }
}

/* Fused activation-and-quantize ("Gemma 4 Optimization with Agentic Kernel
 * Engineering", "What it found": a fused activation-and-quantize kernel on
 * MI355X): the fused gate/up output out = fp16(GELU(gate) * up) of
 * orc_int2_rmsnorm_gateup_gelu, then each row's 32-value blocks quantised
 * to MXFP4 for the next MXFP4 GEMM.  codes uint8 [M][N/2], e8m0 uint8
 * [M][N/32]; N a multiple of 32. */
ORC_API void orc_int2_rmsnorm_gateup_gelu_mxfp4(const uint16_t *x, const uint16_t *residual,
                                                uint16_t *residual_out, const uint16_t *gamma, float eps,
                                                const uint32_t *wq_gate, const uint16_t *s_gate,
                                                const uint32_t *wq_up, const uint16_t *s_up,
                                                uint8_t *codes, uint8_t *e8m0,
                                                int64_t M, int64_t N, int64_t K, int nthreads)
{
    uint16_t *out = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(M * N));
    orc_int2_rmsnorm_gateup_gelu(x, residual, residual_out, gamma, eps, wq_gate, s_gate, wq_up, s_up,
                                 out, NULL, NULL, M, N, K, nthreads);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t b = 0; b < N / 32; ++b)
            orc_quant_mxfp4_block(out + m * N + 32 * b, codes + m * (N / 2) + 16 * b, e8m0 + m * (N / 32) + b);
    free(out);
}

/* Shared-prologue q/k/v ([A19] "What moved the needle", dispatch-count
 * fusion: the residual-add RMSNorm folded into the next matvec's prologue,
 * and q/k/v in a single dispatch): the prologue above on each activation
 * row, then three independent int2 FO matvecs on the normalised row.
 * x, residual: fp16 [M][K]; gamma fp16 [K]; residual_out fp16 [M][K] or NULL;
 * wq_z [N_z][K/16], s_z fp16 [N_z]; y_z fp32 [M][N_z] for z = q, k, v. */
ORC_API void orc_int2_rmsnorm_qkv(const uint16_t *x, const uint16_t *residual, uint16_t *residual_out,
                                  const uint16_t *gamma, float eps,
                                  const uint32_t *wq_q, const uint16_t *s_q, int64_t Nq,
                                  const uint32_t *wq_k, const uint16_t *s_k, int64_t Nk,
                                  const uint32_t *wq_v, const uint16_t *s_v, int64_t Nv,
                                  float *yq, float *yk, float *yv, int64_t M, int64_t K, int nthreads)
{
    uint16_t *h = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(M * K));
    uint16_t *xn = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(M * K));
    for (int64_t m = 0; m < M; ++m)
        orc_rmsnorm_prologue(x + m * K, residual + m * K, gamma, eps, K, h + m * K, xn + m * K);
    orc_qmv_int2(wq_q, s_q, xn, yq, M, Nq, K, nthreads);
    orc_qmv_int2(wq_k, s_k, xn, yk, M, Nk, K, nthreads);
    orc_qmv_int2(wq_v, s_v, xn, yv, M, Nv, K, nthreads);
    if (residual_out) memcpy(residual_out, h, sizeof(uint16_t) * (size_t)(M * K));
    free(h); free(xn);
}

/* ------------------------------------------------------------------------ */
/* lm_head: int2 FO logits + argmax, first maximum wins ([A19] parked levers) */
/* ------------------------------------------------------------------------ */

ORC_API void orc_int2_argmax(const uint32_t *wq, const uint16_t *scale, const uint16_t *x,
                             int32_t *idx, float *maxval, float *logits,
                             int64_t M, int64_t N, int64_t K, int nthreads)
{
    float *y = (float *)malloc(sizeof(float) * (size_t)(M * N));
    orc_qmv_int2(wq, scale, x, y, M, N, K, nthreads);
    for (int64_t m = 0; m < M; ++m) {
        int64_t best = 0;
        for (int64_t n = 1; n < N; ++n)
            if (y[m * N + n] > y[m * N + best]) best = n; /* strict: first max kept; -0 == +0 */
        idx[m] = (int32_t)best;
        if (maxval) maxval[m] = y[m * N + best];
    }
    if (logits) memcpy(logits, y, sizeof(float) * (size_t)(M * N));
    free(y);
}

/* ------------------------------------------------------------------------ */
/* Binary64 references: dequantize, then an ordinary dot product in double.  */
/* Used only to bound the FO results (Higham) in the self-tests.             */
/* ------------------------------------------------------------------------ */

ORC_API void orc_ref64_int2(const uint32_t *wq, const uint16_t *scale, const uint16_t *x, double *y,
                            double *absy, int64_t M, int64_t N, int64_t K)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double w = (double)orc_int2_value(wq[n * (K / 16) + k / 16] >> (2 * (k % 16)));
                double xv = (double)orc_f16_to_f32(x[m * K + k]);
                acc += w * xv;
                aacc += fabs(w * xv);
            }
            double s = (double)orc_f16_to_f32(scale[n]);
            y[m * N + n] = s * acc;
            if (absy) absy[m * N + n] = fabs(s) * aacc;
        }
}

ORC_API void orc_ref64_int4(const uint32_t *wq, const uint16_t *scales, const uint16_t *x, double *y,
                            double *absy, int64_t M, int64_t N, int64_t K)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double w = (double)orc_int4_value(wq[n * (K / 8) + k / 8] >> (4 * (k % 8)));
                w *= (double)orc_f16_to_f32(scales[n * (K / 32) + k / 32]);
                double xv = (double)orc_f16_to_f32(x[m * K + k]);
                acc += w * xv;
                aacc += fabs(w * xv);
            }
            y[m * N + n] = acc;
            if (absy) absy[m * N + n] = aacc;
        }
}

ORC_API void orc_ref64_mxfp4(const uint8_t *wq, const uint8_t *e8m0, const uint16_t *x, double *y,
                             double *absy, int64_t M, int64_t N, int64_t K)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                uint8_t b = wq[n * (K / 2) + k / 2];
                double w = (double)orc_e2m1_value((k % 2 == 0) ? (b & 15u) : (b >> 4));
                w *= (double)orc_e8m0_value(e8m0[n * (K / 32) + k / 32]);
                double xv = (double)orc_bf16_to_f32(x[m * K + k]);
                acc += w * xv;
                aacc += fabs(w * xv);
            }
            y[m * N + n] = acc;
            if (absy) absy[m * N + n] = aacc;
        }
}
