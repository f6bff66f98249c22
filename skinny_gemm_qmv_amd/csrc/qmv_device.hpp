// qmv_device.hpp -- device helpers for the gfx950 quantized matvec kernels:
// weight decode, the fixed-order (FO) tree, conversions, exp and GELU.
//
// Definitions implemented here (cited by page title and section):
//  * "Gemma4 raw-Metal loop on A19 -- findings + the remaining (parked)
//    levers", "What moved the needle": int2 codes, 16 per 32-bit word, four
//    per byte; products x*c with c in {-2,-1,0,1} are exact; fp32
//    accumulation in code order; the strided merge order is fixed by the
//    tile and must not change with it.
//  * OCP Microscaling Formats v1.0: E2M1 elements, E8M0 block scale.
//
// Arithmetic contract (shared with the C header, written independently of
// any reference implementation): every fp32 operation is one IEEE binary32
// round-to-nearest-even operation, nothing is contracted unless written as an
// explicit fma, denormals are preserved (the default gfx950 float mode).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmv {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef float f2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u3_t __attribute__((ext_vector_type(3)));

enum Fmt : int { FMT_INT2 = 0, FMT_INT4 = 1, FMT_MXFP4 = 2, FMT_TERN = 3 };

// Codes held by one 16-byte segment (one dwordx4 load) of a packed row.
template <int F> struct SegCodes;
template <> struct SegCodes<FMT_INT2> { static constexpr int v = 64; };
template <> struct SegCodes<FMT_INT4> { static constexpr int v = 32; };
template <> struct SegCodes<FMT_MXFP4> { static constexpr int v = 32; };
template <> struct SegCodes<FMT_TERN> { static constexpr int v = 80; };

// Formats with one fp16 scale per row, applied to the reduced total (int2,
// ternary); the others scale every segment.
template <int F> constexpr bool kRowScale = F == FMT_INT2 || F == FMT_TERN;

__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ h2_t u2h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }
__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return u2f((uint32_t)b << 16); }

// Compile-time loop: f(Index<0>{}) ... f(Index<N-1>{}), always expanded
// (a #pragma unroll may be refused for a large body).
template <int I> struct Index { static constexpr int value = I; };
template <int I, int N, class Fn>
__device__ __forceinline__ void static_for_from(Fn &&f) {
    if constexpr (I < N) {
        f(Index<I>{});
        static_for_from<I + 1, N>(f);
    }
}
template <int N, class Fn>
__device__ __forceinline__ void static_for(Fn &&f) {
    static_for_from<0, N>(f);
}

__device__ __forceinline__ h2_t fma_h2(h2_t a, float mul, float add) {
    const h2_t m = {(_Float16)mul, (_Float16)mul};
    const h2_t c = {(_Float16)add, (_Float16)add};
    return __builtin_elementwise_fma(a, m, c);
}

// Hide a value from constant folding (no instruction is emitted).  gfx9 VOP3
// encodings cannot carry literal constants, so the decode masks live in
// SGPRs and the fp16 magic in a VGPR; v_and_or_b32 then does mask-and-insert
// in one instruction.
__device__ __forceinline__ uint32_t in_sgpr(uint32_t v) {
    asm volatile("" : "+s"(v));
    return v;
}
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// fp16 1024.0 in both halves: OR-ing a field into the low mantissa bits of
// this pattern gives the fp16 value 1024 + field * 2^(bit position).
constexpr uint32_t kMagic1024 = 0x64006400u;

struct DecodeConsts {
    uint32_t magic;                // VGPR
    uint32_t m4lo, m4hi;           // int4 masks
    uint32_t m8;                   // ternary byte-pair mask
    uint32_t t2, m03;              // int2 byte table (fp16 high bytes of 0, 1, -2, -1), byte-field mask
    __device__ __forceinline__ DecodeConsts() {
        magic = in_vgpr(kMagic1024);
        m4lo = in_sgpr(0x000F000Fu);
        m4hi = in_sgpr(0x00F000F0u);
        m8 = in_sgpr(0x00FF00FFu);
        t2 = in_sgpr(0xBCC03C00u);
        m03 = in_sgpr(0x03030303u);
    }
};

// int2: 16 two's-complement 2-bit fields of one word -> 8 packed fp16 pairs,
// pair i = (code i, code i+8), by a register byte table (the pages' byte ->
// value lookup, done with v_perm_b32): every code value v in {0, 1, -2, -1}
// is an fp16 number whose low byte is 0, so byte f of t2 holds the high
// byte of fp16(value of field f) and one byte select per four fields picks
// them: t = the fields s, s+4, s+8, s+12 one per byte (a shift and a mask),
// p = t2 indexed by t, then two selects place (s, s+8) and (s+4, s+12) as
// fp16 pairs with zero low bytes.  Code 0 gives +0, as the arithmetic
// decode did.  Per word 12 byte selects and 7 shift/mask ops, against 16
// VOP3-class ops for the magic-number decode (1024 + 4^i f in a mantissa,
// then one exact packed fma per pair): 4.8 % less time on the lm_head
// shape, same bits.
__device__ __forceinline__ void int2_decode_word(uint32_t w, const DecodeConsts &k, h2_t (&c)[8]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint32_t t = (s == 0 ? w : w >> (2 * s)) & k.m03;     // fields s, s+4, s+8, s+12
        const uint32_t p = __builtin_amdgcn_perm(k.t2, k.t2, t);     // their fp16 high bytes
        c[s] = u2h2(__builtin_amdgcn_perm(0u, p, 0x020C000Cu));      // (code s, code s+8)
        c[s + 4] = u2h2(__builtin_amdgcn_perm(0u, p, 0x030C010Cu));  // (code s+4, code s+12)
    }
}

// int4: 8 nibbles q of one word -> 4 packed fp16 pairs of q - 8,
// pair i = (code i, code i+4).
__device__ __forceinline__ void int4_decode_word(uint32_t w, const DecodeConsts &k, h2_t (&c)[4]) {
    const uint32_t v = w >> 8;
    c[0] = fma_h2(u2h2((w & k.m4lo) | k.magic), 1.0f, -1032.0f);
    c[1] = fma_h2(u2h2((w & k.m4hi) | k.magic), 0.0625f, -72.0f);
    c[2] = fma_h2(u2h2((v & k.m4lo) | k.magic), 1.0f, -1032.0f);
    c[3] = fma_h2(u2h2((v & k.m4hi) | k.magic), 0.0625f, -72.0f);
}

// E8M0 block scale as an fp32 value: 2^(E-127), exact for E in 0..254
// (E = 0 is the subnormal 2^-127), NaN for E = 255.
// Branch-free: the exponent field is E, and the mantissa bit 22 is set for
// E = 0 (giving 2^-127) and E = 255 (turning +inf into a quiet NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
    const uint32_t special = (e == 0u || e == 255u) ? 0x00400000u : 0u;
    return u2f((e << 23) | special);
}

// Ternary: one word holds four bytes of five base-3 digits each (byte c of
// the word = codes 5c .. 5c+4 of its 20).  Decoded with packed fp16
// arithmetic, two bytes per instruction, every step exact:
//   e = b - 1 from the magic-number placement (1024 + b) - 1025;
//   per digit i: r = round(e / 3) (an fma with fp16(1/3) onto the magic 1536
//   rounds to the nearest integer; e/3 lies within 1/3 + 0.03 of the integer
//   floor(b / 3^(i+1)), so the rounding is never close), the digit value
//   t_i - 1 = e - 3r (exact), then e = r - 1 for the next digit; after four
//   digits e itself is t_4 - 1 (for the 243 valid codes, b < 243).
// c[2i] holds digit i of bytes 0 and 2 (low, high half), c[2i+1] digit i of
// bytes 1 and 3.
__device__ __forceinline__ void tern_decode_word(uint32_t w, const DecodeConsts &k, h2_t (&c)[10]) {
    const h2_t bias = {(_Float16)-1025.0f, (_Float16)-1025.0f};
    const h2_t third = {(_Float16)(1.0f / 3.0f), (_Float16)(1.0f / 3.0f)};
    const h2_t mg = {(_Float16)1536.0f, (_Float16)1536.0f};
    const h2_t m3 = {(_Float16)-3.0f, (_Float16)-3.0f};
    const h2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    h2_t e[2];
    e[0] = u2h2((w & k.m8) | k.magic) + bias;
    e[1] = u2h2(((w >> 8) & k.m8) | k.magic) + bias;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const h2_t r = __builtin_elementwise_fma(e[p], third, mg) - mg;
            c[2 * i + p] = __builtin_elementwise_fma(r, m3, e[p]);
            e[p] = r - one;
        }
    c[8] = e[0];
    c[9] = e[1];
}

// v_fma_mix_f32 with two fp16 sources taken from halves of packed
// registers (AH / BH = 1 selects the high half) and an fp32 addend:
// acc = acc (+) a*b with one rounding.  fp16 x fp16 products are exact in
// fp32, so this is the fixed-order step.  Written as an instruction so that
// the compiler keeps the operands in fp16 (it would otherwise widen a shared
// operand once and hold the fp32 copies in registers).
template <int AH, int BH>
__device__ __forceinline__ void mix_mac(float &acc, uint32_t a2, uint32_t b2) {
    if constexpr (AH == 0 && BH == 0)
        asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel_hi:[1,1,0]" : "+v"(acc) : "v"(a2), "v"(b2));
    else if constexpr (AH == 1 && BH == 0)
        asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel:[1,0,0] op_sel_hi:[1,1,0]" : "+v"(acc) : "v"(a2), "v"(b2));
    else if constexpr (AH == 0 && BH == 1)
        asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel:[0,1,0] op_sel_hi:[1,1,0]" : "+v"(acc) : "v"(a2), "v"(b2));
    else
        asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel:[1,1,0] op_sel_hi:[1,1,0]" : "+v"(acc) : "v"(a2), "v"(b2));
}

// Ternary inner step (80 codes per segment): for k = 0 .. 79 in order,
// t[a][m] = t[a][m] (+) value_k * x[m][k]; the words are decoded as the
// codes reach them and each 16-byte activation vector is fetched once.
template <int NS, int MC, class XF>
__device__ __forceinline__ void tern_sums(const u4_t (&w)[NS], const DecodeConsts &kc, XF &&xf,
                                          float (&t)[NS][MC]) {
    h2_t c[NS][10];
    u4_t xa[NS][MC];
#pragma unroll
    for (int k = 0; k < 80; ++k) {
        if (k % 20 == 0) {
#pragma unroll
            for (int a = 0; a < NS; ++a) tern_decode_word(w[a][k / 20], kc, c[a]);
        }
        if (k % 8 == 0) {
#pragma unroll
            for (int a = 0; a < NS; ++a)
#pragma unroll
                for (int m = 0; m < MC; ++m) xa[a][m] = xf(a, m, k / 8);
        }
        const int byte = (k % 20) / 5, dig = k % 5;
        const int pair = 2 * dig + (byte & 1);
        const bool wh = byte >= 2, xh = k & 1;
#pragma unroll
        for (int a = 0; a < NS; ++a) {
            const uint32_t cp = __builtin_bit_cast(uint32_t, c[a][pair]);
#pragma unroll
            for (int m = 0; m < MC; ++m) {
                const uint32_t xp = xa[a][m][(k & 7) >> 1];
                if (wh) {
                    if (xh) mix_mac<1, 1>(t[a][m], cp, xp);
                    else mix_mac<1, 0>(t[a][m], cp, xp);
                } else {
                    if (xh) mix_mac<0, 1>(t[a][m], cp, xp);
                    else mix_mac<0, 0>(t[a][m], cp, xp);
                }
            }
        }
    }
}

// Inner step for the NS segments a lane holds in one row group, for MC
// activation columns:
//   t[a][m] = t[a][m] (+) value_k * x[m][k]   for k ascending over segment a.
// The NS x MC chains are independent; they are advanced together one code at
// a time so consecutive fused multiply-adds never depend on each other, while
// each chain still adds its products in code order.  XF(a, m, v) returns 8
// consecutive activation values (16 bytes) of column m at offset 8v of the
// lane's segment a.
template <int F, int NS, int MC, class XF>
__device__ __forceinline__ void segment_sums(const u4_t (&w)[NS], const DecodeConsts &kc, XF &&xf,
                                             float (&t)[NS][MC]) {
    if constexpr (F == FMT_TERN) {
        tern_sums<NS, MC>(w, kc, xf, t);
        return;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if constexpr (F == FMT_INT2) {
            h2_t c[NS][8];
#pragma unroll
            for (int a = 0; a < NS; ++a) int2_decode_word(w[a][q], kc, c[a]);
#pragma unroll
            for (int half = 0; half < 2; ++half) {  // codes 16q + 8half .. +7
                u4_t xa[NS][MC];
#pragma unroll
                for (int a = 0; a < NS; ++a)
#pragma unroll
                    for (int m = 0; m < MC; ++m) xa[a][m] = xf(a, m, 2 * q + half);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
#pragma unroll
                    for (int a = 0; a < NS; ++a) {
                        const uint32_t cp = __builtin_bit_cast(uint32_t, c[a][i]);
#pragma unroll
                        for (int m = 0; m < MC; ++m) {
                            const uint32_t xp = xa[a][m][i >> 1];
                            if (half) {
                                if (i & 1) mix_mac<1, 1>(t[a][m], cp, xp);
                                else mix_mac<1, 0>(t[a][m], cp, xp);
                            } else {
                                if (i & 1) mix_mac<0, 1>(t[a][m], cp, xp);
                                else mix_mac<0, 0>(t[a][m], cp, xp);
                            }
                        }
                    }
                }
            }
        } else if constexpr (F == FMT_INT4) {
            h2_t c[NS][4];
#pragma unroll
            for (int a = 0; a < NS; ++a) int4_decode_word(w[a][q], kc, c[a]);
            u4_t xa[NS][MC];
#pragma unroll
            for (int a = 0; a < NS; ++a)
#pragma unroll
                for (int m = 0; m < MC; ++m) xa[a][m] = xf(a, m, q);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int a = 0; a < NS; ++a) {
                    // code i of the word: low half of pair i (i < 4) or high
                    // half of pair i - 4
                    const uint32_t cp = __builtin_bit_cast(uint32_t, c[a][i & 3]);
#pragma unroll
                    for (int m = 0; m < MC; ++m) {
                        const uint32_t xp = xa[a][m][i >> 1];
                        if (i >= 4) {
                            if (i & 1) mix_mac<1, 1>(t[a][m], cp, xp);
                            else mix_mac<1, 0>(t[a][m], cp, xp);
                        } else {
                            if (i & 1) mix_mac<0, 1>(t[a][m], cp, xp);
                            else mix_mac<0, 0>(t[a][m], cp, xp);
                        }
                    }
                }
            }
        } else {  // MXFP4: byte b of word q holds elements 8q+2b (low) and 8q+2b+1 (high)
            f2_t c[NS][4];
#pragma unroll
            for (int a = 0; a < NS; ++a) {
                c[a][0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[a][q], 1.0f, 0);
                c[a][1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[a][q], 1.0f, 1);
                c[a][2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[a][q], 1.0f, 2);
                c[a][3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[a][q], 1.0f, 3);
            }
            u4_t xa[NS][MC];
#pragma unroll
            for (int a = 0; a < NS; ++a)
#pragma unroll
                for (int m = 0; m < MC; ++m) xa[a][m] = xf(a, m, q);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int a = 0; a < NS; ++a) {
                    const float cv = (i & 1) ? c[a][i >> 1].y : c[a][i >> 1].x;
#pragma unroll
                    for (int m = 0; m < MC; ++m) {
                        const uint32_t xp = xa[a][m][i >> 1];
                        const float xv = (i & 1) ? u2f(xp & 0xFFFF0000u) : u2f(xp << 16);
                        t[a][m] = __builtin_fmaf(cv, xv, t[a][m]);
                    }
                }
            }
        }
    }
}


// MXFP4 inner step with the activations already in fp32 (bf16 widens
// exactly): for the NS segments, t[a] = t[a] (+) e2m1_k * x_k for k ascending,
// one fused multiply-add per code.  XF(a, k) returns activation k of segment
// a as a float.  Byte b of word q holds elements 8q+2b (low nibble) and
// 8q+2b+1 (high nibble).
template <int NS, class XF>
__device__ __forceinline__ void mx_sums_f32(const u4_t (&w)[NS], XF &&xf, float (&t)[NS][1]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        f2_t c[NS][4];
#pragma unroll
        for (int a = 0; a < NS; ++a) {
            c[a][0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[a][q], 1.0f, 0);
            c[a][1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[a][q], 1.0f, 1);
            c[a][2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[a][q], 1.0f, 2);
            c[a][3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[a][q], 1.0f, 3);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int a = 0; a < NS; ++a) {
                const float cv = (i & 1) ? c[a][i >> 1].y : c[a][i >> 1].x;
                t[a][0] = __builtin_fmaf(cv, xf(a, 8 * q + i), t[a][0]);
            }
    }
}

// Inner step for one segment of R rows (the same segment index of R
// different rows) and MC activation columns read from LDS:
//   t[r][m] = t[r][m] (+) value[r]_k * x[m][k]   for k ascending over the segment.
// xs + xo is the segment's first activation of column 0; column m is K
// elements further on.  The segment is walked in steps of 8 codes; each
// step reads one 16-byte activation vector per column and uses every value
// for all R rows.  The LDS offset is re-derived through an opaque copy at
// every step so the reads stay next to their use (hoisting them makes the
// compiler hold a whole segment of activations for every column).
// Ternary several-column inner step: R rows (the same segment of R rows)
// and MC activation columns read from LDS; each word is decoded once for all
// MC columns and each activation vector is used for all R rows.  Codes run
// in order k = 0 .. 79 in every (row, column) chain; the opaque offsets and
// words follow the generic several-column step below.
template <int R, int MC>
__device__ __forceinline__ void tern_sums_rows(const u4_t (&w)[R], const DecodeConsts &kc, const uint16_t *xs,
                                               int xo, int K, float (&t)[R][MC]) {
    h2_t c[R][10];
    u4_t xa[MC];
    float dep = 0.0f;
#pragma unroll
    for (int k = 0; k < 80; ++k) {
        if (k % 20 == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                uint32_t wv = w[r][k / 20];
                asm volatile("" : "+v"(wv) : "v"(dep));
                tern_decode_word(wv, kc, c[r]);
            }
        }
        if (k % 8 == 0) {
            int o = xo + k;
            asm volatile("" : "+v"(o) : "v"(dep));
#pragma unroll
            for (int m = 0; m < MC; ++m) xa[m] = *reinterpret_cast<const u4_t *>(xs + m * K + o);
        }
        const int byte = (k % 20) / 5, dig = k % 5;
        const int pair = 2 * dig + (byte & 1);
        const bool wh = byte >= 2, xh = k & 1;
#pragma unroll
        for (int m = 0; m < MC; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t cp = __builtin_bit_cast(uint32_t, c[r][pair]);
                const uint32_t xp = xa[m][(k & 7) >> 1];
                if (wh) {
                    if (xh) mix_mac<1, 1>(t[r][m], cp, xp);
                    else mix_mac<1, 0>(t[r][m], cp, xp);
                } else {
                    if (xh) mix_mac<0, 1>(t[r][m], cp, xp);
                    else mix_mac<0, 0>(t[r][m], cp, xp);
                }
            }
        if (k % 8 == 0) dep = t[0][0];
        if (k % 8 == 7) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < MC; ++m) asm volatile("" : "+v"(t[r][m]));
        }
    }
}

template <int F, int R, int MC>
__device__ __forceinline__ void segment_sums_rows(const u4_t (&w)[R], const DecodeConsts &kc,
                                                  const uint16_t *xs, int xo, int K,
                                                  float (&t)[R][MC]) {
    if constexpr (F == FMT_TERN) {
        tern_sums_rows<R, MC>(w, kc, xs, xo, K, t);
        return;
    }
    constexpr int STEPS = SegCodes<F>::v / 8;
    // `dep` carries a value of the previous step into the opaque offset, so
    // a step's reads can be issued once the previous step has started but
    // not earlier (an opaque copy alone may be scheduled anywhere before).
    float dep = 0.0f;
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
        int o = xo + 8 * st;
        asm volatile("" : "+v"(o) : "v"(dep));
        u4_t xa[MC];
#pragma unroll
        for (int m = 0; m < MC; ++m) xa[m] = *reinterpret_cast<const u4_t *>(xs + m * K + o);
        if constexpr (F == FMT_INT2) {
            // word st/2; fp16 pair i of a word = (code i, code i+8)
            h2_t c[R][8];
#pragma unroll
            for (int r = 0; r < R; ++r) int2_decode_word(w[r][st >> 1], kc, c[r]);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int m = 0; m < MC; ++m)
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const uint32_t cp = __builtin_bit_cast(uint32_t, c[r][i]);
                        const uint32_t xp = xa[m][i >> 1];
                        if (st & 1) {
                            if (i & 1) mix_mac<1, 1>(t[r][m], cp, xp);
                            else mix_mac<1, 0>(t[r][m], cp, xp);
                        } else {
                            if (i & 1) mix_mac<0, 1>(t[r][m], cp, xp);
                            else mix_mac<0, 0>(t[r][m], cp, xp);
                        }
                    }
                if (i == 0) dep = t[0][0];
            }
        } else if constexpr (F == FMT_INT4) {
            // fp16 pair p of a word = (code p, code p+4)
            h2_t c[R][4];
#pragma unroll
            for (int r = 0; r < R; ++r) int4_decode_word(w[r][st], kc, c[r]);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int m = 0; m < MC; ++m)
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const uint32_t cp = __builtin_bit_cast(uint32_t, c[r][i & 3]);
                        const uint32_t xp = xa[m][i >> 1];
                        if (i >= 4) {
                            if (i & 1) mix_mac<1, 1>(t[r][m], cp, xp);
                            else mix_mac<1, 0>(t[r][m], cp, xp);
                        } else {
                            if (i & 1) mix_mac<0, 1>(t[r][m], cp, xp);
                            else mix_mac<0, 0>(t[r][m], cp, xp);
                        }
                    }
                if (i == 0) dep = t[0][0];
            }
        } else {  // MXFP4: byte b of word st holds elements 8st+2b (low) and 8st+2b+1 (high)
            // the word goes through an opaque copy too: converted early, the
            // codes of every step would be live at once
            f2_t c[R][4];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                uint32_t wv = w[r][st];
                asm volatile("" : "+v"(wv) : "v"(dep));
                c[r][0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wv, 1.0f, 0);
                c[r][1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wv, 1.0f, 1);
                c[r][2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wv, 1.0f, 2);
                c[r][3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wv, 1.0f, 3);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int m = 0; m < MC; ++m) {
                    const uint32_t xp = xa[m][i >> 1];
                    const float xv = (i & 1) ? u2f(xp & 0xFFFF0000u) : u2f(xp << 16);
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const float cv = (i & 1) ? c[r][i >> 1].y : c[r][i >> 1].x;
                        t[r][m] = __builtin_fmaf(cv, xv, t[r][m]);
                    }
                }
                if (i == 0) dep = t[0][0];
            }
        }
        // every chain finishes this step before any starts the next: left
        // free, the compiler runs chains one after another and then needs the
        // activations of all steps at once
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MC; ++m) asm volatile("" : "+v"(t[r][m]));
    }
}

// The value of lane l + S for lanes l whose group of 2S lanes starts at a
// multiple of 2S (other lanes get values that the tree never reads).
// S <= 8: a DPP row shift inside the 16-lane row (one VALU instruction,
// folded into the add); S = 16, 32 cross 16-lane rows and go through
// ds_bpermute.
template <int S>
__device__ __forceinline__ float lane_down(float r) {
    if constexpr (S >= 16) {
        return __shfl_down(r, S, 64);
    } else {
        return __builtin_bit_cast(
            float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, r), 0x100 + S, 0xF, 0xF, true));
    }
}

// One cross-lane tree level of distance S in groups of RL lanes (levels with
// S >= RL do not exist; levels above the padded width s0 are skipped).
template <int RL, int S>
__device__ __forceinline__ void lane_level(float &r, int s0) {
    if constexpr (S < RL) {
        const float o = lane_down<S>(r);
        if (S <= s0) r = r + o;
    }
}


// Fixed-order tree over the segment values of one row.  Lane q of a group
// of RL lanes holds the segments j = q + RL*a in v[a] (+0 beyond the row's
// segment count).  The halving tree over P2 entries
//   for s = P2/2 .. 1:  v_p = v_p (+) v_{p+s}  (p < s)
// pairs entries of the same lane while s >= RL and lanes q and q+s after
// that.  The total is returned in lane q == 0 of the group.
template <int RL, int NIP>
__device__ __forceinline__ float fo_tree(float (&v)[NIP], int P2) {
    if (P2 > RL) {
        const int ll = P2 / RL;  // lane-local entries, a power of two <= NIP
#pragma unroll
        for (int s = NIP / 2; s >= 1; s >>= 1) {
            if (s < ll) {
#pragma unroll
                for (int a = 0; a < s; ++a) v[a] = v[a] + v[a + s];
            }
        }
    }
    float r = v[0];
    // rows shorter than a lane group (P2 < RL) skip the levels above P2/2
    const int s0 = P2 >= RL ? RL / 2 : P2 / 2;
    lane_level<RL, 32>(r, s0);
    lane_level<RL, 16>(r, s0);
    lane_level<RL, 8>(r, s0);
    lane_level<RL, 4>(r, s0);
    lane_level<RL, 2>(r, s0);
    lane_level<RL, 1>(r, s0);
    return r;
}

// Round an fp32 value (already rounded to fp32) to fp16 / bf16, nearest-even.
// The empty asm pins the fp32 value in a register: without it the compiler
// may fold the producing fp32 multiply and this conversion into one
// mixed-precision fma (v_fma_mixlo_f16), which rounds the exact product once
// to fp16 instead of first to fp32 -- a different result in rare ties.
__device__ __forceinline__ _Float16 to_f16(float v) {
    asm volatile("" : "+v"(v));
    return (_Float16)v;
}
__device__ __forceinline__ __bf16 to_bf16(float v) {
    asm volatile("" : "+v"(v));
    return (__bf16)v;
}

// Output conversions: one round-to-nearest-even of the fp32 value.
__device__ __forceinline__ void store_out(void *y, size_t idx, float v, int dtype) {
    if (dtype == 0)
        reinterpret_cast<float *>(y)[idx] = v;
    else if (dtype == 1)
        reinterpret_cast<_Float16 *>(y)[idx] = to_f16(v);
    else
        reinterpret_cast<__bf16 *>(y)[idx] = to_bf16(v);
}

// Output stores that every lane of the wave issues, with no divergent
// branch around them: a lane with nothing to store passes an offset past the
// end of the buffer, and the hardware drops that store.  Inside a loop that
// streams weights through a ring of loads, a store under a divergent branch
// makes the compiler's count of outstanding memory operations inexact, and it
// then waits for every load in flight at the top of each row.  dtype
// (uniform): 0 fp32, 1 fp16, 2 bf16; the buffer holds `elems` elements
// (elems times the element size must stay below 4 GiB).
constexpr uint32_t kStoreOob = 0xFFFFFFF0u;
// The same offset on a buffer load returns zeros without touching memory.
constexpr uint32_t kLoadOob = 0xFFFFFFF0u;
struct OutBuf {
    __amdgpu_buffer_rsrc_t r;
    int dtype;
    __device__ __forceinline__ OutBuf(void *p, uint32_t elems, int dtype_) : dtype(dtype_) {
        const uint32_t esz = dtype_ == 0 ? 4u : 2u;
        r = __builtin_amdgcn_make_buffer_rsrc(p, 0, elems * esz, 0x00020000);
    }
    __device__ __forceinline__ void put(bool active, uint32_t idx, float v) const {
        if (dtype == 0) {
            __builtin_amdgcn_raw_buffer_store_b32(f2u(v), r, active ? idx * 4u : kStoreOob, 0, 0);
        } else if (dtype == 1) {
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, to_f16(v)), r,
                                                  active ? idx * 2u : kStoreOob, 0, 0);
        } else {
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, to_bf16(v)), r,
                                                  active ? idx * 2u : kStoreOob, 0, 0);
        }
    }
};

// MXFP4 quantisation of one 32-value block per 32-lane half of the wave
// (OCP MX v1.0 conversion): lane l of the half holds element l as fp16 bits.
// The shared exponent is floor(log2(max |v|)) - 2 (2 = the exponent of
// E2M1's largest value 6): for a normal fp32 max with biased exponent ex the
// E8M0 byte is ex - 2 and 2^-shared has the exponent field 256 - ex; an
// all-zero block takes the byte 0.  v * 2^-shared is exact (|q| < 8) and the
// hardware conversion rounds it to E2M1 (nearest, ties to even, clamped to
// 6, sign kept).  Element 2j goes to the low nibble of byte j, 2j+1 to the
// high nibble.  Every lane of the wave must call this (cross-lane reads);
// only halves with `store` set write.
__device__ __forceinline__ void mx_quant_half(uint16_t h, bool store, uint8_t *codes, uint8_t *scale) {
    const int l = threadIdx.x & 31;
    const float v = half_bits_to_f32(h);
    float a = __builtin_fabsf(v);
#pragma unroll
    for (int s = 16; s >= 1; s >>= 1) a = __builtin_fmaxf(a, __shfl_xor(a, s, 32));
    const uint32_t ex = f2u(a) >> 23;  // a >= 0, finite
    const bool zero = !(a > 0.0f);
    const float inv = u2f((256u - ex) << 23);
    const float q = zero ? v : v * inv;
    const float q_odd = __shfl_down(q, 1, 32);
    const uint32_t b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q, q_odd, 1.0f, 0) & 0xFFu;
    if (store && (l & 1) == 0) codes[l >> 1] = (uint8_t)b;
    if (store && l == 0) *scale = (uint8_t)(zero ? 0u : ex - 2u);
}

// e^z for z in [-87, 87]: z = n ln2 + r (Cody & Waite: ln2 split into a
// 15-significant-bit head, exact when multiplied by |n| <= 127, and a tail),
// e^r by the degree-7 Taylor polynomial with binary32-rounded coefficients
// 1/j! in Horner form with fused multiply-adds, times 2^n built from its
// exponent field.
__device__ __forceinline__ float qmv_exp(float z) {
    const float kLog2e = 0x1.715476p+0f;
    const float kLn2Hi = 0x1.62e4p-1f;
    const float kLn2Lo = 0x1.7f7d1cp-20f;
    const float t = z * kLog2e;
    const float n = __builtin_rintf(t);
    float r = __builtin_fmaf(-n, kLn2Hi, z);
    r = __builtin_fmaf(-n, kLn2Lo, r);
    float p = 0x1.a01a02p-13f;            // 1/7!
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);  // 1/6!
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);   // 1/5!
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);   // 1/4!
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);   // 1/3!
    p = __builtin_fmaf(p, r, 0x1p-1f);          // 1/2!
    p = __builtin_fmaf(p, r, 0x1p+0f);          // 1/1!
    p = __builtin_fmaf(p, r, 0x1p+0f);          // 1/0!
    const int ni = (int)n;
    const float two_n = u2f((uint32_t)(ni + 127) << 23);
    return p * two_n;
}

// GELU, tanh form, through (1 + tanh u)/2 = 1/(1 + e^(-2u)):
//   u = sqrt(2/pi) * (g + 0.044715 g^3),  GELU = g / (1 + e^(clamp(-2u)))
__device__ __forceinline__ float qmv_gelu(float g) {
    const float kSqrt2OverPi = 0x1.988454p-1f;
    const float kC = 0x1.6e4e26p-5f;  // 0.044715
    const float g2 = g * g;
    const float g3 = g2 * g;
    const float cg3 = kC * g3;
    const float inner = g + cg3;
    const float u = kSqrt2OverPi * inner;
    float z = -2.0f * u;
    if (z > 87.0f) z = 87.0f;
    if (z < -87.0f) z = -87.0f;
    const float e = qmv_exp(z);
    const float den = 1.0f + e;
    return g / den;
}

// argmax key: order by value (-0 == +0), then by smaller row index; the
// lowest bit keeps the sign of a zero so the winning logit is returned
// with its own bits.
__device__ __forceinline__ uint64_t argmax_key(float y, int n) {
    const uint32_t sign0 = f2u(y) >> 31;
    const float yc = y + 0.0f;  // -0 -> +0; identity otherwise
    const uint32_t b = f2u(yc);
    const uint32_t mono = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    const uint32_t lo = ((0x7FFFFFFFu - (uint32_t)n) << 1) | sign0;
    return ((uint64_t)mono << 32) | lo;
}

__device__ __forceinline__ void argmax_key_decode(uint64_t key, int &n, float &y) {
    const uint32_t mono = (uint32_t)(key >> 32), lo = (uint32_t)key;
    const uint32_t b = (mono & 0x80000000u) ? (mono & 0x7FFFFFFFu) : ~mono;
    n = (int)(0x7FFFFFFFu - (lo >> 1));
    y = u2f(b);
    if (y == 0.0f && (lo & 1u)) y = -0.0f;
}

}  // namespace qmv
