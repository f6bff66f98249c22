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

enum Fmt : int { FMT_INT2 = 0, FMT_INT4 = 1, FMT_MXFP4 = 2 };

// Codes held by one 16-byte segment (one dwordx4 load) of a packed row.
template <int F> struct SegCodes;
template <> struct SegCodes<FMT_INT2> { static constexpr int v = 64; };
template <> struct SegCodes<FMT_INT4> { static constexpr int v = 32; };
template <> struct SegCodes<FMT_MXFP4> { static constexpr int v = 32; };

__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ h2_t u2h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }
__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return u2f((uint32_t)b << 16); }

__device__ __forceinline__ h2_t fma_h2(h2_t a, float mul, float add) {
    const h2_t m = {(_Float16)mul, (_Float16)mul};
    const h2_t c = {(_Float16)add, (_Float16)add};
    return __builtin_elementwise_fma(a, m, c);
}

// fp16 1024.0 in both halves: OR-ing a field into the low mantissa bits of
// this pattern gives the fp16 value 1024 + field * 2^(bit position).
constexpr uint32_t kMagic1024 = 0x64006400u;

// int2: 16 two's-complement 2-bit fields of one word -> 8 packed fp16 pairs,
// pair i = (code i, code i+8).  XOR with 0b10 in every field maps the field
// f to f^2 = value + 2 in 0..3; the field is placed in an fp16 mantissa
// (1024 + 4^i (value+2)) and one exact packed fma scales by 4^-i and removes
// the bias: (1024 + 4^i b) 4^-i - (1024 4^-i + 2) = b - 2.
__device__ __forceinline__ void int2_decode_word(uint32_t w, h2_t (&c)[8]) {
    const uint32_t u = w ^ 0xAAAAAAAAu;
    const uint32_t v = u >> 10;  // fields 5..7 and 13..15 to bits 0..5 / 16..21
    c[0] = fma_h2(u2h2((u & 0x00030003u) | kMagic1024), 1.0f, -1026.0f);
    c[1] = fma_h2(u2h2((u & 0x000C000Cu) | kMagic1024), 0.25f, -258.0f);
    c[2] = fma_h2(u2h2((u & 0x00300030u) | kMagic1024), 0.0625f, -66.0f);
    c[3] = fma_h2(u2h2((u & 0x00C000C0u) | kMagic1024), 0.015625f, -18.0f);
    c[4] = fma_h2(u2h2((u & 0x03000300u) | kMagic1024), 0.00390625f, -6.0f);
    c[5] = fma_h2(u2h2((v & 0x00030003u) | kMagic1024), 1.0f, -1026.0f);
    c[6] = fma_h2(u2h2((v & 0x000C000Cu) | kMagic1024), 0.25f, -258.0f);
    c[7] = fma_h2(u2h2((v & 0x00300030u) | kMagic1024), 0.0625f, -66.0f);
}

// int4: 8 nibbles q of one word -> 4 packed fp16 pairs of q - 8,
// pair i = (code i, code i+4).
__device__ __forceinline__ void int4_decode_word(uint32_t w, h2_t (&c)[4]) {
    const uint32_t v = w >> 8;
    c[0] = fma_h2(u2h2((w & 0x000F000Fu) | kMagic1024), 1.0f, -1032.0f);
    c[1] = fma_h2(u2h2((w & 0x00F000F0u) | kMagic1024), 0.0625f, -72.0f);
    c[2] = fma_h2(u2h2((v & 0x000F000Fu) | kMagic1024), 1.0f, -1032.0f);
    c[3] = fma_h2(u2h2((v & 0x00F000F0u) | kMagic1024), 0.0625f, -72.0f);
}

// E8M0 block scale as an fp32 value: 2^(E-127), exact for E in 0..254
// (E = 0 is the subnormal 2^-127), NaN for E = 255.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
    return e == 0u ? u2f(0x00400000u) : (e == 255u ? u2f(0x7FC00000u) : u2f(e << 23));
}

// Inner step of one 16-byte segment for MC activation columns:
//   t[m] = t[m] (+) value_k * x[m][k]   for k ascending over the segment.
// XF(m, v) returns 8 consecutive activation values (16 bytes) of column m at
// segment offset 8v.
template <int F, int MC, class XF>
__device__ __forceinline__ void segment_sum(const u4_t &w, XF &&xf, float (&t)[MC]) {
    if constexpr (F == FMT_INT2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            h2_t c[8];
            int2_decode_word(w[q], c);
#pragma unroll
            for (int m = 0; m < MC; ++m) {
                const u4_t xa = xf(m, 2 * q), xb = xf(m, 2 * q + 1);
                const uint32_t xs[8] = {xa[0], xa[1], xa[2], xa[3], xb[0], xb[1], xb[2], xb[3]};
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const _Float16 cv = (i < 8) ? c[i].x : c[i - 8].y;
                    const h2_t xp = u2h2(xs[i >> 1]);
                    const _Float16 xv = (i & 1) ? xp.y : xp.x;
                    t[m] = __builtin_fmaf((float)cv, (float)xv, t[m]);  // exact product
                }
            }
        }
    } else if constexpr (F == FMT_INT4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            h2_t c[4];
            int4_decode_word(w[q], c);
#pragma unroll
            for (int m = 0; m < MC; ++m) {
                const u4_t xa = xf(m, q);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const _Float16 cv = (i < 4) ? c[i].x : c[i - 4].y;
                    const h2_t xp = u2h2(xa[i >> 1]);
                    const _Float16 xv = (i & 1) ? xp.y : xp.x;
                    t[m] = __builtin_fmaf((float)cv, (float)xv, t[m]);
                }
            }
        }
    } else {  // MXFP4: byte b of word q holds elements 8q+2b (low) and 8q+2b+1 (high)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f2_t c[4];
            c[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 0);
            c[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 1);
            c[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 2);
            c[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 3);
#pragma unroll
            for (int m = 0; m < MC; ++m) {
                const u4_t xa = xf(m, q);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float cv = (i & 1) ? c[i >> 1].y : c[i >> 1].x;
                    const uint32_t xp = xa[i >> 1];
                    const float xv = (i & 1) ? u2f(xp & 0xFFFF0000u) : u2f(xp << 16);
                    t[m] = __builtin_fmaf(cv, xv, t[m]);
                }
            }
        }
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
    const int s0 = (P2 < RL ? P2 : RL) / 2;
#pragma unroll
    for (int s = RL / 2; s >= 1; s >>= 1) {
        const float o = __shfl_down(r, s, RL);
        if (s <= s0) r = r + o;
    }
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
