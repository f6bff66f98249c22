// qmv_fo.hip -- fixed-order (bit-exact) kernels for gfx950:
//   * int2 / int4 / MXFP4 matvec and skinny GEMM,
//   * residual-add + RMSNorm prologue -> dual int2 gate/up -> GELU*up,
//   * int2 lm_head with single-dispatch first-max argmax.
//
// Design (MI355X): one 16-byte segment per lane per load (global_load_dwordx4)
// so a wave streams whole rows with fully used cache lines; the activation
// chunk [MC][K] is staged once per workgroup in LDS and, for MC = 1, copied
// into registers per lane (each lane always works on the same segment
// indices, so its slice of x is loop-invariant); the per-segment sums are
// reduced with the fixed halving tree (in-lane levels, then lane shuffles).
// Decoding happens inside the dot product (no dequantized weights are ever
// written): "26 Iterations: Porting Cleanroom Kernels to Gemma 4", "The
// Wins", scalar inline-dequant.  The order is the one fixed in qmv.h and is
// independent of the lane layout, MC, and the grid ("Gemma4 raw-Metal loop on
// A19", "What moved the needle": tiles must not change the merge order).
#include "qmv_device.hpp"
#include "qmv_internal.hpp"

namespace qmv {

// Launch shape; the macros let a build explore other shapes.
#ifndef QMV_BLOCK
#define QMV_BLOCK 256
#endif
#ifndef QMV_MAX_GRID
#define QMV_MAX_GRID 1024
#endif
#ifndef QMV_MX_XF32
#define QMV_MX_XF32 1
#endif
#ifndef QMV_XREG_BUDGET
#define QMV_XREG_BUDGET 96
#endif
constexpr int kBlock = QMV_BLOCK;  // waves of 64 lanes per workgroup
constexpr int kWaves = kBlock / 64;
constexpr int kMaxGrid = QMV_MAX_GRID;

bool pick_shape(int nseg, LaneShape &s) {
    if (nseg <= 0) return false;
    if (nseg <= 8) s = {8, 1, 1};
    else if (nseg <= 16) s = {16, 1, 1};
    else if (nseg <= 24) s = {8, 3, 4};
    else if (nseg <= 32) s = {32, 1, 1};
    else if (nseg <= 64) s = {64, 1, 1};
    // two rows per wave: half the tree and epilogue work per row
    else if (nseg <= 96) s = {32, 3, 4};
    else if (nseg <= 128) s = {32, 4, 4};
    else if (nseg <= 192) s = {64, 3, 4};
    else if (nseg <= 256) s = {64, 4, 4};
    else if (nseg <= 512) s = {64, 8, 8};
    else return false;
    return true;
}

// Few rows: when N fills fewer than one row group per SIMD (1024 on
// MI355X), spread a row over more lanes (fewer rows per wave, more waves) as
// long as at least half of the row's lanes hold a segment.  The order of the sums does not depend
// on the layout.
// Measured: the fused gate/up at N=8192 (1024 row groups of eight rows)
// runs 7.7 us widened to 32 lanes per row and 6.0 us as is; the int2 matvec
// at N=2048 (256 row groups) 3.8 us as is and 3.0 us widened.
#ifndef QMV_FEW_RG
#define QMV_FEW_RG 1024
#endif
constexpr long kFewRowGroups = QMV_FEW_RG;

bool pick_shape_rows(int nseg, long N, LaneShape &s) {
    if (!pick_shape(nseg, s)) return false;
    static const LaneShape wider[] = {{16, 1, 1}, {32, 1, 1}, {64, 1, 1}};
    for (const LaneShape &w : wider) {
        const long rg = (N + 64 / s.RL - 1) / (64 / s.RL);
        if (rg >= kFewRowGroups) break;
        if (w.RL <= s.RL || w.RL * w.NI < nseg || w.RL > 2 * nseg) continue;
        s = w;
    }
    return true;
}

static inline int pow2_ceil(int n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

// ---------------------------------------------------------------------------
// Activation staging: rows m0 .. m0+MC-1 of x[M][K] -> LDS xs[MC][K]
// (zeros for rows beyond M), 16-byte vectors.  Split in two so that the
// global loads of x are issued before the weight prefetch: vector loads
// retire in issue order, so waiting for x issued after the weights would
// also wait for the weights.  Up to kXpt vectors per thread go through
// registers; any remainder is copied after the prefetch.
constexpr int kXpt = 4;

template <int MC>
struct XStage {
    u4_t v[kXpt];
    // Row m of the staged chunk is x[m0 + m][0 .. len); `ld` is the row
    // stride of x (len < ld when one K split is staged).
    // Only the first `valid` values of a row exist in x (a row padded to whole
    // segments); the rest of the staged row is zero.
    __device__ __forceinline__ void load(const uint16_t *__restrict__ x, int M, int ld, int len, int m0,
                                         int valid = -1) {
        const int per_row = len / 8, vrow = (valid < 0 ? len : valid) / 8;
#pragma unroll
        for (int r = 0; r < kXpt; ++r) {
            const int e = threadIdx.x + r * blockDim.x;
            v[r] = u4_t{0u, 0u, 0u, 0u};
            if (e < MC * per_row) {
                const int m = MC == 1 ? 0 : e / per_row, kk = e - m * per_row;
                if (m0 + m < M && kk < vrow)
                    v[r] = *reinterpret_cast<const u4_t *>(x + (size_t)(m0 + m) * ld + 8 * kk);
            }
        }
    }
    __device__ __forceinline__ void store(const uint16_t *__restrict__ x, uint16_t *xs, int M, int ld, int len,
                                          int m0, int valid = -1) {
        const int vrow = (valid < 0 ? len : valid) / 8;
        const int per_row = len / 8;
#pragma unroll
        for (int r = 0; r < kXpt; ++r) {
            const int e = threadIdx.x + r * blockDim.x;
            if (e < MC * per_row) *reinterpret_cast<u4_t *>(xs + 8 * e) = v[r];
        }
        for (int e = threadIdx.x + kXpt * blockDim.x; e < MC * per_row; e += blockDim.x) {
            const int m = MC == 1 ? 0 : e / per_row, kk = e - m * per_row;
            u4_t w = {0u, 0u, 0u, 0u};
            if (m0 + m < M && kk < vrow) w = *reinterpret_cast<const u4_t *>(x + (size_t)(m0 + m) * ld + 8 * kk);
            *reinterpret_cast<u4_t *>(xs + (size_t)m * len + 8 * kk) = w;
        }
    }
};

// Ring depth: how many row groups a wave keeps in flight besides the one it
// is computing.  One measured fastest on MI355X for every format: deeper
// rings cost registers (fewer resident waves) without adding bandwidth.
template <int NI, int NMAT>
constexpr int ring_depth() {
#ifdef QMV_RING
    return QMV_RING;
#else
    return 1;
#endif
}

// Rows blocked per unit: several activation columns read from LDS use each
// activation value for QMV_ROWS rows (QMV_ROWS_MX for MXFP4, whose bf16
// activations take one widening instruction per value and column); one
// column keeps the register copy.  Measured on MI355X (N=21504, K=5376,
// bit-identical results): MXFP4 M = 16 / 64 / 256 take 120.5 / 441.9 /
// 1761.5 us with two rows, 112.5 / 406.3 / 1569.4 with four, 125.1 / 460.2 /
// 1797.4 with eight; int4 (N=16384, K=4096) M = 4 takes 20.9 us with two
// rows and 25.9 with four, M = 8 and 16 within 3 %.
#ifndef QMV_ROWS
#define QMV_ROWS 2
#endif
#ifndef QMV_ROWS1
#define QMV_ROWS1 1
#endif
#ifndef QMV_ROWS_MX
#define QMV_ROWS_MX 4
#endif
template <int MC, bool XREG, int F = -1>
constexpr int rows_block() {
    return (MC > 1 && !XREG) ? (F == FMT_MXFP4 ? QMV_ROWS_MX : QMV_ROWS) : (MC == 1 ? QMV_ROWS1 : 1);
}

// Raw loaded bits only: converting a scale in the load routine would make
// the wave wait for that load right there.  A slot holds R row groups.
template <int F, int NI, int NMAT, int R>
struct RowSlot {
    u4_t w[NMAT][R][NI];
    uint32_t seg[NMAT][R][NI];  // int4 / MXFP4 segment scale bits (fp16 / E8M0)
    uint32_t rs[NMAT][R];       // int2 row scale bits (fp16)
};

template <int F>
__device__ __forceinline__ float seg_scale(uint32_t bits) {
    if constexpr (F == FMT_INT4) return half_bits_to_f32((uint16_t)bits);
    else return e8m0_to_f32(bits);
}

// The FO row engine.  NMAT weight matrices (1, or 2 for gate/up) share the
// activation chunk.  A wave walks units u = first, first+stride, ...; a unit
// is R adjacent row groups of RPG rows each.  With one activation column and
// R = 1 the weights stream through a ring of one-segment slots (run_stream);
// otherwise loads go through a ring of D unit slots: the next D units are in
// flight while one is computed.  prefetch() issues the first loads and is
// called before the activations are staged, so staging overlaps the first
// weight fetches.  For every row group, lane
// q == 0 of each RL-lane group hands the reduced totals tot[mat][m] (before
// the int2 row scale) and the row scales rs[mat] to the epilogue.
//
// R > 1 (used with several activation columns read from LDS): every
// activation value read (and widened) is used for R rows, which divides the
// LDS traffic and conversion work per multiply-add by R.
template <int F, int RL, int NI, int NIP, int MC, bool XREG, int NMAT, int D, int R, int WV = kWaves>
struct FoEngine {
    static constexpr int CODES = SegCodes<F>::v;
    static constexpr int XV = CODES / 8;  // 16-byte activation vectors per segment per column
    static constexpr int RPG = 64 / RL;   // rows per wave per row group
    static constexpr int kRowsPerUnit = R * RPG;

    int N, K, nseg, P2, q, rsub, total_units, stride, first;
    uint32_t row_bytes, srow;
    // Buffer descriptors (SGPRs) for the packed weights and their scales.
    // Raw buffer loads take a 32-bit per-lane offset and return zero for any
    // offset past the end of the buffer, so rows past N (a partial last row
    // group, or units past the end) need no clamps or branches.
    __amdgpu_buffer_rsrc_t rw[NMAT], rsc[NMAT];
    uint32_t woff, soff;        // offsets of the next unit to load
    uint32_t wstep, sstep;      // bytes between consecutive units of a wave
    // With one activation column a slot is refilled before the unit in it is
    // computed (D units always in flight), which takes D + 1 slots; the unit
    // loop is unrolled over all of them so no slot is ever copied.  With
    // several columns read from LDS the kernel is bound by arithmetic and a
    // slot is refilled after its unit, keeping registers (and occupancy).
    static constexpr bool kRefillFirst = XREG || MC == 1;
    static constexpr int NSLOT = kRefillFirst ? D + 1 : D;
    // One activation column and one row group per unit: the loads stream at
    // the granularity of one segment (16 bytes per lane, 1 KB per wave).
    // Segment i of a unit sits in slot i and is refilled with segment i of
    // the wave's next unit as soon as it has been summed, so about NI
    // segments are in flight at all times and the refills are spread evenly
    // over the computation (rather than one unit's worth at a time, which
    // leaves the memory system idle and then floods it).  A lane with one
    // segment per unit uses two slots over two units.
    static constexpr bool kStream = MC == 1 && R == 1;
    static constexpr int NS = NI >= 2 ? NI : 2;
    static constexpr int NU = NS / NI;  // units per pass over the slots
    struct SegSlot {
        u4_t w[NMAT];
        uint32_t sb[NMAT];  // int4 / MXFP4 segment scale bits
        uint32_t rs[NMAT];  // int2 row scale bits (loaded with segment 0)
    };
    SegSlot ss[kStream ? NS : 1];
    int sseg = 0;  // segment index of the next streamed load
    RowSlot<F, NI, NMAT, R> slot[kStream ? 1 : NSLOT];

    static constexpr int kNT = 2;  // non-temporal: the weights are read once

    // K_ is the number of codes this engine sums per row (a whole row, or one
    // K split of nseg_row-segment rows starting at segment seg0).
    // blk / nblk: this workgroup's index among the nblk workgroups that share
    // the rows (default: the whole grid along x)
    __device__ __forceinline__ FoEngine(const uint8_t *const (&wq)[NMAT], const void *const (&sc)[NMAT],
                                        int N_, int K_, int seg0 = 0, int nseg_row = 0, int blk = -1,
                                        int nblk = -1)
        : N(N_), K(K_) {
        if (blk < 0) {
            blk = blockIdx.x;
            nblk = gridDim.x;
        }
        nseg = K / CODES;
        if (nseg_row == 0) nseg_row = nseg;
        P2 = 1;
        while (P2 < nseg) P2 <<= 1;
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        q = lane % RL;
        rsub = lane / RL;
        row_bytes = (uint32_t)nseg_row * 16u;
        const int total_rg = (N + RPG - 1) / RPG;
        total_units = (total_rg + R - 1) / R;
        stride = nblk * WV;
        // wave-uniform: read it through a scalar so that the unit loop is a
        // scalar loop (no exec-masked control flow around the load ring)
        first = __builtin_amdgcn_readfirstlane(blk * WV + wave);
        // bytes of scale data per row
        srow = kRowScale<F> ? 2u : (F == FMT_INT4 ? 2u * nseg_row : (uint32_t)nseg_row);
        const uint32_t ssz = F == FMT_INT2 ? 2u : (F == FMT_INT4 ? 2u : 1u);  // bytes per scale
#pragma unroll
        for (int t = 0; t < NMAT; ++t) {
            rw[t] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(wq[t]), 0,
                                                     (uint32_t)N * row_bytes, 0x00020000);
            rsc[t] = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(sc[t]), 0,
                                                      (uint32_t)N * srow, 0x00020000);
        }
        const uint32_t n0 = (uint32_t)first * R * RPG + rsub;
        woff = n0 * row_bytes + (uint32_t)(seg0 + q) * 16u;
        soff = n0 * srow + (kRowScale<F> ? 0u : (uint32_t)(seg0 + q) * ssz);
        wstep = (uint32_t)stride * R * RPG * row_bytes;
        sstep = (uint32_t)stride * R * RPG * srow;
    }

    // Byte offset of slot i's load (weights: step 16, scales: step ssz) from
    // `base`; a slot past the row end (j = q + RL*i >= nseg) gets an offset
    // past the end of the buffer, so it reads zeros and costs no memory
    // traffic (its value is the tree's +0 padding anyway).  With the lane
    // layouts pick_shape chooses, every slot below kSureLive is inside the
    // row for every lane, so only the last slots need the test.
    static constexpr int kSureLive = NI == 1 ? 0 : (NI == 8 ? 4 : NI - 1);
    __device__ __forceinline__ uint32_t slot_off(uint32_t base, int i, uint32_t step) const {
        const uint32_t c = (uint32_t)(i * RL) * step;
        if (i < kSureLive) return base + c;
        // select the base, then add the constant, which then fits the load's
        // immediate offset field: one v_cndmask per load and no add
        uint32_t b = q + RL * i < nseg ? base : kLoadOob - c;
        asm volatile("" : "+v"(b));
        return b + c;
    }

    // Issue the loads of the next unit in this wave's sequence into `sl`.
    // Loads are unconditional (the compiler can then count outstanding loads
    // exactly); slots past a row's end load zeros (slot_off).
    __device__ __forceinline__ void load(RowSlot<F, NI, NMAT, R> &sl) {
        constexpr uint32_t ssz = F == FMT_INT2 ? 2u : (F == FMT_INT4 ? 2u : 1u);
#pragma unroll
        for (int t = 0; t < NMAT; ++t)
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t wo = woff + (uint32_t)r * RPG * row_bytes;
                const uint32_t so = soff + (uint32_t)r * RPG * srow;
                if constexpr (kRowScale<F>) sl.rs[t][r] = __builtin_amdgcn_raw_buffer_load_b16(rsc[t], so, 0, 0);
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    sl.w[t][r][i] = __builtin_bit_cast(
                        u4_t, __builtin_amdgcn_raw_buffer_load_b128(rw[t], slot_off(wo, i, 16u), 0, kNT));
                    if constexpr (F == FMT_INT4)
                        sl.seg[t][r][i] = __builtin_amdgcn_raw_buffer_load_b16(rsc[t], slot_off(so, i, ssz), 0, 0);
                    else if constexpr (F == FMT_MXFP4)
                        sl.seg[t][r][i] = __builtin_amdgcn_raw_buffer_load_b8(rsc[t], slot_off(so, i, ssz), 0, 0);
                }
            }
        woff += wstep;
        soff += sstep;
    }

    // Issue the loads of segment i of the unit at (woff, soff) into `s`;
    // after the last segment the offsets move to the wave's next unit.
    __device__ __forceinline__ void load_seg(SegSlot &s, int i) {
        constexpr uint32_t ssz = F == FMT_INT2 ? 2u : (F == FMT_INT4 ? 2u : 1u);
#pragma unroll
        for (int t = 0; t < NMAT; ++t) {
            if constexpr (kRowScale<F>)
                if (i == 0) s.rs[t] = __builtin_amdgcn_raw_buffer_load_b16(rsc[t], soff, 0, 0);
            s.w[t] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(rw[t], slot_off(woff, i, 16u), 0, kNT));
            if constexpr (F == FMT_INT4)
                s.sb[t] = __builtin_amdgcn_raw_buffer_load_b16(rsc[t], slot_off(soff, i, ssz), 0, 0);
            else if constexpr (F == FMT_MXFP4)
                s.sb[t] = __builtin_amdgcn_raw_buffer_load_b8(rsc[t], slot_off(soff, i, ssz), 0, 0);
        }
        if (i == NI - 1) {
            woff += wstep;
            soff += sstep;
        }
    }

    __device__ __forceinline__ void prefetch() {
        if constexpr (kStream) {
#pragma unroll
            for (int g = 0; g < NS; ++g) load_seg(ss[g], g % NI);
        } else {
#pragma unroll
            for (int d = 0; d < D; ++d) load(slot[d]);
        }
    }

    // The scaled sum of one segment (the int2 row scale comes at the end).
    __device__ __forceinline__ float scaled(float t, uint32_t sbits) const {
        if constexpr (kRowScale<F>) return t;
        else if constexpr (F == FMT_INT4) return seg_scale<F>(sbits) * t;
        else return t * seg_scale<F>(sbits);
    }

    // Pad the scaled segment sums past the row end (+0), then reduce.
    __device__ __forceinline__ float reduce_scaled(const float (&val)[NI]) const {
        float v[NIP];
#pragma unroll
        for (int a = 0; a < NIP; ++a) v[a] = (a < NI && q + RL * a < nseg) ? val[a] : 0.0f;
        return fo_tree<RL, NIP>(v, P2);
    }

    // Scale the segment sums and pad past the row end (+0), then reduce.
    __device__ __forceinline__ float finish(const float (&seg)[NI], const uint32_t (&sbits)[NI]) const {
        float v[NIP];
#pragma unroll
        for (int a = 0; a < NIP; ++a) {
            float val = 0.0f;
            if (a < NI) {
                if constexpr (kRowScale<F>) val = seg[a];
                else if constexpr (F == FMT_INT4) val = seg_scale<F>(sbits[a]) * seg[a];
                else val = seg[a] * seg_scale<F>(sbits[a]);
                // segments past the row end are the tree's +0 padding
                val = (q + RL * a < nseg) ? val : 0.0f;
            }
            v[a] = val;
        }
        return fo_tree<RL, NIP>(v, P2);
    }

    // MXFP4 with the activation slice in registers holds it widened to fp32
    // (twice the registers): the inner step is then one conversion per two
    // codes and one fused multiply-add per code, with no per-code widening.
    static constexpr bool kXf32 = F == FMT_MXFP4 && XREG && QMV_MX_XF32;

    template <class Epi>
    __device__ __forceinline__ void run_stream(const uint16_t *xs, Epi &epi) {
        DecodeConsts kc;
        u4_t xr[XREG && !kXf32 ? NI : 1][XREG && !kXf32 ? XV : 1];
        float xw[kXf32 ? NI : 1][kXf32 ? CODES : 1];
        int xoff[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int j = q + RL * i;
            xoff[i] = (j < nseg ? j : nseg - 1) * CODES;
            if constexpr (kXf32) {
#pragma unroll
                for (int v = 0; v < XV; ++v) {
                    const u4_t p = (j < nseg) ? *reinterpret_cast<const u4_t *>(xs + j * CODES + 8 * v)
                                              : u4_t{0u, 0u, 0u, 0u};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        xw[i][8 * v + e] = (e & 1) ? u2f(p[e >> 1] & 0xFFFF0000u) : u2f(p[e >> 1] << 16);
                }
            } else if constexpr (XREG) {
#pragma unroll
                for (int v = 0; v < XV; ++v)
                    xr[i][v] = (j < nseg) ? *reinterpret_cast<const u4_t *>(xs + j * CODES + 8 * v)
                                          : u4_t{0u, 0u, 0u, 0u};
            }
        }
        for (int base = first; base < total_units; base += NU * stride) {
#pragma unroll
            for (int uu = 0; uu < NU; ++uu) {
                const int u = base + uu * stride;
                float val[NMAT][NI];
                uint32_t rsb[NMAT];
                float segdep = 0.0f;
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    SegSlot &s = ss[(uu * NI + i) % NS];
                    if (u < total_units) {  // uniform across the wave
                        // keep the activations opaque to loop-invariant code
                        // motion (see the unit-ring path)
                        if constexpr (kXf32) {
#pragma unroll
                            for (int k = 0; k < CODES; ++k) asm volatile("" : "+v"(xw[i][k]));
                        } else if constexpr (XREG) {
#pragma unroll
                            for (int v = 0; v < XV; ++v) asm volatile("" : "+v"(xr[i][v]));
                        } else {
                            asm volatile("" : "+v"(xoff[i]));
                        }
                        // the NMAT matrices are independent chains over the
                        // same activations
                        float a[NMAT][1];
#pragma unroll
                        for (int t = 0; t < NMAT; ++t) a[t][0] = 0.0f;
                        // segment i's words become available only once segment
                        // i-1 is summed: left free, the scheduler decodes the
                        // unit's later segments first, and the wave then waits
                        // for its newest loads at the top of every unit
                        if (i > 0) {
#pragma unroll
                            for (int t = 0; t < NMAT; ++t)
#pragma unroll
                                for (int v = 0; v < 4; ++v) asm volatile("" : "+v"(s.w[t][v]) : "v"(segdep));
                        }
                        if constexpr (kXf32)
                            mx_sums_f32<NMAT>(s.w, [&](int, int k) { return xw[i][k]; }, a);
                        else if constexpr (XREG)
                            segment_sums<F, NMAT, 1>(s.w, kc, [&](int, int, int vv) { return xr[i][vv]; }, a);
                        else
                            segment_sums<F, NMAT, 1>(
                                s.w, kc,
                                [&](int, int, int vv) {
                                    return *reinterpret_cast<const u4_t *>(xs + xoff[i] + 8 * vv);
                                },
                                a);
                        segdep = a[0][0];
#pragma unroll
                        for (int t = 0; t < NMAT; ++t) {
                            val[t][i] = scaled(a[t][0], s.sb[t]);
                            if (i == 0) rsb[t] = kRowScale<F> ? s.rs[t] : 0u;
                        }
                    }
                    // refill with the same segment of the unit NS segments on
                    // (unconditional: past the end the loads return zeros)
                    load_seg(s, i);
                }
                if (u < total_units) {
                    float tot[1][NMAT][1];
                    float rs[NMAT];
#pragma unroll
                    for (int t = 0; t < NMAT; ++t) {
                        tot[0][t][0] = reduce_scaled(val[t]);
                        rs[t] = half_bits_to_f32((uint16_t)rsb[t]);
                    }
                    epi(u * RPG + rsub, q, tot[0], rs);
                }
            }
        }
    }

    template <class Epi>
    __device__ __forceinline__ void run(const uint16_t *xs, Epi &epi) {
        if constexpr (kStream) {
            run_stream(xs, epi);
            return;
        }
        DecodeConsts kc;
        // x slice of this lane: segments q + RL*i (zeros past the row end)
        u4_t xr[XREG ? NI : 1][XREG ? MC : 1][XREG ? XV : 1];
        if constexpr (XREG) {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int j = q + RL * i;
#pragma unroll
                for (int m = 0; m < MC; ++m)
#pragma unroll
                    for (int v = 0; v < XV; ++v)
                        xr[i][m][v] = (j < nseg) ? *reinterpret_cast<const u4_t *>(
                                                       xs + (size_t)m * K + j * CODES + 8 * v)
                                                 : u4_t{0u, 0u, 0u, 0u};
            }
        }
        int xoff[NI];  // LDS offset of each segment's activations (clamped)
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int j = q + RL * i;
            xoff[i] = (j < nseg ? j : nseg - 1) * CODES;
        }
        for (int base = first; base < total_units; base += NSLOT * stride) {
#pragma unroll
            for (int d = 0; d < NSLOT; ++d) {
                const int u = base + d * stride;
                // slot d holds unit u; refill-first loads unit u + D*stride
                // into the slot that was computed last
                if constexpr (kRefillFirst) load(slot[(d + D) % NSLOT]);
                const RowSlot<F, NI, NMAT, R> &cur = slot[d];
                if (u < total_units) {  // uniform across the wave
                    if constexpr (XREG) {
                        // keep the register copy of x opaque to loop-invariant
                        // code motion (it would hoist fp16->fp32 conversions
                        // and double the registers x occupies)
#pragma unroll
                        for (int i = 0; i < NI; ++i)
#pragma unroll
                            for (int m = 0; m < MC; ++m)
#pragma unroll
                                for (int v = 0; v < XV; ++v) asm volatile("" : "+v"(xr[i][m][v]));
                    } else {
                        // the LDS copy of x never changes, so the compiler
                        // would hoist every read (and a widening of it) out of
                        // the row loop and run out of registers; opaque
                        // offsets keep the reads here
#pragma unroll
                        for (int i = 0; i < NI; ++i) asm volatile("" : "+v"(xoff[i]));
                    }
                    float tot[R][NMAT][MC];
                    // expanded at compile time: with two matrices and eight
                    // segments per lane the body is past the unroller's size
                    // limit, and a rolled loop would index register arrays
                    // at run time (scratch memory)
                    static_for<NMAT>([&](auto tc) {
                        constexpr int t = decltype(tc)::value;
                        float acc[R][MC][NI];
                        if constexpr (R == 1 && MC == 1) {
                            // one row, one column: the lane's segments are the
                            // independent chains, advanced together
                            float a1[NI][1];
#pragma unroll
                            for (int i = 0; i < NI; ++i) a1[i][0] = 0.0f;
                            if constexpr (XREG)
                                segment_sums<F, NI, 1>(cur.w[t][0], kc,
                                                       [&](int a, int m, int vv) { return xr[a][m][vv]; }, a1);
                            else
                                segment_sums<F, NI, 1>(
                                    cur.w[t][0], kc,
                                    [&](int a, int m, int vv) {
                                        return *reinterpret_cast<const u4_t *>(xs + xoff[a] + 8 * vv);
                                    },
                                    a1);
#pragma unroll
                            for (int i = 0; i < NI; ++i) acc[0][0][i] = a1[i][0];
                        } else {
                            // rows x columns are the independent chains;
                            // segments go one after another so only one
                            // segment's codes and activations are live
                            static_for<NI>([&](auto ic) {
                                constexpr int i = decltype(ic)::value;
                                u4_t wr[R];
#pragma unroll
                                for (int r = 0; r < R; ++r) wr[r] = cur.w[t][r][i];
                                float ar[R][MC];
#pragma unroll
                                for (int r = 0; r < R; ++r)
#pragma unroll
                                    for (int m = 0; m < MC; ++m) ar[r][m] = 0.0f;
                                segment_sums_rows<F, R, MC>(wr, kc, xs, xoff[i], K, ar);
#pragma unroll
                                for (int r = 0; r < R; ++r)
#pragma unroll
                                    for (int m = 0; m < MC; ++m) acc[r][m][i] = ar[r][m];
                                // keep the next segment's LDS reads from being
                                // scheduled ahead of this one (register budget)
                                __builtin_amdgcn_sched_barrier(0);
                            });
                        }
#pragma unroll
                        for (int r = 0; r < R; ++r)
#pragma unroll
                            for (int m = 0; m < MC; ++m) tot[r][t][m] = finish(acc[r][m], cur.seg[t][r]);
                    });
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        float rs[NMAT];
#pragma unroll
                        for (int t = 0; t < NMAT; ++t) rs[t] = half_bits_to_f32((uint16_t)cur.rs[t][r]);
                        epi((u * R + r) * RPG + rsub, q, tot[r], rs);
                    }
                }
                if constexpr (!kRefillFirst) load(slot[d]);
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Plain matvec / skinny GEMM.
// Stores y (fixed order), or, in split-K mode, the split's partial sum
// before the int2 row scale into part[m][n].
template <int F, int MC>
struct StoreEpi {
    OutBuf out;    // y, or this split's fp32 partial sums
    bool partial;  // uniform
    int M, N, m0;
    __device__ __forceinline__ void operator()(int n, int q, const float (&tot)[1][MC],
                                               const float (&rs)[1]) {
        const float s = rs[0];
        const bool act = q == 0 && n < N;
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            if (m0 + m < M) {  // uniform
                float r = tot[0][m];
                if constexpr (kRowScale<F>)
                    if (!partial) r = s * r;
                out.put(act, (uint32_t)((m0 + m) * N + n), r);
            }
        }
    }
};

// blockIdx.z selects a K split of seg_split segments (one split covering the
// whole row in fixed-order mode, part == nullptr); split z writes its partial
// sums to part + z*M*N.
template <int F, int RL, int NI, int NIP, int MC, bool XREG, int WV = kWaves>
__global__ __launch_bounds__(64 * WV) void k_fo_matvec(const uint8_t *__restrict__ wq,
                                                      const void *__restrict__ sc,
                                                      const uint16_t *__restrict__ x, void *y,
                                                      int y_dtype, int M, int N, int K, int seg_split,
                                                      float *part) {
    extern __shared__ __align__(16) uint16_t xs[];
    constexpr int CODES = SegCodes<F>::v;
    const int m0 = blockIdx.y * MC;
    // a ternary row is padded to whole segments; codes past K meet x = 0
    const int nseg_row = (K + CODES - 1) / CODES;
    const int seg0 = blockIdx.z * seg_split;
    const int nloc = nseg_row - seg0 < seg_split ? nseg_row - seg0 : seg_split;
    const int klen = nloc * CODES;
    const int kval = K - seg0 * CODES < klen ? K - seg0 * CODES : klen;  // real activations staged
    const uint16_t *xz = x + (size_t)seg0 * CODES;
    const uint8_t *const w1[1] = {wq};
    const void *const s1[1] = {sc};
    FoEngine<F, RL, NI, NIP, MC, XREG, 1, ring_depth<NI, 1>(), rows_block<MC, XREG, F>(), WV> eng(
        w1, s1, N, klen, seg0, nseg_row);
    XStage<MC> xst;
    xst.load(xz, M, K, klen, m0, kval);
    eng.prefetch();
    xst.store(xz, xs, M, K, klen, m0, kval);
    __syncthreads();
    StoreEpi<F, MC> epi{OutBuf(part == nullptr ? y : static_cast<void *>(part + (size_t)blockIdx.z * M * N),
                               (uint32_t)M * (uint32_t)N, part == nullptr ? y_dtype : 0),
                        part != nullptr, M, N, m0};
    eng.run(xs, epi);
}

// Split-K reduction: y[m][n] = (int2 row scale) * sum over z = 0 .. S-1 of
// part[z][m][n], summed in increasing z.
__global__ void k_splitk_reduce(const float *__restrict__ part, int S, int M, int N,
                                const uint16_t *__restrict__ rscale, void *y, int y_dtype) {
    const size_t total = (size_t)M * N;
    for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
        float acc = part[e];
        for (int z = 1; z < S; ++z) acc = acc + part[(size_t)z * total + e];
        if (rscale != nullptr) acc = half_bits_to_f32(rscale[e % N]) * acc;
        store_out(y, e, acc, y_dtype);
    }
}

// ---------------------------------------------------------------------------
// Fused residual-add + RMSNorm prologue -> dual int2 gate/up -> GELU*up.
// Every workgroup recomputes the prologue for its activation chunk (identical
// arithmetic everywhere); workgroup (0, y) writes residual_out.

template <int MC>
__device__ void rmsnorm_prologue(const uint16_t *__restrict__ x, const uint16_t *__restrict__ res,
                                 const uint16_t *__restrict__ gamma, uint16_t *res_out, float eps,
                                 int M, int K, int m0, uint16_t *hs, uint16_t *xs, float *inv_s) {
    // h = fp16(x + r): one fp16 addition, correctly rounded.
    for (int e = threadIdx.x; e < MC * K; e += blockDim.x) {
        const int m = e / K, k = e - m * K;
        _Float16 h = (_Float16)0.0f;
        if (m0 + m < M) {
            const size_t g = (size_t)(m0 + m) * K + k;
            const _Float16 a = __builtin_bit_cast(_Float16, x[g]);
            const _Float16 b = __builtin_bit_cast(_Float16, res[g]);
            h = a + b;
            if (res_out != nullptr && blockIdx.x == 0) res_out[g] = __builtin_bit_cast(uint16_t, h);
        }
        hs[e] = __builtin_bit_cast(uint16_t, h);
    }
    __syncthreads();
    // sum of squares in the fixed order (64-element segments, halving tree),
    // one wave per activation row.
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nseg = K / 64;
    const int P2 = [nseg] {
        int p = 1;
        while (p < nseg) p <<= 1;
        return p;
    }();
    for (int m = wave; m < MC; m += kWaves) {
        constexpr int NIPP = 4;  // K <= 16384: at most 256 segments = 64 lanes x 4
        float v[NIPP];
#pragma unroll
        for (int a = 0; a < NIPP; ++a) {
            const int j = lane + 64 * a;
            float t = 0.0f;
            if (j < nseg) {
                const uint16_t *hp = hs + (size_t)m * K + 64 * j;
                for (int k = 0; k < 64; ++k) {
                    const float hf = half_bits_to_f32(hp[k]);
                    const float sq = hf * hf;  // exact
                    t = t + sq;
                }
            }
            v[a] = t;
        }
        const float ss = fo_tree<64, NIPP>(v, P2);
        if (lane == 0) {
            const float ms = ss / (float)K;
            const float r = ms + eps;
            const float root = __builtin_sqrtf(r);
            inv_s[m] = 1.0f / root;
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < MC * K; e += blockDim.x) {
        const int m = e / K, k = e - m * K;
        const float hf = half_bits_to_f32(hs[e]);
        const float a = hf * inv_s[m];
        const float b = a * half_bits_to_f32(gamma[k]);
        xs[e] = __builtin_bit_cast(uint16_t, to_f16(b));
    }
    __syncthreads();
}

// The same prologue for one activation row per workgroup (M = 1 decode),
// in two phases so that the global loads of x,
// the residual and gamma are issued before the weight prefetch (vector loads
// retire in issue order: loaded after the weights, the prologue would wait
// for them).  load(): every thread takes one 16-byte vector of x, r and
// gamma (K <= 2048; longer rows load the rest in finish()).  finish():
// h = fp16(x + r) to LDS (and residual_out from workgroup 0), then wave 0
// sums the exact squares segment by segment (64 values, k order) and reduces
// the segment sums with the fixed tree, then every thread normalises its
// vectors in place: xn = fp16((fl32(h) * inv) * fl32(gamma)).
struct RmsStage1 {
    u4_t xv, rv, gv;
    __device__ __forceinline__ void load(const uint16_t *__restrict__ x, const uint16_t *__restrict__ res,
                                         const uint16_t *__restrict__ gamma, int K, int m) {
        const int v = threadIdx.x, nvec = K / 8;
        const size_t row = (size_t)m * K;
        xv = rv = gv = u4_t{0u, 0u, 0u, 0u};
        if (v < nvec) {
            xv = *reinterpret_cast<const u4_t *>(x + row + 8 * v);
            rv = *reinterpret_cast<const u4_t *>(res + row + 8 * v);
            gv = *reinterpret_cast<const u4_t *>(gamma + 8 * v);
        }
    }
    __device__ static u4_t hsum(const u4_t &a, const u4_t &b) {
        u4_t h;
#pragma unroll
        for (int e = 0; e < 4; ++e)  // h = fp16(x + r), one rounding per element
            h[e] = __builtin_bit_cast(uint32_t, u2h2(a[e]) + u2h2(b[e]));
        return h;
    }
    __device__ static u4_t normalise(const u4_t &hv, const u4_t &g, float inv) {
        u4_t o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const h2_t hh = u2h2(hv[e]), gg = u2h2(g[e]);
            const float a0 = (float)hh.x * inv, a1 = (float)hh.y * inv;
            const float b0 = a0 * (float)gg.x, b1 = a1 * (float)gg.y;
            const uint32_t lo = __builtin_bit_cast(uint16_t, to_f16(b0));
            const uint32_t hi = __builtin_bit_cast(uint16_t, to_f16(b1));
            o[e] = lo | (hi << 16);
        }
        return o;
    }
    __device__ __forceinline__ void finish(const uint16_t *__restrict__ x, const uint16_t *__restrict__ res,
                                           const uint16_t *__restrict__ gamma, uint16_t *res_out, float eps,
                                           int K, int m, uint16_t *xs, float *inv_s) {
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        const int nvec = K / 8;
        const size_t row = (size_t)m * K;
        const bool write_res = res_out != nullptr && blockIdx.x == 0;
        for (int v = tid; v < nvec; v += kBlock) {
            const u4_t h = v == tid ? hsum(xv, rv)
                                    : hsum(*reinterpret_cast<const u4_t *>(x + row + 8 * v),
                                           *reinterpret_cast<const u4_t *>(res + row + 8 * v));
            *reinterpret_cast<u4_t *>(xs + 8 * v) = h;
            if (write_res) *reinterpret_cast<u4_t *>(res_out + row + 8 * v) = h;
        }
        __syncthreads();
        if (wave == 0) {
            const int nseg = K / 64;
            int P2 = 1;
            while (P2 < nseg) P2 <<= 1;
            constexpr int NIPP = 4;  // K <= 16384: at most 256 segments = 64 lanes x 4
            float sv[NIPP];
#pragma unroll
            for (int a = 0; a < NIPP; ++a) {
                const int j = lane + 64 * a;
                float t = 0.0f;
                if (j < nseg) {
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const u4_t hv = *reinterpret_cast<const u4_t *>(xs + 64 * j + 8 * q);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const h2_t hh = u2h2(hv[e]);
                            const float h0 = (float)hh.x, h1 = (float)hh.y;
                            t = t + h0 * h0;  // squares exact in fp32; k order
                            t = t + h1 * h1;
                        }
                    }
                }
                sv[a] = t;
            }
            const float ss = fo_tree<64, NIPP>(sv, P2);
            if (lane == 0) {
                const float ms = ss / (float)K;
                const float r = ms + eps;
                const float root = __builtin_sqrtf(r);
                inv_s[0] = 1.0f / root;
            }
        }
        __syncthreads();
        const float inv = inv_s[0];
        for (int v = tid; v < nvec; v += kBlock) {
            const u4_t g = v == tid ? gv : *reinterpret_cast<const u4_t *>(gamma + 8 * v);
            const u4_t hv = *reinterpret_cast<const u4_t *>(xs + 8 * v);
            *reinterpret_cast<u4_t *>(xs + 8 * v) = normalise(hv, g, inv);
        }
        __syncthreads();
    }
};

// QM (quantised output): 0 none, the fp16 output goes to `out`; 1 the fp16
// values go to this workgroup's LDS staging area (its 32-row blocks, see
// mxfp4_local); 2 they go to `out` (the workspace staging area) for
// mxfp4_tail.
template <int MC, int QM = 0>
struct GateUpEpi {
    OutBuf out;  // fp16 [M][N]
    int M, N, m0;
    uint16_t *stage = nullptr;  // QM == 1: [slots][MC] fp16 bits
    int bpr = 1;                // QM == 1: 32-row blocks per workgroup round
    __device__ __forceinline__ void operator()(int n, int q, const float (&tot)[2][MC],
                                               const float (&rs)[2]) {
        const float sg = rs[0];
        const float su = rs[1];
        const bool act = q == 0 && n < N;
        int slot = 0;
        if constexpr (QM == 1) {
            // block b = n / 32 lies in round r = (b / bpr - blockIdx.x) / gridDim.x of this workgroup
            const int b = n >> 5;
            const int r = (b / bpr - (int)blockIdx.x) / (int)gridDim.x;
            slot = (r * bpr + b % bpr) * 32 + (n & 31);
        }
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            if (m0 + m < M) {  // uniform
                const float g = sg * tot[0][m];
                const float u = su * tot[1][m];
                const float ge = qmv_gelu(g);
                const float o = ge * u;
                if constexpr (QM == 1) {
                    if (act) stage[slot * MC + m] = __builtin_bit_cast(uint16_t, to_f16(o));
                } else {
                    out.put(act, (uint32_t)((m0 + m) * N + n), o);
                }
            }
        }
    }
};

// Workgroup-local quantisation (QM == 1): with kWaves * (rows per unit) a
// multiple of 32, round r of workgroup g covers the whole 32-row blocks
// (g + r * G) * bpr + j, j < bpr (G workgroups), so after its last unit the
// workgroup holds every value of its blocks in LDS and quantises them there:
// no other workgroup is involved and nothing waits across the grid.
template <int MC>
__device__ __forceinline__ void mxfp4_local(const uint16_t *stage, int rounds, int bpr, uint8_t *qcodes,
                                            uint8_t *qscale, int M, int N, int m0) {
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nb = N / 32, total = rounds * bpr * MC;
    for (int t0 = 2 * wave; t0 < total; t0 += 2 * kWaves) {  // two blocks per wave
        const int t = t0 + (lane >> 5);
        const int m = t % MC, rj = t / MC;  // rj = r * bpr + j
        const int b = ((int)blockIdx.x + (rj / bpr) * (int)gridDim.x) * bpr + rj % bpr;
        const bool live = t < total && b < nb && m0 + m < M;
        const uint16_t h = live ? stage[(rj * 32 + (lane & 31)) * MC + m] : (uint16_t)0;
        const size_t row = live ? (size_t)(m0 + m) : 0;
        mx_quant_half(h, live, qcodes + row * (N / 2) + (size_t)b * 16, qscale + row * nb + b);
    }
}

// Fused activation-and-quantize ("Gemma 4 Optimization with Agentic Kernel
// Engineering", "What it found"), for lane layouts whose workgroup rounds do
// not cover whole 32-row blocks: the fp16 outputs go to the workspace; after
// its units the workgroup makes them visible (each wave completes its
// stores, a barrier, then one agent-scope release by wave 0), and wave 0
// adds one arrival per unit of the workgroup to the unit's 32-row block.
// The arrival that brings a block's count to 32 / (rows per unit) takes an
// acquire fence, quantises the block from the staged fp16 values and resets
// the counter to zero for the next call.  No workgroup waits for another.
template <int MC, class Eng>
__device__ __forceinline__ void mxfp4_tail(const Eng &eng, const uint16_t *stage, uint8_t *qcodes,
                                           uint8_t *qscale, uint32_t *qcnt, int M, int N, int m0) {
    constexpr uint32_t kArrivals = 32 / Eng::kRowsPerUnit;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nblk = N / 32;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (wave != 0) return;  // no barrier follows
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    // wave 0's units are the first of each round of the workgroup's kWaves
    // consecutive units; lane t < kWaves * MC adds the arrival of unit
    // u0 + t / MC, activation row t % MC (all in flight at once)
    for (int u0 = eng.first; u0 < eng.total_units; u0 += eng.stride) {
        const int tw = lane / MC, tm = lane % MC;
        const int tu = u0 + tw;
        const bool valid = lane < kWaves * MC && tu < eng.total_units && m0 + tm < M;
        uint32_t old = 0;
        if (valid)
            old = __hip_atomic_fetch_add(&qcnt[(size_t)(m0 + tm) * nblk + tu * Eng::kRowsPerUnit / 32], 1u,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        uint64_t last = __ballot(valid && old == kArrivals - 1);
        while (last != 0) {  // uniform
            const int t = __builtin_ctzll(last);
            last &= last - 1;
            const int m = t % MC, blk = (u0 + t / MC) * Eng::kRowsPerUnit / 32;
            const size_t c = (size_t)(m0 + m) * nblk + blk;
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            const uint16_t h = lane < 32 ? stage[(size_t)(m0 + m) * N + (size_t)blk * 32 + lane] : (uint16_t)0;
            mx_quant_half(h, lane < 32, qcodes + (size_t)(m0 + m) * (N / 2) + (size_t)blk * 16, qscale + c);
            if (lane == 0) __hip_atomic_store(&qcnt[c], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int RL, int NI, int NIP, int MC, bool XREG, int QM>
__global__ __launch_bounds__(kBlock) void k_fo_gateup(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ residual,
    uint16_t *residual_out, const uint16_t *__restrict__ gamma, float eps,
    const uint32_t *__restrict__ wq_gate, const uint16_t *__restrict__ s_gate,
    const uint32_t *__restrict__ wq_up, const uint16_t *__restrict__ s_up, uint16_t *out, int M,
    int N, int K, uint8_t *qcodes, uint8_t *qscale, uint32_t *qcnt, int qrounds) {
    extern __shared__ __align__(16) uint16_t smem[];
    uint16_t *xs = smem;  // [MC][K]: h, then overwritten in place by the normalised xn
    float *inv_s = reinterpret_cast<float *>(smem + (size_t)MC * K);
    const int m0 = blockIdx.y * MC;
    const uint8_t *const w2[2] = {reinterpret_cast<const uint8_t *>(wq_gate),
                                  reinterpret_cast<const uint8_t *>(wq_up)};
    const void *const s2[2] = {s_gate, s_up};
    FoEngine<FMT_INT2, RL, NI, NIP, MC, XREG, 2, ring_depth<NI, 2>(), rows_block<MC, XREG>()> eng(w2, s2, N, K);
    if constexpr (MC == 1) {
        RmsStage1 rs1;
        rs1.load(x, residual, gamma, K, m0);
        eng.prefetch();
        rs1.finish(x, residual, gamma, residual_out, eps, K, m0, xs, inv_s);
    } else {
        eng.prefetch();
        rmsnorm_prologue<MC>(x, residual, gamma, residual_out, eps, M, K, m0, xs, xs, inv_s);
    }
    using Eng = decltype(eng);
    GateUpEpi<MC, QM> epi{OutBuf(out, (uint32_t)M * (uint32_t)N, 1), M, N, m0};
    constexpr int kBpr = kWaves * Eng::kRowsPerUnit / 32;
    uint16_t *stage = reinterpret_cast<uint16_t *>(inv_s + 16 * MC);  // after the prologue's scratch
    if constexpr (QM == 1) {
        static_assert((kWaves * Eng::kRowsPerUnit) % 32 == 0, "workgroup rounds must cover whole blocks");
        epi.stage = stage;
        epi.bpr = kBpr;
    }
    eng.run(xs, epi);
    if constexpr (QM == 1) mxfp4_local<MC>(stage, qrounds, kBpr, qcodes, qscale, M, N, m0);
    if constexpr (QM == 2) mxfp4_tail<MC>(eng, out, qcodes, qscale, qcnt, M, N, m0);
}

// ---------------------------------------------------------------------------
// int2 lm_head + argmax, one dispatch ("The parked levers": argmax stages 1
// and 2 merged, first-max tie-break kept).  Each lane keeps the best key of
// the rows it produced; the workgroup reduces them and folds its best key per
// activation row into a 64-bit key in the workspace with an agent-scope
// atomic max (order-independent, so the result is exact).  Only after those
// atomics have returned does the workgroup take a ticket from the completion
// counter; the workgroup that
// takes the last ticket reads each key with an atomic exchange (which also
// resets it to zero), writes idx / maxval and resets the counter, leaving the
// workspace zeroed for the next call.
template <int MC>
struct ArgmaxEpi {
    float *logits;
    int M, N, m0;
    uint64_t best[MC];
    __device__ __forceinline__ void operator()(int n, int q, const float (&tot)[1][MC],
                                               const float (&rs)[1]) {
        const float s = rs[0];
        if (q != 0 || n >= N) return;
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            const float yv = s * tot[0][m];
            if (logits != nullptr && m0 + m < M) logits[(size_t)(m0 + m) * N + n] = yv;
            const uint64_t k = argmax_key(yv, n);
            best[m] = k > best[m] ? k : best[m];
        }
    }
};

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
        const uint64_t o = __shfl_xor(v, s, 64);
        v = o > v ? o : v;
    }
    return v;
}

template <int RL, int NI, int NIP, int MC, bool XREG>
__global__ __launch_bounds__(kBlock) void k_fo_argmax(const uint32_t *__restrict__ wq,
                                                      const uint16_t *__restrict__ scale,
                                                      const uint16_t *__restrict__ x, int32_t *idx,
                                                      float *maxval, float *logits, int M, int N,
                                                      int K, uint64_t *keys, uint32_t *counter) {
    extern __shared__ __align__(16) uint16_t xs[];
    __shared__ uint64_t wbest[kWaves][MC];
    __shared__ uint64_t returned[MC];
    __shared__ int is_last;
    const int m0 = blockIdx.y * MC;
    const uint8_t *const w1[1] = {reinterpret_cast<const uint8_t *>(wq)};
    const void *const s1[1] = {scale};
    FoEngine<FMT_INT2, RL, NI, NIP, MC, XREG, 1, ring_depth<NI, 1>(), rows_block<MC, XREG>()> eng(w1, s1, N, K);
    XStage<MC> xst;
    xst.load(x, M, K, K, m0);
    eng.prefetch();
    xst.store(x, xs, M, K, K, m0);
    __syncthreads();
    ArgmaxEpi<MC> epi{logits, M, N, m0, {}};
#pragma unroll
    for (int m = 0; m < MC; ++m) epi.best[m] = 0ull;
    eng.run(xs, epi);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int m = 0; m < MC; ++m) {
        const uint64_t b = wave_max_u64(epi.best[m]);
        if (lane == 0) wbest[wave][m] = b;
    }
    __syncthreads();
    if (threadIdx.x < MC && m0 + (int)threadIdx.x < M) {
        uint64_t b = 0;
        for (int w = 0; w < kWaves; ++w) b = wbest[w][threadIdx.x] > b ? wbest[w][threadIdx.x] : b;
        // the returned value is consumed (written to LDS) before the barrier,
        // so every key update of this workgroup has been performed before the
        // ticket below is taken
        returned[threadIdx.x] = __hip_atomic_fetch_max(&keys[m0 + threadIdx.x], b, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        // Relaxed on purpose.  The key updates and the final exchanges are
        // agent-scope atomic read-modify-writes, performed at the device's
        // coherence point in the order they reach it; a workgroup asks for
        // its ticket only after its key updates have returned (their values
        // are consumed before the barrier), and the last workgroup issues its
        // exchanges only after its ticket has returned, so every update is
        // performed before the exchange that reads it.  No ordinary store
        // needs publishing.  (An acquire-release ticket would also give the
        // language-level ordering, but at agent scope it writes back the
        // XCD's L2 once per workgroup: measured 56 vs 36 us per call on the
        // N=262144 lm_head.)
        const uint32_t ticket = __hip_atomic_fetch_add(&counter[blockIdx.y], 1u, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
        is_last = (ticket == gridDim.x - 1) ? 1 : 0;
    }
    __syncthreads();
    if (!is_last) return;
    if (threadIdx.x < MC && m0 + (int)threadIdx.x < M) {
        const uint64_t b = __hip_atomic_exchange(&keys[m0 + threadIdx.x], 0ull, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
        int n;
        float yv;
        argmax_key_decode(b, n, yv);
        idx[m0 + threadIdx.x] = n;
        if (maxval != nullptr) maxval[m0 + threadIdx.x] = yv;
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&counter[blockIdx.y], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void k_fill_zero(uint32_t *p, size_t words) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Host launchers.

// Workgroups for N rows: enough waves that each has about `depth` row
// groups (its ring filled once), but no more than can be resident on the
// device at once (occupancy x CUs), so every workgroup starts in the first
// wave of the launch and none waits for a free CU.
//
// `per_cu` (if > 0) caps the resident workgroups per CU below what occupancy
// allows.  A full launch then has the same number of workgroups on every CU.
template <class Kern>
static int grid_for(Kern kernel, size_t lds, long N, int RL, int depth, int per_cu = 0, int block = kBlock) {
    const int rpg = 64 / RL;
    const int waves = block / 64;
    const long total_rg = ((long)N + rpg - 1) / rpg;
    long g = (total_rg + (long)waves * depth - 1) / ((long)waves * depth);
    const int cus = device_cus();
    int occ = cached_occupancy(kernel, block, lds);
    if (per_cu > 0 && occ > per_cu) occ = per_cu;
    const long cap = (long)occ * cus;
    if (g > cap) g = cap;
    if (kMaxGrid > 0 && g > kMaxGrid) g = kMaxGrid;
    if (g < 1) g = 1;
    return (int)g;
}

// Workgroups per CU for a one-column (streaming) launch.  A streaming wave
// keeps about one 1 KB segment per slot and matrix in flight (NI slots, at
// least two).  Sized so that a CU has about kStreamKB = 12 such segments per
// SIMD in flight (~48 KB per CU, e.g. three workgroups of waves holding four
// segments each), which measured fastest on MI355X: more waves put requests
// to more DRAM rows in flight at once, fewer leave the latency uncovered.
#ifndef QMV_STREAM_KB
#define QMV_STREAM_KB 12
#endif
template <int NI, int NMAT>
constexpr int stream_per_cu() {
    constexpr int kb = (NI >= 2 ? NI : 2) * NMAT;
    constexpr int w = (QMV_STREAM_KB + kb / 2) / kb;
    return w < 1 ? 1 : w;
}

// M = 1 keeps the activation slice in registers (MC = 1); wider M uses
// chunks of 4 activation rows read from LDS.
// Activation rows per workgroup for M > 1: 4, or 2 where four would push
// the kernel into scratch (eight segments per lane, or the two-matrix gate/up
// kernel with three or more).  Every chunk of rows streams the whole weight
// matrix once, so wider chunks mean fewer passes (int4 M=16: 4 instead of 8).
#ifndef QMV_MCW
#define QMV_MCW 4
#endif
#ifndef QMV_MCW_NARROW
#define QMV_MCW_NARROW 2
#endif
template <int NI, int NMAT = 1>
constexpr int mc_wide() {
    return (NI >= 8 || (NMAT == 2 && NI >= 3)) ? QMV_MCW_NARROW : QMV_MCW;
}

// Units (row blocks) per wave aimed at when sizing a launch that reads the
// activations from LDS: every workgroup stages its activation chunk once,
// so fewer, longer-lived workgroups amortise that copy.
#ifndef QMV_WIDE_UNITS
#define QMV_WIDE_UNITS 2
#endif
constexpr int kWideUnits = QMV_WIDE_UNITS;

// Waves per workgroup and units per wave of the several-column matvec: for
// int4 eight waves of one unit each, i.e. as many workgroups (two per CU,
// each staging its activation chunk once) as four waves of two units, with
// twice the resident waves (four per SIMD).  N=16384, K=4096, M = 4 / 8 /
// 16: eight waves of two units (one workgroup per CU) took 18.8 / 32.6 /
// 57.7 us against 20.1 / 33.8 / 59.0 with four, and eight waves of one unit
// another 4-5 % less at M = 4 and 8 on two boxes (17.9 / 29.4 against 18.8 /
// 30.7; M = 16 within +-2 %).  The other formats keep four waves of
// kWideUnits (MXFP4 M = 16 / 64 measured 7 % slower with eight waves).
template <int F>
constexpr int kWideWaves = F == FMT_INT4 ? 8 : kWaves;
template <int F>
constexpr int kWideUnitsF = F == FMT_INT4 ? 1 : kWideUnits;

// Registers a lane spends on its activation slice when MC = 1 (16-byte
// vectors x 4 VGPRs); above this budget the slice is read from LDS instead.
constexpr int kXregBudget = QMV_XREG_BUDGET;

// Dynamic LDS per workgroup is kept within 64 KB; chunks of kMcWide
// activation rows are used when they fit, single rows otherwise.
constexpr size_t kLdsBudget = 65536;
static inline bool wide_fits(int K, int copies, int mc) {
    return (size_t)copies * mc * K * 2 + 64 * mc <= kLdsBudget;
}

template <int F, int NI>
constexpr bool xreg_fits() {
    return NI * (SegCodes<F>::v / 8) * 4 <= kXregBudget;
}

template <int F, int RL, int NI, int NIP>
static hipError_t fo_matvec_shape(const MatvecArgs &a, hipStream_t st) {
    constexpr int D = ring_depth<NI, 1>();
    constexpr int CODES = SegCodes<F>::v;
    const uint8_t *wq = reinterpret_cast<const uint8_t *>(a.wq);
    const int seg_split = a.seg_split > 0 ? a.seg_split : (a.K + CODES - 1) / CODES;
    const int S = a.splits > 0 ? a.splits : 1;
    const int klen = seg_split * CODES;  // activation values staged per column
    // workgroups along x for one split: sized as if the S splits were S*N rows
    auto gx = [&](auto k, size_t lds, int depth, int per_cu = 0, int block = kBlock) {
        const int g = grid_for(k, lds, (long)a.N * S, RL, depth, per_cu, block);
        return (g + S - 1) / S;
    };
    if (a.M == 1) {
        constexpr bool xreg = xreg_fits<F, NI>();
        auto k = k_fo_matvec<F, RL, NI, NIP, 1, xreg>;
        const size_t lds = (size_t)klen * 2;
        hipLaunchKernelGGL(k, dim3(gx(k, lds, D * QMV_ROWS1, stream_per_cu<NI, 1>()), 1, S), dim3(kBlock), lds, st, wq, a.sc, a.x, a.y, a.y_dtype, a.M,
                           a.N, a.K, seg_split, a.part);
    } else if (wide_fits(klen, 1, mc_wide<NI>())) {
        constexpr int MCW = mc_wide<NI>();
        constexpr int WV = kWideWaves<F>;
        auto k = k_fo_matvec<F, RL, NI, NIP, MCW, false, WV>;
        const size_t lds = (size_t)MCW * klen * 2;
        const int gy = (a.M + MCW - 1) / MCW;
        hipLaunchKernelGGL(k, dim3(gx(k, lds, kWideUnitsF<F> * QMV_ROWS, 0, 64 * WV), gy, S), dim3(64 * WV), lds, st, wq,
                           a.sc, a.x, a.y, a.y_dtype, a.M, a.N, a.K, seg_split, a.part);
    } else {
        auto k = k_fo_matvec<F, RL, NI, NIP, 1, false>;
        const size_t lds = (size_t)klen * 2;
        hipLaunchKernelGGL(k, dim3(gx(k, lds, kWideUnits * QMV_ROWS), a.M, S), dim3(kBlock), lds, st, wq, a.sc, a.x,
                           a.y, a.y_dtype, a.M, a.N, a.K, seg_split, a.part);
    }
    return hipGetLastError();
}

#define QMV_SHAPE_SWITCH(FN, ...)                                           \
    switch (sh.RL * 100 + sh.NI * 10 + sh.NIP) {                            \
    case 811: return FN<8, 1, 1>(__VA_ARGS__);                              \
    case 1611: return FN<16, 1, 1>(__VA_ARGS__);                            \
    case 834: return FN<8, 3, 4>(__VA_ARGS__);                              \
    case 3211: return FN<32, 1, 1>(__VA_ARGS__);                            \
    case 6411: return FN<64, 1, 1>(__VA_ARGS__);                            \
    case 3234: return FN<32, 3, 4>(__VA_ARGS__);                            \
    case 3244: return FN<32, 4, 4>(__VA_ARGS__);                            \
    case 6434: return FN<64, 3, 4>(__VA_ARGS__);                            \
    case 6444: return FN<64, 4, 4>(__VA_ARGS__);                            \
    case 6488: return FN<64, 8, 8>(__VA_ARGS__);                            \
    default: return hipErrorInvalidValue;                                   \
    }

template <int RL, int NI, int NIP>
static hipError_t mv_int2(const MatvecArgs &a, hipStream_t st) { return fo_matvec_shape<FMT_INT2, RL, NI, NIP>(a, st); }
template <int RL, int NI, int NIP>
static hipError_t mv_int4(const MatvecArgs &a, hipStream_t st) { return fo_matvec_shape<FMT_INT4, RL, NI, NIP>(a, st); }
template <int RL, int NI, int NIP>
static hipError_t mv_mxfp4(const MatvecArgs &a, hipStream_t st) { return fo_matvec_shape<FMT_MXFP4, RL, NI, NIP>(a, st); }
template <int RL, int NI, int NIP>
static hipError_t mv_tern(const MatvecArgs &a, hipStream_t st) { return fo_matvec_shape<FMT_TERN, RL, NI, NIP>(a, st); }

hipError_t launch_fo_matvec(const MatvecArgs &a, hipStream_t st) {
    const int codes = a.fmt == FMT_INT2 ? 64 : (a.fmt == FMT_TERN ? 80 : 32);
    LaneShape sh;
    if (!pick_shape_rows(a.seg_split > 0 ? a.seg_split : (a.K + codes - 1) / codes,
                         (long)a.N * (a.splits > 0 ? a.splits : 1), sh))
        return hipErrorInvalidValue;
    if (a.fmt == FMT_INT2) { QMV_SHAPE_SWITCH(mv_int2, a, st) }
    if (a.fmt == FMT_INT4) { QMV_SHAPE_SWITCH(mv_int4, a, st) }
    if (a.fmt == FMT_TERN) { QMV_SHAPE_SWITCH(mv_tern, a, st) }
    QMV_SHAPE_SWITCH(mv_mxfp4, a, st)
}

// Launch one gate/up kernel variant: QM as in GateUpEpi; for QM == 1 the
// LDS also holds the workgroup's staged outputs (rounds x blocks per round x
// 32 x MC fp16 values).
template <int RL, int NI, int NIP, int MC, bool XREG>
static void gu_launch(const GateUpArgs &a, hipStream_t st, size_t lds, int depth, int per_cu, int gy) {
    constexpr int R = rows_block<MC, XREG>();
    constexpr int kRpu = R * (64 / RL);
    constexpr bool local_ok = (kWaves * kRpu) % 32 == 0;
    if (a.qcodes == nullptr) {
        auto k = k_fo_gateup<RL, NI, NIP, MC, XREG, 0>;
        hipLaunchKernelGGL(k, dim3(grid_for(k, lds, a.N, RL, depth, per_cu), gy), dim3(kBlock), lds, st, a.x,
                           a.residual, a.residual_out, a.gamma, a.eps, a.wq_gate, a.s_gate, a.wq_up, a.s_up,
                           a.out, a.M, a.N, a.K, nullptr, nullptr, nullptr, 0);
    } else if constexpr (local_ok) {
        constexpr int bpr = kWaves * kRpu / 32;
        auto k = k_fo_gateup<RL, NI, NIP, MC, XREG, 1>;
        // sized without the staging area first, then given it: the rounds
        // depend on the grid and the staging is small
        const int g = grid_for(k, lds, a.N, RL, depth, per_cu);
        const long units = a.N / kRpu;
        const int rounds = (int)((units + (long)g * kWaves - 1) / ((long)g * kWaves));
        const size_t lds_q = lds + (size_t)rounds * bpr * 32 * MC * 2;
        hipLaunchKernelGGL(k, dim3(g, gy), dim3(kBlock), lds_q, st, a.x, a.residual, a.residual_out, a.gamma,
                           a.eps, a.wq_gate, a.s_gate, a.wq_up, a.s_up, a.out, a.M, a.N, a.K, a.qcodes,
                           a.qscale, a.qcnt, rounds);
    } else {
        auto k = k_fo_gateup<RL, NI, NIP, MC, XREG, 2>;
        hipLaunchKernelGGL(k, dim3(grid_for(k, lds, a.N, RL, depth, per_cu), gy), dim3(kBlock), lds, st, a.x,
                           a.residual, a.residual_out, a.gamma, a.eps, a.wq_gate, a.s_gate, a.wq_up, a.s_up,
                           a.out, a.M, a.N, a.K, a.qcodes, a.qscale, a.qcnt, 0);
    }
}

template <int RL, int NI, int NIP>
static hipError_t gu_shape(const GateUpArgs &a, hipStream_t st) {
    constexpr int D = ring_depth<NI, 2>();
    constexpr int MCW = mc_wide<NI, 2>();
    if (a.M == 1 || !wide_fits(a.K, 1, MCW)) {
        const size_t lds = (size_t)a.K * 2 + 64;
        if (a.M == 1)
            gu_launch<RL, NI, NIP, 1, xreg_fits<FMT_INT2, NI>()>(a, st, lds, D, stream_per_cu<NI, 2>(), 1);
        else
            gu_launch<RL, NI, NIP, 1, false>(a, st, lds, kWideUnits * QMV_ROWS, 0, a.M);
    } else {
        const size_t lds = (size_t)MCW * a.K * 2 + 64 * MCW;
        gu_launch<RL, NI, NIP, MCW, false>(a, st, lds, kWideUnits * QMV_ROWS, 0, (a.M + MCW - 1) / MCW);
    }
    return hipGetLastError();
}

hipError_t launch_fo_gateup(const GateUpArgs &a, hipStream_t st) {
    LaneShape sh;
    const int nseg = a.K / 64;
    if (a.qcodes != nullptr && nseg <= 64) {
        // quantised output: eight lanes per row (eight rows per wave and unit),
        // so that a workgroup's round covers whole 32-row blocks (longer rows
        // use the counter fallback of mxfp4_tail)
        if (nseg > 24) return gu_shape<8, 8, 8>(a, st);
        sh = nseg <= 8 ? LaneShape{8, 1, 1} : LaneShape{8, 3, 4};
    } else if (!pick_shape_rows(nseg, a.N, sh)) {
        return hipErrorInvalidValue;
    }
    QMV_SHAPE_SWITCH(gu_shape, a, st)
}

size_t gateup_mxfp4_workspace_bytes(int M, int N) {
    const size_t cnt = ((size_t)M * (N / 32) * 4 + 255) / 256 * 256;
    return cnt + (size_t)M * N * 2;
}

// Two blocks per wave (one per 32-lane half), grid-stride over wave pairs of
// blocks so that every lane of a wave runs the same iterations.
__global__ void k_quant_mxfp4(const uint16_t *__restrict__ v, uint8_t *codes, uint8_t *scale, int nblk) {
    const int lane = threadIdx.x & 63;
    const int waves = gridDim.x * (blockDim.x >> 6);
    for (int w = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); 2 * w < nblk; w += waves) {
        const int b = 2 * w + (lane >> 5);
        const bool live = b < nblk;
        const uint16_t h = live ? v[(size_t)b * 32 + (lane & 31)] : (uint16_t)0;
        mx_quant_half(h, live, codes + (size_t)b * 16, scale + b);
    }
}

hipError_t launch_quant_mxfp4(const uint16_t *v, uint8_t *codes, uint8_t *scale, int M, int N,
                              hipStream_t st) {
    const int nblk = (int)((size_t)M * N / 32);
    int g = (nblk + 7) / 8;  // 4 waves of 2 blocks per workgroup
    if (g > 4096) g = 4096;
    hipLaunchKernelGGL(k_quant_mxfp4, dim3(g), dim3(256), 0, st, v, codes, scale, nblk);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Shared-prologue q/k/v ([A19] "What moved the needle", dispatch-count
// fusion): the residual-add RMSNorm prologue and three int2 fixed-order
// matvecs (q, k, v; their own row counts) in one dispatch.  Workgroups
// [0, bq) take q's rows, [bq, bq+bk) k's, the rest v's; every workgroup
// computes the prologue of its activation row (blockIdx.y) itself, exactly
// as the fused gate/up kernel does, and workgroup 0 of q writes
// residual_out.
template <int MC>
struct QkvEpi {
    OutBuf out;
    int M, N, m0;
    __device__ __forceinline__ void operator()(int n, int q, const float (&tot)[1][MC],
                                               const float (&rs)[1]) {
        const bool act = q == 0 && n < N;
#pragma unroll
        for (int m = 0; m < MC; ++m)
            if (m0 + m < M) out.put(act, (uint32_t)((m0 + m) * N + n), rs[0] * tot[0][m]);
    }
};

template <int RL, int NI, int NIP, bool XREG>
__global__ __launch_bounds__(kBlock) void k_fo_qkv(const QkvArgs a, int bq, int bk, int bv) {
    extern __shared__ __align__(16) uint16_t smem[];
    uint16_t *xs = smem;  // [K]: h, then the normalised xn in place
    float *inv_s = reinterpret_cast<float *>(smem + a.K);
    const int b = blockIdx.x, m = blockIdx.y;
    // uniform per workgroup: which matrix, and this workgroup's index in it
    const int z = b < bq ? 0 : (b < bq + bk ? 1 : 2);
    const int blk = z == 0 ? b : (z == 1 ? b - bq : b - bq - bk);
    const int nblk = z == 0 ? bq : (z == 1 ? bk : bv);
    const int N = a.N[z];
    const uint8_t *const w1[1] = {reinterpret_cast<const uint8_t *>(a.wq[z])};
    const void *const s1[1] = {a.s[z]};
    FoEngine<FMT_INT2, RL, NI, NIP, 1, XREG, 1, ring_depth<NI, 1>(), 1> eng(w1, s1, N, a.K, 0, 0, blk, nblk);
    RmsStage1 rs1;
    rs1.load(a.x, a.residual, a.gamma, a.K, m);
    eng.prefetch();
    rs1.finish(a.x, a.residual, a.gamma, b == 0 ? a.residual_out : nullptr, a.eps, a.K, m, xs, inv_s);
    QkvEpi<1> epi{OutBuf(a.y[z], (uint32_t)a.M * (uint32_t)N, a.y_dtype), a.M, N, m};
    eng.run(xs, epi);
}

template <int RL, int NI, int NIP>
static hipError_t qkv_shape(const QkvArgs &a, hipStream_t st) {
    constexpr int D = ring_depth<NI, 1>();
    auto k = k_fo_qkv<RL, NI, NIP, xreg_fits<FMT_INT2, NI>()>;
    const size_t lds = (size_t)a.K * 2 + 64;
    const long ntot = (long)a.N[0] + a.N[1] + a.N[2];
    // the workgroups one launch over all rows would use, shared out by rows
    const int g = grid_for(k, lds, ntot, RL, D, stream_per_cu<NI, 1>());
    int bz[3];
    for (int z = 0; z < 3; ++z) {
        const int rpg = 64 / RL;
        const long need = ((long)a.N[z] + rpg * kWaves - 1) / (rpg * kWaves);  // one row group per wave
        long share = ((long)g * a.N[z] + ntot - 1) / ntot;
        if (share > need) share = need;
        bz[z] = share < 1 ? 1 : (int)share;
    }
    hipLaunchKernelGGL(k, dim3(bz[0] + bz[1] + bz[2], a.M), dim3(kBlock), lds, st, a, bz[0], bz[1], bz[2]);
    return hipGetLastError();
}

hipError_t launch_fo_qkv(const QkvArgs &a, hipStream_t st) {
    LaneShape sh;
    if (!pick_shape_rows(a.K / 64, (long)a.N[0] + a.N[1] + a.N[2], sh)) return hipErrorInvalidValue;
    QMV_SHAPE_SWITCH(qkv_shape, a, st)
}

// ---------------------------------------------------------------------------
// Expert-gather MXFP4 matvec: output plane p = (m, j), m = p / topk, is the
// fixed-order matvec of activation row m with expert e = idx[p], read in
// place (no gathered copy of the weights).  grid.y = the M*topk planes; the
// workgroups along x share the plane's rows like a plain M = 1 launch.  The
// expert's weights and scales are addressed through buffer descriptors that
// cover that expert only, so no load reaches another expert's rows.  An id
// outside [0, E) reads nothing and sets the plane's outputs to NaN.
template <int RL, int NI, int NIP, bool XREG>
__global__ __launch_bounds__(kBlock) void k_fo_gather(const GatherArgs a) {
    extern __shared__ __align__(16) uint16_t xs[];
    const int p = blockIdx.y;
    const int m = p / a.topk;
    const int e = __builtin_amdgcn_readfirstlane(a.idx[p]);
    const uint32_t total = (uint32_t)a.M * (uint32_t)a.topk * (uint32_t)a.N;
    if (e < 0 || e >= a.E) {  // uniform over the workgroup
        const OutBuf out(a.y, total, a.y_dtype);
        for (int n = blockIdx.x * kBlock + threadIdx.x; n < a.N; n += gridDim.x * kBlock)
            out.put(true, (uint32_t)p * a.N + n, __builtin_nanf(""));
        return;
    }
    const uint8_t *const w1[1] = {a.wq + (size_t)e * a.N * (a.K / 2)};
    const void *const s1[1] = {a.e8m0 + (size_t)e * a.N * (a.K / 32)};
    FoEngine<FMT_MXFP4, RL, NI, NIP, 1, XREG, 1, ring_depth<NI, 1>(), 1> eng(w1, s1, a.N, a.K);
    const uint16_t *xm = a.x + (size_t)m * a.K;
    XStage<1> xst;
    xst.load(xm, 1, a.K, a.K, 0);
    eng.prefetch();
    xst.store(xm, xs, 1, a.K, a.K, 0);
    __syncthreads();
    StoreEpi<FMT_MXFP4, 1> epi{OutBuf(a.y, total, a.y_dtype), false, a.M * a.topk, a.N, p};
    eng.run(xs, epi);
}

template <int RL, int NI, int NIP>
static hipError_t gather_shape(const GatherArgs &a, hipStream_t st) {
    constexpr int D = ring_depth<NI, 1>();
    auto k = k_fo_gather<RL, NI, NIP, xreg_fits<FMT_MXFP4, NI>()>;
    const size_t lds = (size_t)a.K * 2;
    const int planes = a.M * a.topk;
    // the workgroups one launch over all planes' rows would use, per plane
    const int g = grid_for(k, lds, (long)a.N * planes, RL, D, stream_per_cu<NI, 1>());
    const int gx = (g + planes - 1) / planes;
    hipLaunchKernelGGL(k, dim3(gx, planes), dim3(kBlock), lds, st, a);
    return hipGetLastError();
}

hipError_t launch_fo_gather(const GatherArgs &a, hipStream_t st) {
    LaneShape sh;
    if (!pick_shape_rows(a.K / 32, (long)a.N * a.M * a.topk, sh)) return hipErrorInvalidValue;
    QMV_SHAPE_SWITCH(gather_shape, a, st)
}

// Activation rows per argmax workgroup chunk, and the number of chunks.
static void argmax_chunks(int M, int K, int mcw, int &mc, int &gy) {
    mc = (M > 1 && wide_fits(K, 1, mcw)) ? mcw : 1;
    gy = (M + mc - 1) / mc;
}

constexpr size_t kCounterBytes = 1024;  // one 32-bit completion counter per chunk (<= 256)

size_t argmax_workspace_bytes(int M, int N, int K) {
    LaneShape sh;
    if (M < 1 || N < 1 || !pick_shape(K / 64, sh)) return 0;
    return kCounterBytes + (((size_t)M * sizeof(uint64_t) + 255) / 256) * 256;  // counters, keys
}

template <int RL, int NI, int NIP>
static hipError_t am_shape(const ArgmaxArgs &a, hipStream_t st) {
    constexpr int D = ring_depth<NI, 1>();
    uint32_t *counter = reinterpret_cast<uint32_t *>(a.ws);
    uint64_t *keys = reinterpret_cast<uint64_t *>(reinterpret_cast<uint8_t *>(a.ws) + kCounterBytes);
    constexpr int MCW = mc_wide<NI>();
    int mc, gy;
    argmax_chunks(a.M, a.K, MCW, mc, gy);
    if (a.M == 1) {
        auto k = k_fo_argmax<RL, NI, NIP, 1, xreg_fits<FMT_INT2, NI>()>;
        const size_t lds = (size_t)a.K * 2;
        hipLaunchKernelGGL(k, dim3(grid_for(k, lds, a.N, RL, D, stream_per_cu<NI, 1>()), 1), dim3(kBlock), lds, st, a.wq,
                           a.scale, a.x, a.idx, a.maxval, a.logits, a.M, a.N, a.K, keys, counter);
    } else if (mc == 1) {
        auto k = k_fo_argmax<RL, NI, NIP, 1, false>;
        const size_t lds = (size_t)a.K * 2;
        hipLaunchKernelGGL(k, dim3(grid_for(k, lds, a.N, RL, kWideUnits * QMV_ROWS), gy), dim3(kBlock), lds, st, a.wq,
                           a.scale, a.x, a.idx, a.maxval, a.logits, a.M, a.N, a.K, keys, counter);
    } else {
        auto k = k_fo_argmax<RL, NI, NIP, MCW, false>;
        const size_t lds = (size_t)MCW * a.K * 2;
        hipLaunchKernelGGL(k, dim3(grid_for(k, lds, a.N, RL, kWideUnits * QMV_ROWS), gy), dim3(kBlock), lds, st, a.wq,
                           a.scale, a.x, a.idx, a.maxval, a.logits, a.M, a.N, a.K, keys, counter);
    }
    return hipGetLastError();
}

hipError_t launch_fo_argmax(const ArgmaxArgs &a, hipStream_t st) {
    LaneShape sh;
    if (!pick_shape_rows(a.K / 64, a.N, sh)) return hipErrorInvalidValue;
    QMV_SHAPE_SWITCH(am_shape, a, st)
}

// Split-K plan: the smallest power-of-two split count (at most 16, at
// least 4 segments per split) that gives every SIMD about four row groups;
// K splits only pay when N alone leaves the GPU short of work.
constexpr long kSplitTargetRowGroups = 4096;

int splitk_plan(int fmt, int M, int N, int K, int &seg_split) {
    (void)M;
    const int codes = fmt == FMT_INT2 ? 64 : 32;
    const int nseg = K / codes;
    LaneShape sh;
    seg_split = nseg;
    if (!pick_shape(nseg, sh)) return 1;
    long rg = ((long)N + 64 / sh.RL - 1) / (64 / sh.RL);
    int best = 1;
    for (int S = 2; S <= 16 && rg < kSplitTargetRowGroups; S *= 2) {
        const int ss = (nseg + S - 1) / S;
        if (ss < 4 || !pick_shape(ss, sh)) break;
        const int seff = (nseg + ss - 1) / ss;
        best = seff;
        seg_split = ss;
        rg = ((long)N + 64 / sh.RL - 1) / (64 / sh.RL) * seff;
    }
    if (best == 1) seg_split = nseg;
    return best;
}

size_t splitk_workspace_bytes(int fmt, int M, int N, int K) {
    int ss;
    const int S = splitk_plan(fmt, M, N, K, ss);
    return S > 1 ? (size_t)S * M * N * sizeof(float) : 0;
}

hipError_t launch_splitk_matvec(const MatvecArgs &a0, void *ws, hipStream_t st) {
    MatvecArgs a = a0;
    int ss;
    const int S = splitk_plan(a.fmt, a.M, a.N, a.K, ss);
    if (S == 1) return launch_fo_matvec(a, st);
    a.seg_split = ss;
    a.splits = S;
    a.part = reinterpret_cast<float *>(ws);
    hipError_t e = launch_fo_matvec(a, st);
    if (e != hipSuccess) return e;
    const size_t total = (size_t)a.M * a.N;
    size_t g = (total + 255) / 256;
    if (g > 4096) g = 4096;
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)g), dim3(256), 0, st, a.part, S, a.M, a.N,
                       a.fmt == FMT_INT2 ? reinterpret_cast<const uint16_t *>(a.sc) : nullptr, a.y, a.y_dtype);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t st) {
    const size_t words = bytes / 4;
    if (words == 0) return hipSuccess;
    size_t g = (words + 255) / 256;
    if (g > 1024) g = 1024;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)g), dim3(256), 0, st, reinterpret_cast<uint32_t *>(p),
                       words);
    return hipGetLastError();
}

}  // namespace qmv
