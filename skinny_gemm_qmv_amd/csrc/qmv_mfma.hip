// qmv_mfma.hip -- opt-in matrix-core mode for MXFP4 weights and bf16
// activations at M >= 32 ("Gemma 4 Optimization with Agentic Kernel
// Engineering", sections "A new chip, the same model" and "How much of the
// chip we use now": the MXFP4 GEMMs of MI355X serving run on the matrix
// cores).
//
//   Y[m][n] = sum_k X[m][k] * W[n][k],  W[n][k] = E2M1 code * 2^(E[n][k/32]-127)
//
// Every weight is dequantized exactly to bf16 by v_cvt_scalef32_pk_bf16_fp4
// (an E2M1 value has at most two significant bits; times the block scale it
// is a bf16 number while |value| * 2^(E-127) stays inside the bf16 normal
// range), and v_mfma_f32_16x16x32_bf16 sums the exact bf16 x bf16 products
// in fp32.  The order of that sum is the matrix core's, not the fixed order:
// this mode belongs to the tolerance class (relative L2 error <= 2e-3).
//
// Work split (MI355X: 256 CUs, one matrix core per SIMD):
//  * Workgroup b owns a contiguous range of 16-row weight tiles (at most one
//    workgroup per CU, so each weight byte is read from HBM once) and all M
//    activation rows; its WV waves split M (MW m-tiles of 16 rows each).
//  * K advances in chunks of 128 = four MXFP4 blocks.  Every load is laid
//    out for the memory system: a weight tile's chunk (16 rows x 64 bytes)
//    is read by four consecutive lanes per row, an activation row's chunk
//    (256 bytes) by sixteen consecutive lanes.
//  * The weight tiles of a chunk are loaded once per workgroup (tile i by
//    wave i mod WV) into a shared LDS buffer (double buffered, one barrier
//    per chunk); each wave keeps its own activation rows in a private LDS
//    pad.  Both are read back in the MFMA layout.
//  * Lane group g = lane / 16 reads the whole 16-byte MXFP4 block 4c + g of
//    weight row l % 16 and its scale; sub-step j dequantizes dword j (8 codes)
//    and the A fragment of lane group g, sub-step j comes from the same k
//    range, so both operands map (g, element e) of sub-step j to
//    k = 128c + 32g + 8j + e.
//  * Each wave dequantizes every tile of the range (4/MW conversions per
//    MFMA); two waves per SIMD (WV = 8) let one wave's conversions overlap
//    the other's matrix work.
#include "qmv_device.hpp"
#include "qmv_internal.hpp"

namespace qmv {

typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr uint32_t kOob = 0xFFFFFFF0u;  // past every buffer: loads return 0
#ifndef QMV_MFMA_WAUX
#define QMV_MFMA_WAUX 0
#endif

constexpr int kXRow = 128 * 2 + 16;  // LDS bytes per activation row of a chunk (+16: bank spread)
constexpr int kWRow = 64 + 16;       // LDS bytes per weight row of a chunk (+16: conflict-free reads)
constexpr int kWTile = 16 * kWRow;   // one 16-row weight tile of a chunk

// Loads of one chunk held by a wave: its weight tile slots (dwordx4 + scale
// byte per lane) and its activation rows (MW m-tiles x 4 dwordx4 per lane).
template <int WT, int MW>
struct ChunkSlot {
    u4_t w[WT];
    uint32_t e[WT];
    u4_t x[MW][4];
};

// Chunks in flight besides the one being multiplied.
// Even, so that the loop unrolled over D slots also alternates the two
// fragment sets.
template <int WV, int MW>
constexpr int mfma_depth() {
    return WV == 4 ? 4 : 2;
}

// Weight fragments of one chunk read back from LDS: the raw MXFP4 dwords of
// every tile (4 sub-steps each) and their scales.  (A fragments are read per
// sub-step inside the multiply; holding a second set of them would cost the
// registers that give two waves per SIMD.)
template <int NB>
struct Frags {
    u4_t braw[NB];
    float sc[NB];
};

template <int WV, int MW, int NB>
__global__ __launch_bounds__(WV * 64) void k_mxfp4_mfma(
    const uint8_t *__restrict__ wq, const uint8_t *__restrict__ e8m0, const uint16_t *__restrict__ x,
    void *y, int y_dtype, int M, int N, int K, int NT, int ranges) {
    constexpr int D = mfma_depth<WV, MW>();
    constexpr int WT = (NB + WV - 1) / WV;  // tile slots loaded by each wave
    __shared__ __align__(16) uint8_t wbuf[2][NB][kWTile];
    __shared__ __align__(16) uint8_t sbuf[2][NB][64];
    __shared__ __align__(16) uint8_t xpad[WV][2][MW * 16 * kXRow];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int lrow = lane >> 2, lpc = lane & 3;  // weight load layout
    const int t0 = (int)(((long)blockIdx.x * NT) / ranges);
    const int t1 = (int)(((long)(blockIdx.x + 1) * NT) / ranges);  // t1 - t0 <= NB (host)
    const int m0w = wave * MW * 16;  // first activation row of this wave

    const int nseg = K >> 5;
    const int nchunk = (nseg + 3) >> 2;
    const uint32_t row_bytes = (uint32_t)K >> 1;
    const uint32_t xrow_bytes = (uint32_t)K * 2u;
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(wq), 0, (uint32_t)N * row_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t re =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(e8m0), 0, (uint32_t)N * nseg, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(x), 0, (uint32_t)M * xrow_bytes, 0x00020000);

    // weight tile slots of this wave: slot i = wave + WV*s of the range
    uint32_t wrow[WT], erow[WT];
    bool sok[WT], tok[WT];
#pragma unroll
    for (int s = 0; s < WT; ++s) {
        const int i = wave + WV * s;
        const uint32_t n = (uint32_t)(t0 + i) * 16u + lrow;
        sok[s] = i < NB;             // slot exists (uniform)
        tok[s] = sok[s] && t0 + i < t1;  // and holds a tile of this range
        wrow[s] = n * row_bytes + 16u * lpc;
        erow[s] = n * (uint32_t)nseg + lpc;
    }
    // activation rows of this wave: load q of m-tile mw covers rows
    // mw*16 + 4q + lane/16; rows >= M read 0 (past the buffer)
    const uint32_t xbase = (uint32_t)(m0w + (lane >> 4)) * xrow_bytes + 16u * (lane & 15);

    auto load = [&](ChunkSlot<WT, MW> &sl, int c) {
        const bool segok = 4 * c + lpc < nseg;  // the last chunk may hold fewer than 4 blocks
#pragma unroll
        for (int s = 0; s < WT; ++s) {
            const bool ok = segok && tok[s];
            sl.w[s] = __builtin_bit_cast(
                u4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, ok ? wrow[s] + 64u * c : kOob, 0, QMV_MFMA_WAUX));
            sl.e[s] = __builtin_amdgcn_raw_buffer_load_b8(re, ok ? erow[s] + 4u * c : kOob, 0, 0);
        }
        const bool cok = c < nchunk;  // chunks past the end read nothing
#pragma unroll
        for (int mw = 0; mw < MW; ++mw)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                sl.x[mw][q] = __builtin_bit_cast(
                    u4_t, __builtin_amdgcn_raw_buffer_load_b128(
                              rx, cok ? xbase + (uint32_t)(mw * 16 + 4 * q) * xrow_bytes + 256u * c : kOob, 0, 0));
    };

    f4_t acc[MW][NB];
#pragma unroll
    for (int mw = 0; mw < MW; ++mw)
#pragma unroll
        for (int i = 0; i < NB; ++i) acc[mw][i] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

    ChunkSlot<WT, MW> slot[D];
#pragma unroll
    for (int d = 0; d < D; ++d) load(slot[d], d);

    const bool active = m0w < M;  // uniform: this wave has activation rows
    // Software pipeline over chunks.  Iteration c: publish chunk c+1 (the
    // wave's weight slots to the shared buffer (c+1)&1, its activation rows
    // to its pad (c+1)&1), one barrier (every wave has then finished reading
    // chunk c-1's fragments, the last reads of those buffers), refill the slot
    // with chunk c+1+D, read chunk c+1's fragments, and multiply chunk c from
    // the fragments read one iteration earlier -- so the LDS reads of the next
    // chunk overlap this chunk's matrix work.
    auto publish = [&](const ChunkSlot<WT, MW> &cur, int c) {
        uint8_t(*wb)[kWTile] = wbuf[c & 1];
        uint8_t(*sb)[64] = sbuf[c & 1];
        uint8_t *xp = xpad[wave][c & 1];
#pragma unroll
        for (int s = 0; s < WT; ++s)
            if (sok[s]) {
                *reinterpret_cast<u4_t *>(&wb[wave + WV * s][lrow * kWRow + 16 * lpc]) = cur.w[s];
                sb[wave + WV * s][lrow * 4 + lpc] = (uint8_t)cur.e[s];
            }
#pragma unroll
        for (int mw = 0; mw < MW; ++mw)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<u4_t *>(&xp[(mw * 16 + 4 * q + (lane >> 4)) * kXRow + 16 * (lane & 15)]) =
                    cur.x[mw][q];
    };
    auto read_frags = [&](Frags<NB> &f, int c) {
        uint8_t(*wb)[kWTile] = wbuf[c & 1];
        uint8_t(*sb)[64] = sbuf[c & 1];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            f.braw[i] = *reinterpret_cast<const u4_t *>(&wb[i][r16 * kWRow + 16 * g]);
            f.sc[i] = e8m0_to_f32(sb[i][r16 * 4 + g]);
        }
    };
    // Per sub-step: dequantize every tile's B fragment into its own
    // registers, then issue the MFMAs.  (Converting into the registers the
    // previous MFMA is still reading would chain every MFMA behind four
    // conversions; separate fragments let conversions run under the matrix
    // work of the previous sub-step.)
    auto multiply = [&](const Frags<NB> &f, int c) {
        const uint8_t *xp = xpad[wave][c & 1];
        // all four sub-steps' A fragments first: one LDS latency per chunk
        u4_t af[4][MW];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int mw = 0; mw < MW; ++mw)
                af[j][mw] = *reinterpret_cast<const u4_t *>(&xp[(mw * 16 + r16) * kXRow + 64 * g + 16 * j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u4_t(&a)[MW] = af[j];
            bf8_t bw[NB];
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const uint32_t wd = f.braw[i][j];
                const bf2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, f.sc[i], 0);
                const bf2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, f.sc[i], 1);
                const bf2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, f.sc[i], 2);
                const bf2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, f.sc[i], 3);
                bw[i] = bf8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
            }
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int mw = 0; mw < MW; ++mw)
                    acc[mw][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8_t, a[mw]), bw[i],
                                                                        acc[mw][i], 0, 0, 0);
        }
    };

    Frags<NB> fr[2];
    publish(slot[0], 0);
    __syncthreads();
    load(slot[0], D);
    read_frags(fr[0], 0);
    // Every iteration issues the same loads and LDS traffic (chunks past the
    // end read nothing and are never multiplied), so the compiler's count of
    // outstanding loads stays exact; the loop runs over whole groups of D.
    for (int c0 = 0; c0 < nchunk; c0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int c = c0 + d;
            ChunkSlot<WT, MW> &nxt = slot[(d + 1) % D];  // holds chunk c+1
            publish(nxt, c + 1);
            __syncthreads();
            load(nxt, c + 1 + D);
            read_frags(fr[(d + 1) & 1], c + 1);
            if (active && c < nchunk) multiply(fr[d & 1], c);
        }
    }

    // D[i][j] of a 16x16 tile: lane l holds rows 4(l/16) .. 4(l/16)+3 of column l%16.
    if (!active) return;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int n = (t0 + i) * 16 + r16;
        if (t0 + i >= t1 || n >= N) continue;
#pragma unroll
        for (int mw = 0; mw < MW; ++mw)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0w + mw * 16 + 4 * g + v;
                if (m < M) store_out(y, (size_t)m * N + n, acc[mw][i][v], y_dtype);
            }
    }
}

// Tiles per workgroup compiled; the host picks the smallest that covers
// ceil(NT / grid).
constexpr int kMfmaMaxNb = 8;

template <int WV, int MW, int NB>
static hipError_t mfma_launch(const MatvecArgs &a, int NT, int ranges, hipStream_t st) {
    hipLaunchKernelGGL((k_mxfp4_mfma<WV, MW, NB>), dim3(ranges), dim3(WV * 64), 0, st,
                       reinterpret_cast<const uint8_t *>(a.wq), reinterpret_cast<const uint8_t *>(a.sc), a.x,
                       a.y, a.y_dtype, a.M, a.N, a.K, NT, ranges);
    return hipGetLastError();
}

template <int WV, int MW>
static hipError_t mfma_nb(const MatvecArgs &a, int NT, int ranges, int nb, hipStream_t st) {
    if (nb <= 1) return mfma_launch<WV, MW, 1>(a, NT, ranges, st);
    if (nb <= 2) return mfma_launch<WV, MW, 2>(a, NT, ranges, st);
    if (nb <= 3) return mfma_launch<WV, MW, 3>(a, NT, ranges, st);
    if (nb <= 4) return mfma_launch<WV, MW, 4>(a, NT, ranges, st);
    if (MW > 1 || nb <= 6) return mfma_launch<WV, MW, 6>(a, NT, ranges, st);
    return mfma_launch<WV, MW, (MW > 1 ? 6 : 8)>(a, NT, ranges, st);
}

hipError_t launch_mxfp4_mfma(const MatvecArgs &a, hipStream_t st) {
    if (a.fmt != FMT_MXFP4 || a.M < 32 || a.M > 256 || a.K % 32 != 0) return hipErrorInvalidValue;
    const int NT = (a.N + 15) / 16;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int mt = (a.M + 15) / 16;
    // two m-tiles per wave leave registers for 6 tiles per workgroup
    const int max_nb = mt > 8 ? 6 : kMfmaMaxNb;
    int ranges = NT < cus ? NT : cus;
    int nb = (NT + ranges - 1) / ranges;
    if (nb > max_nb) {
        nb = max_nb;
        ranges = (NT + nb - 1) / nb;
    }
    // every range t0..t1 then spans at most nb tiles
    if (mt <= 4) return mfma_nb<4, 1>(a, NT, ranges, nb, st);
    if (mt <= 8) return mfma_nb<8, 1>(a, NT, ranges, nb, st);
    return mfma_nb<8, 2>(a, NT, ranges, nb, st);
}

}  // namespace qmv
