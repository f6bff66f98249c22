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
//  * A workgroup (four waves) owns MT m-tiles (16 activation rows each) and
//    a range of up to 4*NBW 16-row weight tiles; wave w owns tiles w, w+4,
//    ... of the range.  A wave converts each of its weight fragments once
//    and multiplies it with all MT activation fragments, so no weight is
//    dequantized twice inside a workgroup.
//  * K advances in chunks of 128 = four MXFP4 blocks.  Lane l of a wave
//    loads, straight from HBM in the matrix-core layout, the 16-byte MXFP4
//    block 4c + l/16 of weight row l%16 of a tile, and that block's scale.
//    Sub-step j of the chunk dequantizes dword j of the block (8 codes), so
//    lane group g = l/16 of sub-step j covers k = 128c + 32g + 8j + e, and
//    the activation fragments use the same map.
//  * The workgroup's activation rows of a chunk (MT*16 rows x 256 bytes) are
//    loaded by all 256 lanes (sixteen lanes per row) and published to a
//    double-buffered LDS tile: one barrier per chunk.
//  * Weight loads run DW chunks ahead and activation loads DX chunks ahead
//    in registers (the weights come from HBM, the activations mostly from
//    L2, so the weight ring is the deep one).
//  * Block scales: when K is a multiple of 128 (every chunk whole, so a
//    row's scale bytes start on a dword), one 16-byte load per tile brings
//    the scales of four chunks (blocks 16G .. 16G+15 of the row) and lane
//    group g takes byte g of dword c % 4; otherwise each chunk loads its
//    scale byte per lane.  A vector-memory instruction costs about the
//    same whatever its width, and the byte loads were a quarter of them.
//  * The workgroup count is sized to cover the CUs once: M is split into
//    ceil(M/16/MT) blocks and each wave takes up to four weight tiles, so
//    every activation fragment read from LDS feeds several matrix ops; with
//    a single m-block the tile ranges are spread over every CU.
#include "qmv_device.hpp"
#include "qmv_internal.hpp"

namespace qmv {

typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr uint32_t kOob = 0xFFFFFFF0u;  // past every buffer: loads return 0
constexpr int kXRow = 128 * 2 + 16;     // LDS bytes per activation row of a chunk (+16: bank spread)
constexpr int kMfmaThreads = 256;

template <int MT, int NBW, int DW, int DX, bool SV>
__global__ __launch_bounds__(kMfmaThreads) void k_mxfp4_mfma(const uint8_t *__restrict__ wq,
                                                             const uint8_t *__restrict__ e8m0,
                                                             const uint16_t *__restrict__ x, void *y,
                                                             int y_dtype, int M, int N, int K, int NT,
                                                             int ranges) {
    constexpr int XP = MT;  // 16-byte activation pieces per lane per chunk
    __shared__ __align__(16) uint8_t xs[2][MT * 16 * kXRow];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int t0 = (int)(((long)blockIdx.x * NT) / ranges);
    const int t1 = (int)(((long)(blockIdx.x + 1) * NT) / ranges);  // t1 - t0 <= 4 * NBW (host)
    const int m0 = blockIdx.y * MT * 16;

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

    // weight tiles of this wave: the s-th is tile t0 + wave + 4s (rows past
    // N and tiles past the range read zeros)
    uint32_t wrow[NBW], erow[NBW], erow0[NBW];
    bool tok[NBW];
#pragma unroll
    for (int s = 0; s < NBW; ++s) {
        const int t = t0 + wave + 4 * s;
        tok[s] = t < t1;
        const uint32_t n = (uint32_t)t * 16u + r16;
        wrow[s] = n * row_bytes + 16u * g;
        erow0[s] = n * (uint32_t)nseg;
        erow[s] = erow0[s] + g;
    }
    // activation pieces of this lane: piece p = threadIdx.x + 256 i is row
    // p / 16, 16-byte column p % 16 of the workgroup's chunk
    uint32_t xoff[XP];
    int xcol[XP];
    bool xrok[XP];
#pragma unroll
    for (int i = 0; i < XP; ++i) {
        const int p = threadIdx.x + kMfmaThreads * i;
        const int row = p >> 4;
        xcol[i] = p & 15;
        xrok[i] = m0 + row < M;
        xoff[i] = (uint32_t)(m0 + row) * xrow_bytes + 16u * (uint32_t)xcol[i];
    }

    static_assert(DW % DX == 0, "the unrolled loop cycles both rings");
    static_assert(!SV || DW == 4, "one scale group per pass over the weight ring");
    u4_t wslot[DW][NBW];
    uint32_t eslot[DW][NBW];
    u4_t xslot[DX][XP];
    auto load_w = [&](u4_t (&w)[NBW], uint32_t (&e)[NBW], int c) {
        const bool segok = 4 * c + g < nseg;  // the last chunk may hold fewer than 4 blocks
#pragma unroll
        for (int s = 0; s < NBW; ++s) {
            const bool ok = segok && tok[s];
            w[s] = __builtin_bit_cast(u4_t,
                                      __builtin_amdgcn_raw_buffer_load_b128(rw, ok ? wrow[s] + 64u * c : kOob, 0, 0));
            if constexpr (!SV) e[s] = __builtin_amdgcn_raw_buffer_load_b8(re, ok ? erow[s] + 4u * c : kOob, 0, 0);
        }
    };
    // scales of chunks 4G .. 4G+3 (rows past N and groups past the row end
    // read zeros or the next row's bytes; neither is ever multiplied)
    auto load_sv = [&](u4_t (&v)[NBW], int G) {
#pragma unroll
        for (int s = 0; s < NBW; ++s)
            v[s] = __builtin_bit_cast(
                u4_t, __builtin_amdgcn_raw_buffer_load_b128(re, tok[s] ? erow0[s] + 16u * (uint32_t)G : kOob, 0, 0));
    };
    auto load_x = [&](u4_t (&xv)[XP], int c) {
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            // columns past K (a partial last chunk) read zeros, so that the
            // zero weights there never meet a non-finite activation
            const bool ok = xrok[i] && 128 * c + 8 * xcol[i] < K;
            xv[i] = __builtin_bit_cast(u4_t,
                                       __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? xoff[i] + 256u * c : kOob, 0, 0));
        }
    };
    auto publish = [&](const u4_t (&xv)[XP], int c) {
        uint8_t *b = xs[c & 1];
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            const int p = threadIdx.x + kMfmaThreads * i;
            *reinterpret_cast<u4_t *>(&b[(p >> 4) * kXRow + 16 * (p & 15)]) = xv[i];
        }
    };

    f4_t acc[MT][NBW];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int s = 0; s < NBW; ++s) acc[mt][s] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

    auto multiply = [&](const u4_t (&w)[NBW], const uint32_t (&e)[NBW], int c) {
        const uint8_t *b = xs[c & 1];
        float sc[NBW];
#pragma unroll
        for (int s = 0; s < NBW; ++s) sc[s] = e8m0_to_f32(e[s]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u4_t af[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                af[mt] = *reinterpret_cast<const u4_t *>(&b[(mt * 16 + r16) * kXRow + 64 * g + 16 * j]);
#pragma unroll
            for (int s = 0; s < NBW; ++s) {
                const uint32_t wd = w[s][j];
                const bf2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc[s], 0);
                const bf2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc[s], 1);
                const bf2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc[s], 2);
                const bf2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc[s], 3);
                const bf8_t bw = bf8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8_t, af[mt]), bw,
                                                                        acc[mt][s], 0, 0, 0);
            }
        }
    };

    // Chunk c's weights sit in wslot[c % DW]; its activations are in LDS
    // buffer c & 1 while it is multiplied, and chunks c+1 .. c+DX wait in the
    // register slots xslot[(c+1) % DX] ...
    // Prologue: chunk 0's activations to LDS, chunks 1..DX in registers,
    // weights of chunks 0..DW-1 (and their scale group) in flight.
    u4_t svc[SV ? NBW : 1], svn[SV ? NBW : 1];
    load_x(xslot[0], 0);
#pragma unroll
    for (int d = 0; d < DW; ++d) load_w(wslot[d], eslot[d], d);
    if constexpr (SV) load_sv(svn, 0);
    publish(xslot[0], 0);
#pragma unroll
    for (int d = 1; d <= DX; ++d) load_x(xslot[d % DX], d);
    __syncthreads();

    // Iteration c: multiply chunk c; publish chunk c+1 to the other LDS
    // buffer (its last readers, the multiply of chunk c-1, finished before
    // the previous barrier) and refill its register slot with chunk c+1+DX;
    // refill chunk c's weight slot with chunk c+DW; barrier.  Every iteration
    // issues the same loads (chunks past the end read nothing and are never
    // multiplied), so the compiler's count of outstanding loads is exact; the
    // loop runs over whole groups of DW.
    for (int c0 = 0; c0 < nchunk; c0 += DW) {
#pragma unroll
        for (int d = 0; d < DW; ++d) {
            const int c = c0 + d;
            if constexpr (SV) {
                if (d == 0) {
#pragma unroll
                    for (int s = 0; s < NBW; ++s) svc[s] = svn[s];
                }
#pragma unroll
                for (int s = 0; s < NBW; ++s) eslot[d][s] = (svc[s][d] >> (8 * g)) & 0xFFu;
            }
            if (c < nchunk) multiply(wslot[d], eslot[d], c);
            u4_t(&nx)[XP] = xslot[(d + 1) % DX];
            publish(nx, c + 1);
            load_x(nx, c + 1 + DX);
            load_w(wslot[d], eslot[d], c + DW);
            if constexpr (SV) {
                if (d == 0) load_sv(svn, c / 4 + 1);
            }
            __syncthreads();
        }
    }

    // D[i][j] of a 16x16 tile: lane l holds rows 4(l/16) .. 4(l/16)+3 of column l%16.
#pragma unroll
    for (int s = 0; s < NBW; ++s) {
        const int n = (t0 + wave + 4 * s) * 16 + r16;
        if (!tok[s] || n >= N) continue;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + mt * 16 + 4 * g + v;
                if (m < M) store_out(y, (size_t)m * N + n, acc[mt][s][v], y_dtype);
            }
    }
}

// Prefetch depths in chunks, measured on MI355X: weights (from HBM) four
// chunks ahead (six measured the same up to 64 rows, eight slower);
// activations (mostly L2 hits) two ahead.  Each iteration issues its activation loads
// before its weight loads: a wave's loads complete in issue order, so the
// wait for an activation chunk only covers older weight loads.  Above 64
// rows M is split into blocks of MT_L = 4 m-tiles.
#ifndef QMV_MFMA_DW_S
#define QMV_MFMA_DW_S 4
#endif
#ifndef QMV_MFMA_DW_L
#define QMV_MFMA_DW_L 4
#endif
#ifndef QMV_MFMA_DX
#define QMV_MFMA_DX 2
#endif
#ifndef QMV_MFMA_MT_L
#define QMV_MFMA_MT_L 4
#endif

template <int MT, int NBW, int DW>
static hipError_t mfma_launch(const MatvecArgs &a, int NT, int ranges, int mblocks, hipStream_t st) {
    const dim3 grid(ranges, mblocks);
    const auto *wq = reinterpret_cast<const uint8_t *>(a.wq);
    const auto *sc = reinterpret_cast<const uint8_t *>(a.sc);
    if (a.K % 128 == 0)
        hipLaunchKernelGGL((k_mxfp4_mfma<MT, NBW, DW, QMV_MFMA_DX, true>), grid, dim3(kMfmaThreads), 0, st, wq, sc,
                           a.x, a.y, a.y_dtype, a.M, a.N, a.K, NT, ranges);
    else
        hipLaunchKernelGGL((k_mxfp4_mfma<MT, NBW, DW, QMV_MFMA_DX, false>), grid, dim3(kMfmaThreads), 0, st, wq,
                           sc, a.x, a.y, a.y_dtype, a.M, a.N, a.K, NT, ranges);
    return hipGetLastError();
}

// Weight tiles per wave: the fewest (at most four) that keep the workgroups
// (ranges x m-blocks) within `slots`.  More tiles per wave means more matrix
// ops per activation fragment read from LDS.  With one m-block the ranges
// are then spread over every slot (one per CU): more ranges only shorten
// them, so none spans more than 4 * nbw tiles, and the per-CU share of the
// weights drops from 4 * nbw tiles to NT / CUs (measured on MI355X at
// N = 21504, K = 5376: M = 32 29.9 -> 27.6 us, M = 64 38.0 -> 37.2 us).
template <int MT, int DW>
static hipError_t mfma_nbw(const MatvecArgs &a, int NT, int mblocks, long slots, hipStream_t st) {
    int nbw = 1;
    while (nbw < 4 && (long)((NT + 4 * nbw - 1) / (4 * nbw)) * mblocks > slots) ++nbw;
    int ranges = (NT + 4 * nbw - 1) / (4 * nbw);  // every range spans <= 4 * nbw tiles
    if (mblocks == 1 && ranges < slots) ranges = (int)(NT < slots ? NT : slots);
    if (nbw == 1) return mfma_launch<MT, 1, DW>(a, NT, ranges, mblocks, st);
    if (nbw == 2) return mfma_launch<MT, 2, DW>(a, NT, ranges, mblocks, st);
    if (nbw == 3) return mfma_launch<MT, 3, DW>(a, NT, ranges, mblocks, st);
    return mfma_launch<MT, 4, DW>(a, NT, ranges, mblocks, st);
}

// Up to 64 rows one block holds all of M and the weight ring is deep (the op
// is bound by HBM there); above that M is split into blocks of MT m-tiles.
hipError_t launch_mxfp4_mfma(const MatvecArgs &a, hipStream_t st) {
    if (a.fmt != FMT_MXFP4 || a.M < 32 || a.M > 256 || a.K % 32 != 0) return hipErrorInvalidValue;
    const int NT = (a.N + 15) / 16;
    const int cus = device_cus();
    const int mt = (a.M + 15) / 16;
    constexpr int MTL = QMV_MFMA_MT_L;
    if (mt <= 2) return mfma_nbw<2, QMV_MFMA_DW_S>(a, NT, 1, cus, st);
    if (mt <= 4) return mfma_nbw<4, QMV_MFMA_DW_S>(a, NT, 1, cus, st);
    // two m-blocks: one workgroup per CU (N = 21504, K = 5376, M = 96 / 128:
    // 51.1 / 52.5 us against 53.3 / 56.4 with two per CU); three or four: two
    // per CU (one per CU measured 71 / 98 us against 69 / 86 at M = 192 / 256)
    const int mblocks = (mt + MTL - 1) / MTL;
    return mfma_nbw<MTL, QMV_MFMA_DW_L>(a, NT, mblocks, (mblocks <= 2 ? 1L : 2L) * cus, st);
}

}  // namespace qmv
