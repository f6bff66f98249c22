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
// Work split (MI355X: 256 CUs in 8 XCDs, one matrix core per SIMD):
//  * The output is cut into blocks of BM = 64 activation rows (4 m-tiles of
//    16) by a contiguous range of 16-row weight tiles.  With S = ceil(M/64)
//    row blocks, 256/S ranges make one workgroup per CU.  Workgroups of the
//    same weight range get block indices that are equal modulo 8, i.e. the
//    same XCD (workgroups go to XCDs round-robin), so the S reads of a weight
//    range meet in that XCD's L2 instead of going to HBM S times.
//  * Per chunk of K (128 = four MXFP4 blocks) the workgroup copies its
//    activation tile [64][128] bf16 to LDS with fully coalesced loads
//    (double buffered, one barrier per chunk).
//  * The 4 waves split the weight tiles of the range (tile t goes to wave
//    t mod 4), so every weight byte is loaded and dequantized once; each
//    wave multiplies its tiles by all 4 m-tiles read from LDS.
//  * Lane group g = lane / 16 holds the whole 16-byte MXFP4 block 4c + g of
//    its weight row (one dwordx4 plus the scale byte); sub-step j hands dword
//    j (8 codes) to the MFMA, and the A fragment of lane group g, sub-step j
//    is read from the same k range, so both operands map (g, element e) of
//    sub-step j to k = 128c + 32g + 8j + e.
#include "qmv_device.hpp"
#include "qmv_internal.hpp"

namespace qmv {

typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int kMfmaWaves = 4;
constexpr uint32_t kOob = 0xFFFFFFF0u;  // past every buffer: loads return 0
#ifndef QMV_MFMA_WAUX
#define QMV_MFMA_WAUX 2
#endif

constexpr int kMT = 4;                  // m-tiles (of 16 rows) per workgroup
constexpr int kXRow = 128 * 2 + 16;     // LDS bytes per activation row of a chunk (+16: bank spread)
constexpr int kXBuf = kMT * 16 * kXRow;  // one LDS buffer

// Loads of one chunk: the weight tiles of a wave (dwordx4 + scale byte per
// lane and tile) and this thread's 64-byte share of the activation tile.
template <int NW>
struct ChunkSlot {
    u4_t w[NW];
    uint32_t e[NW];
    u4_t x[4];
};

// Chunks in flight besides the one being multiplied.  Both the weights (from
// HBM) and the activation tile (from L2) travel D chunks ahead; a wave with
// few tiles has little matrix work per chunk to cover that latency with.
template <int NW>
constexpr int mfma_depth() {
    return NW <= 2 ? 4 : (NW <= 4 ? 3 : 2);
}

template <int NW>
__global__ __launch_bounds__(kMfmaWaves * 64) void k_mxfp4_mfma(
    const uint8_t *__restrict__ wq, const uint8_t *__restrict__ e8m0, const uint16_t *__restrict__ x,
    void *y, int y_dtype, int M, int N, int K, int NT, int S, int ranges, int xcd_map) {
    constexpr int D = mfma_depth<NW>();
    __shared__ __align__(16) uint8_t xs[2][kXBuf];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    // block index -> (weight range, row block); see the work split above
    const int b = blockIdx.x;
    int rg, sb;
    if (xcd_map) {
        sb = (b >> 3) % S;
        rg = (b & 7) + 8 * (b / (8 * S));
    } else {
        sb = b % S;
        rg = b / S;
    }
    const int t0 = (int)(((long)rg * NT) / ranges);
    const int t1 = (int)(((long)(rg + 1) * NT) / ranges);
    const int m0 = sb * kMT * 16;

    const int nseg = K >> 5;
    const int nchunk = (nseg + 3) >> 2;
    const uint32_t row_bytes = (uint32_t)K >> 1;
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(wq), 0, (uint32_t)N * row_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t re =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(e8m0), 0, (uint32_t)N * nseg, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(x), 0, (uint32_t)M * (uint32_t)K * 2u, 0x00020000);

    // this wave's tiles: t0 + wave + 4i, i < NW
    uint32_t wrow[NW], erow[NW];
    bool tok[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int t = t0 + wave + 4 * i;
        const uint32_t n = (uint32_t)t * 16u + r16;
        tok[i] = t < t1;
        wrow[i] = n * row_bytes + 16u * g;
        erow[i] = n * (uint32_t)nseg + g;
    }
    // activation tile copy: thread -> (row tid/4, 64-byte quarter tid%4) of the
    // [64][256 B] chunk; rows >= M read 0 (past the buffer)
    const int xr_row = tid >> 2, xr_q = tid & 3;
    const uint32_t xg = (uint32_t)(m0 + xr_row) * (uint32_t)K * 2u + 64u * xr_q;
    auto load = [&](ChunkSlot<NW> &sl, int c) {
        const bool segok = 4 * c + g < nseg;  // the last chunk may hold fewer than 4 blocks
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const bool ok = segok && tok[i];
            sl.w[i] = __builtin_bit_cast(
                u4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, ok ? wrow[i] + 64u * c : kOob, 0, QMV_MFMA_WAUX));
            sl.e[i] = __builtin_amdgcn_raw_buffer_load_b8(re, ok ? erow[i] + 4u * c : kOob, 0, 0);
        }
        // chunks past the end read nothing (out of range)
        const uint32_t xo = c < nchunk ? xg + 256u * c : kOob;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            sl.x[j] = __builtin_bit_cast(
                u4_t, __builtin_amdgcn_raw_buffer_load_b128(rx, xo == kOob ? kOob : xo + 16u * j, 0, 0));
    };

    f4_t acc[kMT][NW];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int i = 0; i < NW; ++i) acc[mt][i] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

    ChunkSlot<NW> slot[D];
#pragma unroll
    for (int d = 0; d < D; ++d) load(slot[d], d);

    // Chunk c: its activations go to LDS buffer c&1, one barrier makes them
    // visible (every wave has then also finished chunk c-1, the last reader of
    // the other buffer, and chunk c-2, the last reader of this one), the slot
    // is refilled with chunk c+D, and the tile products are accumulated.
    for (int c0 = 0; c0 < nchunk; c0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int c = c0 + d;
            if (c < nchunk) {  // uniform across the workgroup
                const ChunkSlot<NW> cur = slot[d];
                uint8_t *xb = xs[c & 1];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<u4_t *>(&xb[xr_row * kXRow + 64 * xr_q + 16 * j]) = cur.x[j];
                __syncthreads();
                load(slot[d], c + D);
                float sc[NW];
#pragma unroll
                for (int i = 0; i < NW; ++i) sc[i] = e8m0_to_f32(cur.e[i]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    bf8_t bw[NW];
#pragma unroll
                    for (int i = 0; i < NW; ++i) {
                        const uint32_t wd = cur.w[i][j];
                        const bf2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc[i], 0);
                        const bf2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc[i], 1);
                        const bf2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc[i], 2);
                        const bf2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc[i], 3);
                        bw[i] = bf8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
                    }
#pragma unroll
                    for (int mt = 0; mt < kMT; ++mt) {
                        const bf8_t a = __builtin_bit_cast(
                            bf8_t, *reinterpret_cast<const u4_t *>(xb + (mt * 16 + r16) * kXRow + 64 * g + 16 * j));
#pragma unroll
                        for (int i = 0; i < NW; ++i)
                            acc[mt][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bw[i], acc[mt][i], 0, 0, 0);
                    }
                }
            }
        }
    }

    // D[i][j] of a 16x16 tile: lane l holds rows 4(l/16) .. 4(l/16)+3 of column l%16.
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int n = (t0 + wave + 4 * i) * 16 + r16;
        if (!tok[i] || n >= N) continue;
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + mt * 16 + 4 * g + v;
                if (m < M) store_out(y, (size_t)m * N + n, acc[mt][i][v], y_dtype);
            }
    }
}

// Tiles per wave compiled (a range holds up to 4 * NW tiles).
constexpr int kMfmaMaxNw = 6;

template <int NW>
static hipError_t mfma_launch(const MatvecArgs &a, int NT, int S, int ranges, hipStream_t st) {
    const int xcd_map = (ranges % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((k_mxfp4_mfma<NW>), dim3(S * ranges), dim3(kMfmaWaves * 64), 0, st,
                       reinterpret_cast<const uint8_t *>(a.wq), reinterpret_cast<const uint8_t *>(a.sc), a.x,
                       a.y, a.y_dtype, a.M, a.N, a.K, NT, S, ranges, xcd_map);
    return hipGetLastError();
}

hipError_t launch_mxfp4_mfma(const MatvecArgs &a, hipStream_t st) {
    if (a.fmt != FMT_MXFP4 || a.M < 32 || a.M > 256 || a.K % 32 != 0) return hipErrorInvalidValue;
    const int NT = (a.N + 15) / 16;
    const int S = (a.M + kMT * 16 - 1) / (kMT * 16);  // row blocks of 64
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    int ranges = cus / S;
    if (ranges < 1) ranges = 1;
    if (ranges > NT) ranges = NT;
    int per = (NT + ranges - 1) / ranges;  // tiles per range (at most)
    if (per > 4 * kMfmaMaxNw) {
        per = 4 * kMfmaMaxNw;
        ranges = (NT + per - 1) / per;
    }
    const int nw = (per + 3) / 4;  // tiles per wave (at most)
    if (nw <= 1) return mfma_launch<1>(a, NT, S, ranges, st);
    if (nw <= 2) return mfma_launch<2>(a, NT, S, ranges, st);
    if (nw <= 3) return mfma_launch<3>(a, NT, S, ranges, st);
    if (nw <= 4) return mfma_launch<4>(a, NT, S, ranges, st);
    return mfma_launch<6>(a, NT, S, ranges, st);
}

}  // namespace qmv
