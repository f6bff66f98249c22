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

constexpr int kBlock = 256;  // 4 waves of 64
constexpr int kWaves = kBlock / 64;
constexpr int kMaxGrid = 2048;

bool pick_shape(int nseg, LaneShape &s) {
    if (nseg <= 0) return false;
    if (nseg <= 8) s = {8, 1, 1};
    else if (nseg <= 16) s = {16, 1, 1};
    else if (nseg <= 24) s = {8, 3, 4};
    else if (nseg <= 32) s = {32, 1, 1};
    else if (nseg <= 64) s = {64, 1, 1};
    else if (nseg <= 128) s = {64, 2, 2};
    else if (nseg <= 192) s = {64, 3, 4};
    else if (nseg <= 256) s = {64, 4, 4};
    else if (nseg <= 512) s = {64, 8, 8};
    else return false;
    return true;
}

static inline int pow2_ceil(int n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

// ---------------------------------------------------------------------------
// Activation staging: rows m0 .. m0+MC-1 of x[M][K] -> LDS xs[MC][K]
// (zeros for rows beyond M).  16-byte vector copies.
template <int MC>
__device__ __forceinline__ void stage_x(const uint16_t *__restrict__ x, uint16_t *xs, int M, int K,
                                        int m0) {
    const int per_row = K / 8;
    for (int e = threadIdx.x; e < MC * per_row; e += blockDim.x) {
        const int m = e / per_row, kk = e - m * per_row;
        u4_t v = {0u, 0u, 0u, 0u};
        if (m0 + m < M) v = *reinterpret_cast<const u4_t *>(x + (size_t)(m0 + m) * K + 8 * kk);
        *reinterpret_cast<u4_t *>(xs + (size_t)m * K + 8 * kk) = v;
    }
}

// ---------------------------------------------------------------------------
// The FO row engine.  NMAT weight matrices (1, or 2 for gate/up) share the
// activation chunk.  For every row group the wave produces, in lane q == 0 of
// each RL-lane group, the reduced totals tot[mat][m] (before the int2 row
// scale) and hands them to the epilogue.
template <int F, int RL, int NI, int NIP, int MC, bool XREG, int NMAT, class Epi>
__device__ __forceinline__ void fo_rows(const uint8_t *const (&wq)[NMAT],
                                        const void *const (&sc)[NMAT], const uint16_t *xs, int N,
                                        int K, Epi &epi) {
    constexpr int CODES = SegCodes<F>::v;
    constexpr int XV = CODES / 8;  // 16-byte activation vectors per segment per column
    constexpr int RPG = 64 / RL;   // rows per wave per iteration
    const int nseg = K / CODES;
    int P2 = 1;
    while (P2 < nseg) P2 <<= 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane % RL, rsub = lane / RL;
    const size_t row_bytes = (size_t)nseg * 16;
    const int total_rg = (N + RPG - 1) / RPG;
    const int nwaves = gridDim.x * kWaves;

    u4_t xr[XREG ? NI : 1][XREG ? MC : 1][XREG ? XV : 1];
    if constexpr (XREG) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int j = q + RL * i;
#pragma unroll
            for (int m = 0; m < MC; ++m)
#pragma unroll
                for (int v = 0; v < XV; ++v)
                    xr[i][m][v] = (j < nseg)
                                      ? *reinterpret_cast<const u4_t *>(xs + (size_t)m * K + j * CODES + 8 * v)
                                      : u4_t{0u, 0u, 0u, 0u};
        }
    }

    for (int rg = blockIdx.x * kWaves + wave; rg < total_rg; rg += nwaves) {
        const int n = rg * RPG + rsub;
        const int nl = n < N ? n : N - 1;
        u4_t w[NMAT][NI];
        float segscale[NMAT][NI];
#pragma unroll
        for (int t = 0; t < NMAT; ++t)
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int j = q + RL * i;
                w[t][i] = u4_t{0u, 0u, 0u, 0u};
                segscale[t][i] = 0.0f;
                if (j < nseg) {
                    w[t][i] = __builtin_nontemporal_load(
                        reinterpret_cast<const u4_t *>(wq[t] + (size_t)nl * row_bytes + (size_t)j * 16));
                    if constexpr (F == FMT_INT4)
                        segscale[t][i] = half_bits_to_f32(
                            reinterpret_cast<const uint16_t *>(sc[t])[(size_t)nl * nseg + j]);
                    else if constexpr (F == FMT_MXFP4)
                        segscale[t][i] =
                            e8m0_to_f32(reinterpret_cast<const uint8_t *>(sc[t])[(size_t)nl * nseg + j]);
                }
            }
        float tot[NMAT][MC];
#pragma unroll
        for (int t = 0; t < NMAT; ++t) {
            float v[MC][NIP];
#pragma unroll
            for (int m = 0; m < MC; ++m)
#pragma unroll
                for (int a = 0; a < NIP; ++a) v[m][a] = 0.0f;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int j = q + RL * i;
                if (j < nseg) {
                    float acc[MC];
#pragma unroll
                    for (int m = 0; m < MC; ++m) acc[m] = 0.0f;
                    if constexpr (XREG) {
                        segment_sum<F, MC>(w[t][i], [&](int m, int vv) { return xr[i][m][vv]; }, acc);
                    } else {
                        const uint16_t *xseg = xs + (size_t)j * CODES;
                        segment_sum<F, MC>(
                            w[t][i],
                            [&](int m, int vv) {
                                return *reinterpret_cast<const u4_t *>(xseg + (size_t)m * K + 8 * vv);
                            },
                            acc);
                    }
#pragma unroll
                    for (int m = 0; m < MC; ++m) {
                        if constexpr (F == FMT_INT2) v[m][i] = acc[m];
                        else if constexpr (F == FMT_INT4) v[m][i] = segscale[t][i] * acc[m];
                        else v[m][i] = acc[m] * segscale[t][i];
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < MC; ++m) tot[t][m] = fo_tree<RL, NIP>(v[m], P2);
        }
        epi(n, nl, q, tot);
    }
}

// ---------------------------------------------------------------------------
// Plain matvec / skinny GEMM.
template <int F, int MC>
struct StoreEpi {
    const uint16_t *row_scale;  // int2 only
    void *y;
    int y_dtype, M, N, m0;
    __device__ __forceinline__ void operator()(int n, int nl, int q, const float (&tot)[1][MC]) {
        float s = 1.0f;
        if constexpr (F == FMT_INT2) s = half_bits_to_f32(row_scale[nl]);
        if (q != 0 || n >= N) return;
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            if (m0 + m < M) {
                float r = tot[0][m];
                if constexpr (F == FMT_INT2) r = s * r;
                store_out(y, (size_t)(m0 + m) * N + n, r, y_dtype);
            }
        }
    }
};

template <int F, int RL, int NI, int NIP, int MC, bool XREG>
__global__ __launch_bounds__(kBlock) void k_fo_matvec(const uint8_t *__restrict__ wq,
                                                      const void *__restrict__ sc,
                                                      const uint16_t *__restrict__ x, void *y,
                                                      int y_dtype, int M, int N, int K) {
    extern __shared__ __align__(16) uint16_t xs[];
    const int m0 = blockIdx.y * MC;
    stage_x<MC>(x, xs, M, K, m0);
    __syncthreads();
    StoreEpi<F, MC> epi{reinterpret_cast<const uint16_t *>(sc), y, y_dtype, M, N, m0};
    const uint8_t *const w1[1] = {wq};
    const void *const s1[1] = {sc};
    fo_rows<F, RL, NI, NIP, MC, XREG, 1>(w1, s1, xs, N, K, epi);
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

template <int MC>
struct GateUpEpi {
    const uint16_t *s_gate, *s_up;
    uint16_t *out;
    int M, N, m0;
    __device__ __forceinline__ void operator()(int n, int nl, int q, const float (&tot)[2][MC]) {
        const float sg = half_bits_to_f32(s_gate[nl]);
        const float su = half_bits_to_f32(s_up[nl]);
        if (q != 0 || n >= N) return;
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            if (m0 + m < M) {
                const float g = sg * tot[0][m];
                const float u = su * tot[1][m];
                const float ge = qmv_gelu(g);
                const float o = ge * u;
                out[(size_t)(m0 + m) * N + n] = __builtin_bit_cast(uint16_t, to_f16(o));
            }
        }
    }
};

template <int RL, int NI, int NIP, int MC, bool XREG>
__global__ __launch_bounds__(kBlock) void k_fo_gateup(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ residual,
    uint16_t *residual_out, const uint16_t *__restrict__ gamma, float eps,
    const uint32_t *__restrict__ wq_gate, const uint16_t *__restrict__ s_gate,
    const uint32_t *__restrict__ wq_up, const uint16_t *__restrict__ s_up, uint16_t *out, int M,
    int N, int K) {
    extern __shared__ __align__(16) uint16_t smem[];
    uint16_t *xs = smem;  // [MC][K]: h, then overwritten in place by the normalised xn
    float *inv_s = reinterpret_cast<float *>(smem + (size_t)MC * K);
    const int m0 = blockIdx.y * MC;
    rmsnorm_prologue<MC>(x, residual, gamma, residual_out, eps, M, K, m0, xs, xs, inv_s);
    GateUpEpi<MC> epi{s_gate, s_up, out, M, N, m0};
    const uint8_t *const w2[2] = {reinterpret_cast<const uint8_t *>(wq_gate),
                                  reinterpret_cast<const uint8_t *>(wq_up)};
    const void *const s2[2] = {s_gate, s_up};
    fo_rows<FMT_INT2, RL, NI, NIP, MC, XREG, 2>(w2, s2, xs, N, K, epi);
}

// ---------------------------------------------------------------------------
// int2 lm_head + argmax.  Each lane keeps the best key of the rows it
// produced; the workgroup reduces them, writes one key per activation row to
// the workspace, and the last workgroup to finish (completion counter) reduces
// all keys, writes idx / maxval and resets the counter to zero.
template <int MC>
struct ArgmaxEpi {
    const uint16_t *row_scale;
    float *logits;
    int M, N, m0;
    uint64_t best[MC];
    __device__ __forceinline__ void operator()(int n, int nl, int q, const float (&tot)[1][MC]) {
        const float s = half_bits_to_f32(row_scale[nl]);
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
                                                      int K, uint64_t *partial, uint32_t *counter) {
    extern __shared__ __align__(16) uint16_t xs[];
    __shared__ uint64_t wbest[kWaves][MC];
    __shared__ int is_last;
    const int m0 = blockIdx.y * MC;
    stage_x<MC>(x, xs, M, K, m0);
    __syncthreads();
    ArgmaxEpi<MC> epi{scale, logits, M, N, m0, {}};
#pragma unroll
    for (int m = 0; m < MC; ++m) epi.best[m] = 0ull;
    const uint8_t *const w1[1] = {reinterpret_cast<const uint8_t *>(wq)};
    const void *const s1[1] = {scale};
    fo_rows<FMT_INT2, RL, NI, NIP, MC, XREG, 1>(w1, s1, xs, N, K, epi);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int m = 0; m < MC; ++m) {
        const uint64_t b = wave_max_u64(epi.best[m]);
        if (lane == 0) wbest[wave][m] = b;
    }
    __syncthreads();
    uint64_t *slot = partial + ((size_t)blockIdx.y * gridDim.x + blockIdx.x) * MC;
    if (threadIdx.x < MC) {
        uint64_t b = 0;
        for (int w = 0; w < kWaves; ++w) b = wbest[w][threadIdx.x] > b ? wbest[w][threadIdx.x] : b;
        __hip_atomic_store(&slot[threadIdx.x], b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t ticket = __hip_atomic_fetch_add(&counter[blockIdx.y], 1u, __ATOMIC_ACQ_REL,
                                                       __HIP_MEMORY_SCOPE_AGENT);
        is_last = (ticket == gridDim.x - 1) ? 1 : 0;
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    const uint64_t *chunk = partial + (size_t)blockIdx.y * gridDim.x * MC;
    for (int m = wave; m < MC; m += kWaves) {
        uint64_t b = 0;
        for (int g = lane; g < (int)gridDim.x; g += 64) {
            const uint64_t v = __hip_atomic_load(&chunk[(size_t)g * MC + m], __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
            b = v > b ? v : b;
        }
        b = wave_max_u64(b);
        if (lane == 0 && m0 + m < M) {
            int n;
            float yv;
            argmax_key_decode(b, n, yv);
            idx[m0 + m] = n;
            if (maxval != nullptr) maxval[m0 + m] = yv;
        }
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

static int grid_for(int N, int RL) {
    const int rpg = 64 / RL;
    const long total_rg = ((long)N + rpg - 1) / rpg;
    long g = (total_rg + kWaves - 1) / kWaves;
    if (g > kMaxGrid) g = kMaxGrid;
    if (g < 1) g = 1;
    return (int)g;
}

// M = 1 keeps the activation slice in registers (MC = 1); wider M uses
// chunks of 4 activation rows read from LDS.
constexpr int kMcWide = 4;

// Registers a lane spends on its activation slice when MC = 1 (16-byte
// vectors x 4 VGPRs); above this budget the slice is read from LDS instead.
constexpr int kXregBudget = 96;

// Dynamic LDS per workgroup is kept within 64 KB; chunks of kMcWide
// activation rows are used when they fit, single rows otherwise.
constexpr size_t kLdsBudget = 65536;
static inline bool wide_fits(int K, int copies) {
    return (size_t)copies * kMcWide * K * 2 + 64 * kMcWide <= kLdsBudget;
}

template <int F, int NI>
constexpr bool xreg_fits() {
    return NI * (SegCodes<F>::v / 8) * 4 <= kXregBudget;
}

template <int F, int RL, int NI, int NIP>
static hipError_t fo_matvec_shape(const MatvecArgs &a, hipStream_t st) {
    const int grid = grid_for(a.N, RL);
    const uint8_t *wq = reinterpret_cast<const uint8_t *>(a.wq);
    if (a.M == 1) {
        constexpr bool xreg = xreg_fits<F, NI>();
        hipLaunchKernelGGL((k_fo_matvec<F, RL, NI, NIP, 1, xreg>), dim3(grid, 1), dim3(kBlock),
                           (size_t)a.K * 2, st, wq, a.sc, a.x, a.y, a.y_dtype, a.M, a.N, a.K);
    } else if (wide_fits(a.K, 1)) {
        const size_t lds = (size_t)kMcWide * a.K * 2;
        const int gy = (a.M + kMcWide - 1) / kMcWide;
        hipLaunchKernelGGL((k_fo_matvec<F, RL, NI, NIP, kMcWide, false>), dim3(grid, gy),
                           dim3(kBlock), lds, st, wq, a.sc, a.x, a.y, a.y_dtype, a.M, a.N, a.K);
    } else {
        hipLaunchKernelGGL((k_fo_matvec<F, RL, NI, NIP, 1, false>), dim3(grid, a.M), dim3(kBlock),
                           (size_t)a.K * 2, st, wq, a.sc, a.x, a.y, a.y_dtype, a.M, a.N, a.K);
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
    case 6422: return FN<64, 2, 2>(__VA_ARGS__);                            \
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

hipError_t launch_fo_matvec(const MatvecArgs &a, hipStream_t st) {
    const int codes = a.fmt == FMT_INT2 ? 64 : 32;
    LaneShape sh;
    if (!pick_shape(a.K / codes, sh)) return hipErrorInvalidValue;
    if (a.fmt == FMT_INT2) { QMV_SHAPE_SWITCH(mv_int2, a, st) }
    if (a.fmt == FMT_INT4) { QMV_SHAPE_SWITCH(mv_int4, a, st) }
    QMV_SHAPE_SWITCH(mv_mxfp4, a, st)
}

template <int RL, int NI, int NIP>
static hipError_t gu_shape(const GateUpArgs &a, hipStream_t st) {
    const int grid = grid_for(a.N, RL);
    if (a.M == 1 || !wide_fits(a.K, 1)) {
        const size_t lds = (size_t)a.K * 2 + 64;
        if (a.M == 1)
            hipLaunchKernelGGL((k_fo_gateup<RL, NI, NIP, 1, xreg_fits<FMT_INT2, NI>()>), dim3(grid, 1),
                               dim3(kBlock), lds, st, a.x, a.residual, a.residual_out, a.gamma, a.eps,
                               a.wq_gate, a.s_gate, a.wq_up, a.s_up, a.out, a.M, a.N, a.K);
        else
            hipLaunchKernelGGL((k_fo_gateup<RL, NI, NIP, 1, false>), dim3(grid, a.M), dim3(kBlock), lds,
                               st, a.x, a.residual, a.residual_out, a.gamma, a.eps, a.wq_gate,
                               a.s_gate, a.wq_up, a.s_up, a.out, a.M, a.N, a.K);
    } else {
        const size_t lds = (size_t)kMcWide * a.K * 2 + 64 * kMcWide;
        const int gy = (a.M + kMcWide - 1) / kMcWide;
        hipLaunchKernelGGL((k_fo_gateup<RL, NI, NIP, kMcWide, false>), dim3(grid, gy), dim3(kBlock),
                           lds, st, a.x, a.residual, a.residual_out, a.gamma, a.eps, a.wq_gate,
                           a.s_gate, a.wq_up, a.s_up, a.out, a.M, a.N, a.K);
    }
    return hipGetLastError();
}

hipError_t launch_fo_gateup(const GateUpArgs &a, hipStream_t st) {
    LaneShape sh;
    if (!pick_shape(a.K / 64, sh)) return hipErrorInvalidValue;
    QMV_SHAPE_SWITCH(gu_shape, a, st)
}

// Activation rows per argmax workgroup chunk, and the number of chunks.
static void argmax_chunks(int M, int K, int &mc, int &gy) {
    mc = (M > 1 && wide_fits(K, 1)) ? kMcWide : 1;
    gy = (M + mc - 1) / mc;
}

constexpr size_t kCounterBytes = 1024;  // one 32-bit completion counter per chunk (<= 256)

size_t argmax_workspace_bytes(int M, int N, int K) {
    LaneShape sh;
    if (M < 1 || N < 1 || !pick_shape(K / 64, sh)) return 0;
    int mc, gy;
    argmax_chunks(M, K, mc, gy);
    const size_t partial = (size_t)gy * grid_for(N, sh.RL) * mc * sizeof(uint64_t);
    return kCounterBytes + ((partial + 255) / 256) * 256;  // counters, then partial keys
}

template <int RL, int NI, int NIP>
static hipError_t am_shape(const ArgmaxArgs &a, hipStream_t st) {
    const int grid = grid_for(a.N, RL);
    uint32_t *counter = reinterpret_cast<uint32_t *>(a.ws);
    uint64_t *partial = reinterpret_cast<uint64_t *>(reinterpret_cast<uint8_t *>(a.ws) + kCounterBytes);
    int mc, gy;
    argmax_chunks(a.M, a.K, mc, gy);
    if (a.M == 1) {
        hipLaunchKernelGGL((k_fo_argmax<RL, NI, NIP, 1, xreg_fits<FMT_INT2, NI>()>), dim3(grid, 1),
                           dim3(kBlock), (size_t)a.K * 2, st, a.wq, a.scale, a.x, a.idx, a.maxval,
                           a.logits, a.M, a.N, a.K, partial, counter);
    } else if (mc == 1) {
        hipLaunchKernelGGL((k_fo_argmax<RL, NI, NIP, 1, false>), dim3(grid, gy), dim3(kBlock),
                           (size_t)a.K * 2, st, a.wq, a.scale, a.x, a.idx, a.maxval, a.logits, a.M,
                           a.N, a.K, partial, counter);
    } else {
        hipLaunchKernelGGL((k_fo_argmax<RL, NI, NIP, kMcWide, false>), dim3(grid, gy), dim3(kBlock),
                           (size_t)kMcWide * a.K * 2, st, a.wq, a.scale, a.x, a.idx, a.maxval,
                           a.logits, a.M, a.N, a.K, partial, counter);
    }
    return hipGetLastError();
}

hipError_t launch_fo_argmax(const ArgmaxArgs &a, hipStream_t st) {
    LaneShape sh;
    if (!pick_shape(a.K / 64, sh)) return hipErrorInvalidValue;
    QMV_SHAPE_SWITCH(am_shape, a, st)
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
