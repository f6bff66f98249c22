// qmv_internal.hpp -- host-side launch interface between the C ABI layer and
// the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

namespace qmv {

// Launch-shape facts computed on first use and kept: the CU count per
// device, and per (device, kernel, block size, LDS bytes) the workgroups one
// CU holds.  The values are fixed for a process, so a lookup only needs the
// table's short lock (host code only).
constexpr int kMaxDevices = 64;

inline int current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
    return dev;
}

inline int device_cus() {
    static std::atomic<int> cache[kMaxDevices];
    const int dev = current_device();
    int cus = cache[dev].load(std::memory_order_relaxed);
    if (cus <= 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            return 256;
        cache[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

template <class Kern>
inline int cached_occupancy(Kern kernel, int block, size_t lds) {
    struct Entry {
        const void *k;
        int dev, block;
        size_t lds;
        int occ;
    };
    static std::mutex mu;
    static Entry table[512];
    static int used = 0;
    const void *key = reinterpret_cast<const void *>(kernel);
    const int dev = current_device();
    {
        std::lock_guard<std::mutex> g(mu);
        for (int i = 0; i < used; ++i)
            if (table[i].k == key && table[i].dev == dev && table[i].block == block && table[i].lds == lds)
                return table[i].occ;
    }
    int occ = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, block, lds) != hipSuccess || occ < 1) occ = 1;
    std::lock_guard<std::mutex> g(mu);
    if (used < 512) table[used++] = Entry{key, dev, block, lds, occ};
    return occ;
}

// Per-row-group lane layout: RL lanes share one row, each lane owns the
// segments j = q + RL*a (a < NI); NIP = lane-local tree width (power of two).
struct LaneShape {
    int RL, NI, NIP;
};

// Chooses the lane layout for a row of `nseg` 16-byte segments; returns
// false if the row is longer than the compiled layouts allow.
bool pick_shape(int nseg, LaneShape &s);

struct MatvecArgs {
    int fmt;            // 0 int2, 1 int4, 2 mxfp4, 3 ternary
    const void *wq;     // packed rows, 16 bytes per segment (ternary: rows padded to whole segments)
    const void *sc;     // int2, ternary: fp16 [N]; int4: fp16 [N][K/32]; mxfp4: uint8 [N][K/32]
    const uint16_t *x;  // [M][K] fp16 or bf16
    void *y;            // [M][N]
    int y_dtype;
    int M, N, K;
    int seg_split = 0;      // segments per K split (0: the whole row)
    int splits = 1;         // K splits (grid z)
    float *part = nullptr;  // split partial sums [splits][M][N], or nullptr
};

hipError_t launch_fo_matvec(const MatvecArgs &a, hipStream_t stream);

// Split-K (tolerance class): the number of K splits chosen for a shape and
// the segments per split; 1 split means the fixed-order kernel is used.
int splitk_plan(int fmt, int M, int N, int K, int &seg_split);
size_t splitk_workspace_bytes(int fmt, int M, int N, int K);
// Partial sums of every split into `ws`, then their sum in increasing split
// order (plus the int2 row scale) into y.
hipError_t launch_splitk_matvec(const MatvecArgs &a, void *ws, hipStream_t stream);

// Matrix-core MXFP4 GEMM (tolerance class), 32 <= M <= 256.
hipError_t launch_mxfp4_mfma(const MatvecArgs &a, hipStream_t stream);

struct GateUpArgs {
    const uint16_t *x, *residual, *gamma;
    uint16_t *residual_out;
    float eps;
    const uint32_t *wq_gate, *wq_up;
    const uint16_t *s_gate, *s_up;
    uint16_t *out;  // fp16 [M][N] (with quantisation: the staging area in the workspace)
    int M, N, K;
    // MXFP4 quantisation of out (all null: none): codes [M][N/2], E8M0
    // [M][N/32], one arrival counter per block [M][N/32] (zero between calls)
    uint8_t *qcodes = nullptr, *qscale = nullptr;
    uint32_t *qcnt = nullptr;
};

hipError_t launch_fo_gateup(const GateUpArgs &a, hipStream_t stream);

// Workspace of the quantising gate/up: counters, then the fp16 staging area.
size_t gateup_mxfp4_workspace_bytes(int M, int N);

// fp16 [M][N] -> MXFP4 codes [M][N/2] + E8M0 [M][N/32], N a multiple of 32.
hipError_t launch_quant_mxfp4(const uint16_t *v, uint8_t *codes, uint8_t *scale, int M, int N,
                              hipStream_t stream);

// Shared-prologue q/k/v: index 0 = q, 1 = k, 2 = v.
struct QkvArgs {
    const uint16_t *x, *residual, *gamma;
    uint16_t *residual_out;
    float eps;
    const uint32_t *wq[3];
    const uint16_t *s[3];
    void *y[3];
    int N[3];
    int y_dtype, M, K;
};

hipError_t launch_fo_qkv(const QkvArgs &a, hipStream_t stream);

// Expert-gather MXFP4 matvec: y[m][j] = the fixed-order matvec of x[m] with
// expert idx[m][j]; experts are [E][N][K/2] weights + [E][N][K/32] scales.
struct GatherArgs {
    const uint8_t *wq, *e8m0;
    const uint16_t *x;
    const int32_t *idx;  // [M][topk]
    void *y;             // [M][topk][N]
    int y_dtype, E, topk, M, N, K;
};

hipError_t launch_fo_gather(const GatherArgs &a, hipStream_t stream);

struct ArgmaxArgs {
    const uint32_t *wq;
    const uint16_t *scale, *x;
    int32_t *idx;
    float *maxval, *logits;
    int M, N, K;
    void *ws;
};

size_t argmax_workspace_bytes(int M, int N, int K);
hipError_t launch_fo_argmax(const ArgmaxArgs &a, hipStream_t stream);

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t stream);

}  // namespace qmv
