// qmv_measure.hip -- the reference kernels of include/qmv_measure.h: a plain
// streaming read (the clean-stream ceiling on this GPU) and an empty kernel
// (the dispatch floor).  Measurement only; nothing of the method runs here.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmv_measure.h"

namespace {

typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

// One 16-byte non-temporal load per lane and step, grid-stride: the access
// pattern that measured fastest for a cold multi-hundred-megabyte read on
// MI355X (one load in flight per lane, a few thousand workgroups).
__global__ __launch_bounds__(256) void k_stream_read(const uint8_t *__restrict__ src, uint32_t nvec_lo,
                                                     uint32_t nvec_hi, uint32_t *sink) {
    const uint64_t nvec = ((uint64_t)nvec_hi << 32) | nvec_lo;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    for (uint64_t v = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
        const u4_t w = __builtin_nontemporal_load(reinterpret_cast<const u4_t *>(src) + v);
        acc ^= w.x ^ w.y ^ w.z ^ w.w;
    }
    // one word per workgroup: lane 0 of wave 0 after a wave reduction is
    // enough to keep every load live
    for (int s = 32; s >= 1; s >>= 1) acc ^= __shfl_xor(acc, s, 64);
    __shared__ uint32_t wsum[4];
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = wsum[0] ^ wsum[1] ^ wsum[2] ^ wsum[3];
}

__global__ void k_empty() {}

}  // namespace

extern "C" {

int qmv_measure_stream_read(const void *src, size_t bytes, uint32_t *sink, int grid, void *stream) {
    if (src == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0) return 1;
    if (reinterpret_cast<uintptr_t>(src) % 16 != 0) return 1;
    if (grid <= 0) grid = 2048;
    const uint64_t nvec = bytes / 16;
    hipLaunchKernelGGL(k_stream_read, dim3((unsigned)grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint8_t *>(src), (uint32_t)nvec, (uint32_t)(nvec >> 32), sink);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

int qmv_measure_empty(void *stream) {
    hipLaunchKernelGGL(k_empty, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
