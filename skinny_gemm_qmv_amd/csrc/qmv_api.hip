// qmv_api.hip -- the extern "C" entry points declared in include/qmv.h:
// argument validation, mode checks, workspace sizing and kernel dispatch.
// No allocation, no host synchronisation, no global mutable state apart
// from the per-thread text of the last HIP error and the per-device
// launch-shape caches of qmv_internal.hpp (idempotent values).
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "qmv.h"
#include "qmv_internal.hpp"

namespace {

// Scratch of qmv_int2_argmax_static: the argmax workspace (completion
// counters, then one 64-bit key per activation row) for up to QMV_MAX_M
// rows, in device memory the library owns, one copy per GPU for the life of
// the process.  Host code never uses the name `scratch` as an address: each
// device's address comes from hipGetSymbolAddress, taken once per device.
constexpr size_t kStaticScratchBytes = 1024 + ((QMV_MAX_M * 8 + 255) / 256) * 256;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_ptr[qmv::kMaxDevices];

thread_local char g_last_hip_error[256] = "";

qmv_status hip_status(hipError_t e) {
    if (e == hipSuccess) return QMV_OK;
    snprintf(g_last_hip_error, sizeof g_last_hip_error, "%s: %s", hipGetErrorName(e),
             hipGetErrorString(e));
    return QMV_ERR_HIP;
}

// Largest grid.y of a launch.
constexpr long kMaxGridY = 65535;

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t dtype_size(qmv_dtype d) { return d == QMV_F32 ? 4 : 2; }

bool valid_dtype(qmv_dtype d) { return d == QMV_F32 || d == QMV_F16 || d == QMV_BF16; }

bool valid_mode(qmv_mode m) {
    return m == QMV_MODE_FIXED || m == QMV_MODE_SPLITK || m == QMV_MODE_MFMA;
}

// Shape rules shared by every entry point: 1 <= M <= 256, N >= 1,
// K a positive multiple of `kmul`, K <= QMV_MAX_K.
bool valid_shape(int M, int N, int K, int kmul) {
    return M >= 1 && M <= QMV_MAX_M && N >= 1 && K >= kmul && K % kmul == 0 && K <= QMV_MAX_K;
}

// Kernels address each weight / scale tensor with 32-bit byte offsets
// (buffer loads), so one tensor must stay below 4 GiB.
bool fits_32bit(int N, int K, int codes_per_byte) {
    return (uint64_t)N * (uint64_t)(K / codes_per_byte) < (1ull << 32) - (1ull << 16);
}

qmv_status check_matvec(const void *wq, const void *sc, const void *x, const void *y,
                        qmv_dtype dt, int M, int N, int K, int kmul, qmv_mode mode) {
    if (!wq || !sc || !x || !y) return QMV_ERR_INVALID_ARG;
    if (!valid_shape(M, N, K, kmul) || !valid_dtype(dt) || !valid_mode(mode))
        return QMV_ERR_INVALID_ARG;
    if (!fits_32bit(N, K, kmul == 64 ? 4 : 2)) return QMV_ERR_UNSUPPORTED;
    // y (and split-K partials, fp32) are written with 32-bit byte offsets too
    if ((uint64_t)M * (uint64_t)N * 4u >= (1ull << 32) - (1ull << 16)) return QMV_ERR_UNSUPPORTED;
    if (!aligned(wq, 16) || !aligned(x, 16) || !aligned(y, dtype_size(dt)))
        return QMV_ERR_ALIGNMENT;
    return QMV_OK;
}

}  // namespace

extern "C" {

int qmv_abi_version(void) { return QMV_ABI_VERSION; }

const char *qmv_status_string(qmv_status s) {
    switch (s) {
    case QMV_OK: return "ok";
    case QMV_ERR_INVALID_ARG: return "invalid argument";
    case QMV_ERR_ALIGNMENT: return "misaligned pointer";
    case QMV_ERR_WORKSPACE: return "workspace missing or too small";
    case QMV_ERR_UNSUPPORTED: return "mode not supported for this operation or shape";
    case QMV_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

const char *qmv_last_hip_error(void) { return g_last_hip_error; }

void qmv_fo_spec(int *segment_bytes, int *tree_kind, int *inner_step) {
    if (segment_bytes) *segment_bytes = 16;
    if (tree_kind) *tree_kind = 1;
    if (inner_step) *inner_step = 1;
}

size_t qmv_workspace_size(qmv_op op, int M, int N, int K, qmv_mode mode) {
    if (op == QMV_OP_INT2_GATEUP_MXFP4) {
        if (mode != QMV_MODE_FIXED || !valid_shape(M, N, K, 64) || N % 32 != 0) return 0;
        return qmv::gateup_mxfp4_workspace_bytes(M, N);
    }
    if (op == QMV_OP_INT2_ARGMAX) {
        if (mode != QMV_MODE_FIXED || !valid_shape(M, N, K, 64)) return 0;
        return qmv::argmax_workspace_bytes(M, N, K);
    }
    if (mode == QMV_MODE_SPLITK && (op == QMV_OP_INT2 || op == QMV_OP_INT4 || op == QMV_OP_MXFP4)) {
        const int kmul = op == QMV_OP_INT2 ? 64 : 32;
        if (!valid_shape(M, N, K, kmul)) return 0;
        return qmv::splitk_workspace_bytes((int)op, M, N, K);
    }
    return 0;
}

qmv_status qmv_workspace_init(void *ws, size_t bytes, void *stream) {
    if (bytes == 0) return QMV_OK;
    if (!ws) return QMV_ERR_INVALID_ARG;
    if (!aligned(ws, 256) || bytes % 4 != 0) return QMV_ERR_ALIGNMENT;
    return hip_status(qmv::launch_fill_zero(ws, bytes, static_cast<hipStream_t>(stream)));
}

static qmv_status run_matvec(int fmt, const void *wq, const void *sc, const uint16_t *x, void *y,
                             qmv_dtype dt, int M, int N, int K, qmv_mode mode, void *ws, size_t ws_bytes,
                             void *stream) {
    qmv::MatvecArgs a{fmt, wq, sc, x, y, (int)dt, M, N, K};
    if (mode == QMV_MODE_SPLITK) {
        const size_t need = qmv::splitk_workspace_bytes(fmt, M, N, K);
        if (need > 0) {
            if (!ws || ws_bytes < need) return QMV_ERR_WORKSPACE;
            if (!aligned(ws, 256)) return QMV_ERR_ALIGNMENT;
        }
        return hip_status(qmv::launch_splitk_matvec(a, ws, static_cast<hipStream_t>(stream)));
    }
    if (mode != QMV_MODE_FIXED) return QMV_ERR_UNSUPPORTED;
    return hip_status(qmv::launch_fo_matvec(a, static_cast<hipStream_t>(stream)));
}

qmv_status qmv_int2(const uint32_t *wq, const uint16_t *scale, const uint16_t *x, void *y,
                    qmv_dtype y_dtype, int M, int N, int K, qmv_mode mode, void *workspace,
                    size_t ws_bytes, void *stream) {
    qmv_status s = check_matvec(wq, scale, x, y, y_dtype, M, N, K, 64, mode);
    if (s != QMV_OK) return s;
    if (mode == QMV_MODE_MFMA) return QMV_ERR_UNSUPPORTED;
    return run_matvec(0, wq, scale, x, y, y_dtype, M, N, K, mode, workspace, ws_bytes, stream);
}

qmv_status qmv_int4(const uint32_t *wq, const uint16_t *scales, const uint16_t *x, void *y,
                    qmv_dtype y_dtype, int M, int N, int K, qmv_mode mode, void *workspace,
                    size_t ws_bytes, void *stream) {
    qmv_status s = check_matvec(wq, scales, x, y, y_dtype, M, N, K, 32, mode);
    if (s != QMV_OK) return s;
    if (mode == QMV_MODE_MFMA) return QMV_ERR_UNSUPPORTED;
    return run_matvec(1, wq, scales, x, y, y_dtype, M, N, K, mode, workspace, ws_bytes, stream);
}

qmv_status qmm_mxfp4(const uint8_t *wq, const uint8_t *e8m0, const uint16_t *x, void *y,
                     qmv_dtype y_dtype, int M, int N, int K, qmv_mode mode, void *workspace,
                     size_t ws_bytes, void *stream) {
    qmv_status s = check_matvec(wq, e8m0, x, y, y_dtype, M, N, K, 32, mode);
    if (s != QMV_OK) return s;
    if (mode == QMV_MODE_MFMA) {
        if (M < 32) return QMV_ERR_UNSUPPORTED;
        qmv::MatvecArgs a{2, wq, e8m0, x, y, (int)y_dtype, M, N, K};
        return hip_status(qmv::launch_mxfp4_mfma(a, static_cast<hipStream_t>(stream)));
    }
    return run_matvec(2, wq, e8m0, x, y, y_dtype, M, N, K, mode, workspace, ws_bytes, stream);
}

qmv_status qmv_ternary(const uint8_t *wq, const uint16_t *scale, const uint16_t *x, void *y,
                       qmv_dtype y_dtype, int M, int N, int K, qmv_mode mode, void *workspace,
                       size_t ws_bytes, void *stream) {
    (void)workspace; (void)ws_bytes;
    if (!wq || !scale || !x || !y) return QMV_ERR_INVALID_ARG;
    if (!valid_shape(M, N, K, 8) || !valid_dtype(y_dtype) || !valid_mode(mode)) return QMV_ERR_INVALID_ARG;
    const uint64_t row_bytes = (uint64_t)(K + 79) / 80 * 16;
    if ((uint64_t)N * row_bytes >= (1ull << 32) - (1ull << 16)) return QMV_ERR_UNSUPPORTED;
    if ((uint64_t)M * (uint64_t)N * 4u >= (1ull << 32) - (1ull << 16)) return QMV_ERR_UNSUPPORTED;
    if (!aligned(wq, 16) || !aligned(x, 16) || !aligned(y, dtype_size(y_dtype))) return QMV_ERR_ALIGNMENT;
    if (mode != QMV_MODE_FIXED) return QMV_ERR_UNSUPPORTED;
    qmv::MatvecArgs a{3, wq, scale, x, y, (int)y_dtype, M, N, K};
    return hip_status(qmv::launch_fo_matvec(a, static_cast<hipStream_t>(stream)));
}

qmv_status qmv_int2_rmsnorm_gateup_gelu(const uint16_t *x, const uint16_t *residual,
                                        uint16_t *residual_out, const uint16_t *gamma, float eps,
                                        const uint32_t *wq_gate, const uint16_t *s_gate,
                                        const uint32_t *wq_up, const uint16_t *s_up,
                                        uint16_t *out, int M, int N, int K, qmv_mode mode,
                                        void *workspace, size_t ws_bytes, void *stream) {
    (void)workspace; (void)ws_bytes;
    if (!x || !residual || !gamma || !wq_gate || !s_gate || !wq_up || !s_up || !out)
        return QMV_ERR_INVALID_ARG;
    if (!valid_shape(M, N, K, 64) || !valid_mode(mode) || !(eps >= 0.0f)) return QMV_ERR_INVALID_ARG;
    if (!fits_32bit(N, K, 4)) return QMV_ERR_UNSUPPORTED;
    // out (fp16 [M][N]) is written with 32-bit byte offsets
    if ((uint64_t)M * (uint64_t)N * 2u >= (1ull << 32) - (1ull << 16)) return QMV_ERR_UNSUPPORTED;
    // the prologue reads gamma and writes residual_out as 16-byte vectors
    if (!aligned(x, 16) || !aligned(residual, 16) || !aligned(wq_gate, 16) || !aligned(wq_up, 16) ||
        !aligned(gamma, 16) || !aligned(out, 2) || (residual_out && !aligned(residual_out, 16)))
        return QMV_ERR_ALIGNMENT;
    if (mode != QMV_MODE_FIXED) return QMV_ERR_UNSUPPORTED;
    qmv::GateUpArgs a{x, residual, gamma, residual_out, eps, wq_gate, wq_up, s_gate, s_up, out, M, N, K};
    return hip_status(qmv::launch_fo_gateup(a, static_cast<hipStream_t>(stream)));
}

qmv_status qmv_int2_rmsnorm_gateup_gelu_mxfp4(const uint16_t *x, const uint16_t *residual,
                                              uint16_t *residual_out, const uint16_t *gamma, float eps,
                                              const uint32_t *wq_gate, const uint16_t *s_gate,
                                              const uint32_t *wq_up, const uint16_t *s_up, uint8_t *codes,
                                              uint8_t *e8m0, int M, int N, int K, qmv_mode mode,
                                              void *workspace, size_t ws_bytes, void *stream) {
    if (!x || !residual || !gamma || !wq_gate || !s_gate || !wq_up || !s_up || !codes || !e8m0)
        return QMV_ERR_INVALID_ARG;
    if (!valid_shape(M, N, K, 64) || N % 32 != 0 || !valid_mode(mode) || !(eps >= 0.0f))
        return QMV_ERR_INVALID_ARG;
    if (!fits_32bit(N, K, 4)) return QMV_ERR_UNSUPPORTED;
    if ((uint64_t)M * (uint64_t)N * 2u >= (1ull << 32) - (1ull << 16)) return QMV_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(residual, 16) || !aligned(wq_gate, 16) || !aligned(wq_up, 16) ||
        !aligned(gamma, 16) || (residual_out && !aligned(residual_out, 16)))
        return QMV_ERR_ALIGNMENT;
    if (mode != QMV_MODE_FIXED) return QMV_ERR_UNSUPPORTED;
    const size_t need = qmv::gateup_mxfp4_workspace_bytes(M, N);
    if (!workspace || ws_bytes < need) return QMV_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return QMV_ERR_ALIGNMENT;
    const size_t cnt_bytes = ((size_t)M * (N / 32) * 4 + 255) / 256 * 256;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    qmv::GateUpArgs a{x, residual, gamma, residual_out, eps, wq_gate, wq_up, s_gate, s_up,
                      reinterpret_cast<uint16_t *>(ws + cnt_bytes), M, N, K};
    a.qcodes = codes;
    a.qscale = e8m0;
    a.qcnt = reinterpret_cast<uint32_t *>(ws);
    return hip_status(qmv::launch_fo_gateup(a, static_cast<hipStream_t>(stream)));
}

qmv_status qmv_quant_mxfp4(const uint16_t *v, uint8_t *codes, uint8_t *e8m0, int M, int N, void *stream) {
    if (!v || !codes || !e8m0) return QMV_ERR_INVALID_ARG;
    if (M < 1 || N < 32 || N % 32 != 0) return QMV_ERR_INVALID_ARG;
    if ((uint64_t)M * (uint64_t)N >= (1ull << 31)) return QMV_ERR_UNSUPPORTED;
    if (!aligned(v, 2)) return QMV_ERR_ALIGNMENT;
    return hip_status(qmv::launch_quant_mxfp4(v, codes, e8m0, M, N, static_cast<hipStream_t>(stream)));
}

qmv_status qmv_int2_rmsnorm_qkv(const uint16_t *x, const uint16_t *residual, uint16_t *residual_out,
                                const uint16_t *gamma, float eps,
                                const uint32_t *wq_q, const uint16_t *s_q, int Nq,
                                const uint32_t *wq_k, const uint16_t *s_k, int Nk,
                                const uint32_t *wq_v, const uint16_t *s_v, int Nv,
                                void *y_q, void *y_k, void *y_v, qmv_dtype y_dtype, int M, int K,
                                qmv_mode mode, void *workspace, size_t ws_bytes, void *stream) {
    (void)workspace; (void)ws_bytes;
    if (!x || !residual || !gamma || !wq_q || !s_q || !wq_k || !s_k || !wq_v || !s_v || !y_q || !y_k || !y_v)
        return QMV_ERR_INVALID_ARG;
    const int ns[3] = {Nq, Nk, Nv};
    for (int z = 0; z < 3; ++z)
        if (!valid_shape(M, ns[z], K, 64)) return QMV_ERR_INVALID_ARG;
    if (!valid_dtype(y_dtype) || !valid_mode(mode) || !(eps >= 0.0f)) return QMV_ERR_INVALID_ARG;
    for (int z = 0; z < 3; ++z) {
        if (!fits_32bit(ns[z], K, 4)) return QMV_ERR_UNSUPPORTED;
        if ((uint64_t)M * (uint64_t)ns[z] * 4u >= (1ull << 32) - (1ull << 16)) return QMV_ERR_UNSUPPORTED;
    }
    if ((uint64_t)Nq + Nk + Nv > 0x7FFFFFFFull) return QMV_ERR_UNSUPPORTED;
    const size_t es = dtype_size(y_dtype);
    if (!aligned(x, 16) || !aligned(residual, 16) || !aligned(wq_q, 16) || !aligned(wq_k, 16) ||
        !aligned(wq_v, 16) || !aligned(gamma, 16) || !aligned(y_q, es) || !aligned(y_k, es) || !aligned(y_v, es) ||
        (residual_out && !aligned(residual_out, 16)))
        return QMV_ERR_ALIGNMENT;
    if (mode != QMV_MODE_FIXED) return QMV_ERR_UNSUPPORTED;
    qmv::QkvArgs a{x, residual, gamma, residual_out, eps, {wq_q, wq_k, wq_v}, {s_q, s_k, s_v},
                   {y_q, y_k, y_v}, {Nq, Nk, Nv}, (int)y_dtype, M, K};
    return hip_status(qmv::launch_fo_qkv(a, static_cast<hipStream_t>(stream)));
}

qmv_status qmm_mxfp4_gather(const uint8_t *wq, const uint8_t *e8m0, int E, const uint16_t *x,
                            const int32_t *idx, int topk, void *y, qmv_dtype y_dtype, int M, int N, int K,
                            qmv_mode mode, void *workspace, size_t ws_bytes, void *stream) {
    (void)workspace; (void)ws_bytes;
    if (!wq || !e8m0 || !x || !idx || !y) return QMV_ERR_INVALID_ARG;
    if (!valid_shape(M, N, K, 32) || E < 1 || topk < 1 || !valid_dtype(y_dtype) || !valid_mode(mode))
        return QMV_ERR_INVALID_ARG;
    // one expert is addressed with 32-bit offsets; planes go along grid.y
    if (!fits_32bit(N, K, 2) || (long)M * topk > kMaxGridY) return QMV_ERR_UNSUPPORTED;
    if ((uint64_t)M * (uint64_t)topk * (uint64_t)N * 4u >= (1ull << 32) - (1ull << 16))
        return QMV_ERR_UNSUPPORTED;
    if (!aligned(wq, 16) || !aligned(x, 16) || !aligned(idx, 4) || !aligned(y, dtype_size(y_dtype)))
        return QMV_ERR_ALIGNMENT;
    if (mode != QMV_MODE_FIXED) return QMV_ERR_UNSUPPORTED;
    qmv::GatherArgs a{wq, e8m0, x, idx, y, (int)y_dtype, E, topk, M, N, K};
    return hip_status(qmv::launch_fo_gather(a, static_cast<hipStream_t>(stream)));
}

// The calling thread's device's copy of `scratch` (taken and cleared on the
// first call on that device; the argmax kernel leaves it zeroed after every
// call).
static qmv_status static_scratch(hipStream_t st, void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= qmv::kMaxDevices) return QMV_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (p == nullptr) return QMV_ERR_HIP;
        // device globals start zeroed; clear once more with a fill kernel
        // (not a memset), on the caller's stream
        e = qmv::launch_fill_zero(p, kStaticScratchBytes, st);
        if (e != hipSuccess) return hip_status(e);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return QMV_OK;
}

qmv_status qmv_int2_argmax_static(const uint32_t *wq, const uint16_t *scale, const uint16_t *x,
                                  int32_t *idx, float *maxval, float *logits, int M, int N, int K,
                                  qmv_mode mode, void *stream) {
    if (!wq || !scale || !x || !idx) return QMV_ERR_INVALID_ARG;
    if (!valid_shape(M, N, K, 64) || !valid_mode(mode)) return QMV_ERR_INVALID_ARG;
    if (!fits_32bit(N, K, 4)) return QMV_ERR_UNSUPPORTED;
    if (!aligned(wq, 16) || !aligned(x, 16) || !aligned(idx, 4) || (maxval && !aligned(maxval, 4)) ||
        (logits && !aligned(logits, 4)))
        return QMV_ERR_ALIGNMENT;
    if (mode != QMV_MODE_FIXED) return QMV_ERR_UNSUPPORTED;
    const size_t need = qmv::argmax_workspace_bytes(M, N, K);
    if (need == 0 || need > kStaticScratchBytes) return QMV_ERR_WORKSPACE;  // beyond the static scratch
    void *ws = nullptr;
    const qmv_status s = static_scratch(static_cast<hipStream_t>(stream), &ws);
    if (s != QMV_OK) return s;
    qmv::ArgmaxArgs a{wq, scale, x, idx, maxval, logits, M, N, K, ws};
    return hip_status(qmv::launch_fo_argmax(a, static_cast<hipStream_t>(stream)));
}

qmv_status qmv_int2_argmax(const uint32_t *wq, const uint16_t *scale, const uint16_t *x,
                           int32_t *idx, float *maxval, float *logits, int M, int N, int K,
                           qmv_mode mode, void *workspace, size_t ws_bytes, void *stream) {
    if (!wq || !scale || !x || !idx) return QMV_ERR_INVALID_ARG;
    if (!valid_shape(M, N, K, 64) || !valid_mode(mode)) return QMV_ERR_INVALID_ARG;
    if (!fits_32bit(N, K, 4)) return QMV_ERR_UNSUPPORTED;
    if (!aligned(wq, 16) || !aligned(x, 16) || !aligned(idx, 4) || (maxval && !aligned(maxval, 4)) ||
        (logits && !aligned(logits, 4)))
        return QMV_ERR_ALIGNMENT;
    if (mode != QMV_MODE_FIXED) return QMV_ERR_UNSUPPORTED;
    const size_t need = qmv::argmax_workspace_bytes(M, N, K);
    if (!workspace || ws_bytes < need) return QMV_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return QMV_ERR_ALIGNMENT;
    qmv::ArgmaxArgs a{wq, scale, x, idx, maxval, logits, M, N, K, workspace};
    return hip_status(qmv::launch_fo_argmax(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
