/*
 * qmv.h -- C ABI of the MI355X (gfx950) quantized-weight matvec / skinny GEMM
 * library:  Y[M,N] = X[M,K] . dequant(Wq[N,K])^T,  M = 1..256.
 *
 * Sources for the operations (cited by page title and section):
 *  - "Gemma4 raw-Metal loop on A19 -- findings + the remaining (parked)
 *    levers", section "What moved the needle": the int2 weight format (16
 *    codes per 32-bit word, a byte holds 4 codes), exact products with codes
 *    in {-2,-1,0,1}, fp32 accumulation in code order (bit-exact), the fold
 *    of the residual-add RMSNorm into the next matvec, int2 gate/up and the
 *    int2 lm_head; section "The parked levers": single-dispatch argmax that
 *    keeps the first-max tie-break.
 *  - "raw-Metal loop playbook", prefill route table: for M = 8/16 keep every
 *    output's K-dot in the M = 1 accumulation order while the weights are
 *    shared across the M columns; wide-M GEMM tiles change the order
 *    (a tolerance class rather than bit-exact).
 *  - "Gemma 4 Optimization with Agentic Kernel Engineering", sections "A new
 *    chip, the same model" and "How much of the chip we use now": MXFP4
 *    weights and matrix-core GEMMs on MI355X.  Element/scale encodings follow
 *    the OCP Microscaling Formats v1.0 (E2M1 elements, E8M0 scale per 32).
 *  - "26 Iterations: Porting Cleanroom Kernels to Gemma 4", section "The
 *    Wins": dequantize inside the dot product (scalar inline-dequant), fused
 *    RMS+MUL.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE memory owned by the caller; the library
 *    keeps no pointer after the call returns and never allocates
 *    (qmv_int2_argmax_static uses a static device array of the library in
 *    place of a workspace).
 *  - Row-major layouts.  fp16 and bf16 values are passed as uint16_t bit
 *    patterns.  Packed weights:
 *      int2  : uint32_t [N][K/16]; code k = 16w+i is bits 2i+1..2i of word w,
 *              read as a two's-complement integer (0,1,2,3 -> 0,1,-2,-1);
 *              fp16 scale per row [N].
 *      int4  : uint32_t [N][K/8]; code k = 8w+i is bits 4i+3..4i of word w,
 *              value q-8; fp16 scale per 32-element group [N][K/32].
 *      MXFP4 : uint8_t [N][K/2]; element k = 2j in the low nibble of byte j,
 *              k = 2j+1 in the high nibble (E2M1); E8M0 scale byte per
 *              32-element block [N][K/32], value 2^(E-127).
 *  - x is [M][K] (fp16 for int2/int4, bf16 for MXFP4); y is [M][N].
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *    asynchronous: the status reports argument validation and launch errors
 *    only; kernel completion is observed through the stream.
 *  - Inputs must be finite; results for non-finite inputs are unspecified.
 *  - Each packed weight tensor, M*N*4 bytes for the output of the matvec
 *    entry points and M*N*2 bytes for the fused entry point's output must
 *    be smaller than 4 GiB (the kernels use 32-bit byte offsets); larger
 *    ones return QMV_ERR_UNSUPPORTED.
 *  - Calls that share a workspace must not overlap in time (same stream, or
 *    externally ordered).
 *
 * Modes:
 *  QMV_MODE_FIXED  (default) bit-exact fixed order, any M.  For each output
 *      (m, n): split the row's packed codes into 16-byte segments (int2: 64
 *      codes, int4 and MXFP4: 32 codes -- one scale group); sum the exact
 *      products value*x in fp32 in increasing k inside each segment starting
 *      from +0; scale the segment sum (int4: by fp32(group scale), one
 *      rounding; MXFP4: by 2^(E-127)); pad the segment values with +0 to a
 *      power of two P2 and reduce them by the halving tree
 *      v[p] = v[p] + v[p+s] for s = P2/2, ..., 1; int2 finally multiplies by
 *      the fp32 row scale.  Every fp32 operation is one IEEE
 *      round-to-nearest-even operation; denormals are kept.
 *  QMV_MODE_SPLITK opt-in tolerant mode: relative L2 error <= 2e-3 against
 *      the fixed order over the whole output.  The library splits K into S
 *      ranges of whole segments (S <= 16, chosen from the shape so that short
 *      N still fills the GPU; S = 1 when N alone does, and then the call runs
 *      the fixed-order kernel and needs no workspace).  Each range's sum (in
 *      the fixed order restricted to that range, before the int2 row scale)
 *      goes to the workspace as fp32 [S][M][N]; a second kernel adds the S
 *      partials in increasing range order and applies the int2 row scale, so
 *      results are deterministic.  Workspace: qmv_workspace_size(op, M, N, K,
 *      QMV_MODE_SPLITK) bytes, 256-byte aligned, no initialisation needed.
 *  QMV_MODE_MFMA   opt-in tolerant mode (relative L2 <= 2e-3) on the matrix
 *      cores; qmm_mxfp4 with M >= 32 only.
 *  A mode an entry point does not support returns QMV_ERR_UNSUPPORTED; there
 *  is no silent fallback to another mode.
 */
#ifndef QMV_H
#define QMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QMV_ABI_VERSION 1
#define QMV_MAX_M 256
#define QMV_MAX_K 16384

typedef enum qmv_status {
    QMV_OK = 0,
    QMV_ERR_INVALID_ARG = 1, /* null pointer, M/N/K out of range, bad enum */
    QMV_ERR_ALIGNMENT = 2,   /* a pointer is not aligned as documented     */
    QMV_ERR_WORKSPACE = 3,   /* workspace missing or smaller than needed   */
    QMV_ERR_UNSUPPORTED = 4, /* mode not available for this op / shape     */
    QMV_ERR_HIP = 5          /* a HIP launch failed; see qmv_last_hip_error */
} qmv_status;

typedef enum qmv_mode { QMV_MODE_FIXED = 0, QMV_MODE_SPLITK = 1, QMV_MODE_MFMA = 2 } qmv_mode;

typedef enum qmv_dtype { QMV_F32 = 0, QMV_F16 = 1, QMV_BF16 = 2 } qmv_dtype;

typedef enum qmv_op {
    QMV_OP_INT2 = 0,
    QMV_OP_INT4 = 1,
    QMV_OP_MXFP4 = 2,
    QMV_OP_INT2_GATEUP = 3,
    QMV_OP_INT2_ARGMAX = 4,
    QMV_OP_INT2_QKV = 5,
    QMV_OP_MXFP4_GATHER = 6,
    QMV_OP_TERNARY = 7,
    QMV_OP_INT2_GATEUP_MXFP4 = 8
} qmv_op;

/* Version of this ABI (QMV_ABI_VERSION). */
int qmv_abi_version(void);

/* Static description of a status code; never NULL. */
const char *qmv_status_string(qmv_status status);

/* Message of the last QMV_ERR_HIP returned on the calling thread ("" if none). */
const char *qmv_last_hip_error(void);

/* The frozen fixed order: bytes per segment (16), tree kind (1 = halving tree
 * padded with +0 to a power of two), inner step (1 = one product added per
 * binary32 rounding).  Any pointer may be NULL. */
void qmv_fo_spec(int *segment_bytes, int *tree_kind, int *inner_step);

/* Bytes of device workspace the call (op, M, N, K, mode) needs; 0 = none.
 * Returns 0 also for invalid shapes (the call itself then reports the error). */
size_t qmv_workspace_size(qmv_op op, int M, int N, int K, qmv_mode mode);

/* Zero a workspace on `stream` (a fill kernel, no allocation).  Required once
 * after allocating a workspace: kernels that need one keep a completion
 * counter there that they leave at zero after every call. */
qmv_status qmv_workspace_init(void *workspace, size_t ws_bytes, void *stream);

/* int2 matvec / skinny GEMM ("What moved the needle", int2 down / gate-up).
 *  wq     uint32 [N][K/16], 16-byte aligned
 *  scale  fp16 [N]   (per-row scale)
 *  x      fp16 [M][K], 16-byte aligned
 *  y      [M][N] of y_dtype (QMV_F32: fp32; QMV_F16 / QMV_BF16: one RNE
 *         rounding of the fp32 result), aligned to its element size
 *  1 <= M <= 256, N >= 1, K a multiple of 64, K <= 16384.
 *  Modes: FIXED (no workspace), SPLITK (workspace per qmv_workspace_size). */
qmv_status qmv_int2(const uint32_t *wq, const uint16_t *scale, const uint16_t *x, void *y,
                    qmv_dtype y_dtype, int M, int N, int K, qmv_mode mode, void *workspace,
                    size_t ws_bytes, void *stream);

/* int4 symmetric (value q-8) with fp16 scales per 32-element group: the
 * 4-bit quantized matvec ("26 Iterations: Porting Cleanroom Kernels to
 * Gemma 4", "The Dead Ends": the 4-bit Q4K kernel; "raw-Metal loop
 * playbook", next-target table: QAT-int4 weights), dequantized inside the
 * dot product ("26 Iterations", "The Wins": scalar inline-dequant), in the
 * fixed order above with one group scale per 16-byte segment.
 *  wq uint32 [N][K/8] (16-byte aligned); scales fp16 [N][K/32]; x fp16 [M][K]
 *  (16-byte aligned); y as for qmv_int2.  K a multiple of 32, K <= 16384.
 *  Modes: FIXED, SPLITK. */
qmv_status qmv_int4(const uint32_t *wq, const uint16_t *scales, const uint16_t *x, void *y,
                    qmv_dtype y_dtype, int M, int N, int K, qmv_mode mode, void *workspace,
                    size_t ws_bytes, void *stream);

/* MXFP4 skinny-to-wide GEMM ("Gemma 4 Optimization with Agentic Kernel
 * Engineering", MXFP4 matmuls on MI355X).
 *  wq uint8 [N][K/2] E2M1 pairs (16-byte aligned); e8m0 uint8 [N][K/32];
 *  x bf16 [M][K] (16-byte aligned); y as for qmv_int2.  K a multiple of 32,
 *  K <= 16384.  Modes: FIXED (any M), SPLITK, MFMA (M >= 32). */
qmv_status qmm_mxfp4(const uint8_t *wq, const uint8_t *e8m0, const uint16_t *x, void *y,
                     qmv_dtype y_dtype, int M, int N, int K, qmv_mode mode, void *workspace,
                     size_t ws_bytes, void *stream);

/* Ternary matvec ("raw-Metal loop playbook", next-target ranking table: the
 * ternary row, whose unpack is in the same ALU-bound family as the int2 byte
 * decode).  Weights in {-1, 0, +1}, five per byte in base 3:
 * byte = t0 + 3 t1 + 9 t2 + 27 t3 + 81 t4 with digits t_i in {0,1,2} and
 * weight t_i - 1; element k of a row is digit k mod 5 of byte k/5.  A row is
 * ceil(K/80) 16-byte segments (80 codes each); digits past K are ignored.
 * Only the 243 bytes 0..242 are codes (others give unspecified results).
 * Fixed order as for int2 with 80-code segments (the last one summing only
 * codes k < K); the fp16 row scale multiplies the reduced total.
 *  wq uint8 [N][ceil(K/80)*16] (16-byte aligned); scale fp16 [N];
 *  x fp16 [M][K] (16-byte aligned); y as for qmv_int2.  K a multiple of 8,
 *  K <= 16384.  Several activation rows are taken in chunks that share each
 *  weight read.  Mode: FIXED; no workspace. */
qmv_status qmv_ternary(const uint8_t *wq, const uint16_t *scale, const uint16_t *x, void *y,
                       qmv_dtype y_dtype, int M, int N, int K, qmv_mode mode, void *workspace,
                       size_t ws_bytes, void *stream);

/* Residual-add + RMSNorm prologue folded into dual int2 gate/up matvecs with
 * a GELU(gate)*up epilogue, one dispatch ("What moved the needle": the
 * residual-add RMSNorm fold into the next matvec and the int2 gate/up pair).
 * Per activation row m:
 *   h = fp16(x + residual)                       (one rounding)
 *   ss = sum of fp32(h_k)^2 in the fixed order (64-element segments, tree)
 *   inv = 1 / sqrt(ss / K + fp32(eps))           (correctly rounded / and sqrt)
 *   xn = fp16((fp32(h) * inv) * fp32(gamma))
 *   gate, up = fixed-order int2 matvecs of xn with (wq_gate, s_gate), (wq_up, s_up)
 *   out = fp16(GELU(gate) * up), GELU in tanh form evaluated as
 *         g / (1 + exp(-2u)), u = sqrt(2/pi) * (g + 0.044715 g^3), the
 *         exponent clamped to [-87, 87], exp by the library's own
 *         Cody-Waite + degree-7 polynomial.
 *  x, residual fp16 [M][K] (16-byte aligned); residual_out fp16 [M][K] or NULL
 *  (receives h; 16-byte aligned); gamma fp16 [K] (16-byte aligned);
 *  wq_* uint32 [N][K/16] (16-byte aligned); s_* fp16 [N]; out fp16 [M][N].
 *  K a multiple of 64, K <= 16384.  Mode: FIXED. */
qmv_status qmv_int2_rmsnorm_gateup_gelu(const uint16_t *x, const uint16_t *residual,
                                        uint16_t *residual_out, const uint16_t *gamma, float eps,
                                        const uint32_t *wq_gate, const uint16_t *s_gate,
                                        const uint32_t *wq_up, const uint16_t *s_up,
                                        uint16_t *out, int M, int N, int K, qmv_mode mode,
                                        void *workspace, size_t ws_bytes, void *stream);

/* Fused activation-and-quantize ("Gemma 4 Optimization with Agentic Kernel
 * Engineering", "What it found": a fused activation-and-quantize kernel on
 * MI355X): exactly qmv_int2_rmsnorm_gateup_gelu's fp16 output, quantised to
 * MXFP4 per block of 32 consecutive n of a row, in the same dispatch, for
 * the next MXFP4 GEMM.  Quantisation (OCP Microscaling Formats v1.0): the
 * block's shared exponent is floor(log2(max |v|)) - 2 (E8M0 byte = that +
 * 127; an all-zero block gets 0); each element v / 2^shared is rounded to
 * the nearest E2M1 value, ties to the even code, clamped to +-6, sign kept;
 * element 2j in the low nibble of byte j, 2j+1 in the high nibble (the
 * layout qmm_mxfp4 reads).
 *  Inputs (and their alignment) as for qmv_int2_rmsnorm_gateup_gelu; codes uint8 [M][N/2], e8m0
 *  uint8 [M][N/32]; N a multiple of 32.  Needs a workspace of
 *  qmv_workspace_size(QMV_OP_INT2_GATEUP_MXFP4, M, N, K, FIXED) bytes
 *  (256-byte aligned: per-block arrival counters and fp16 staging), zeroed
 *  once by qmv_workspace_init; every call leaves the counters at zero.
 *  Mode: FIXED. */
qmv_status qmv_int2_rmsnorm_gateup_gelu_mxfp4(const uint16_t *x, const uint16_t *residual,
                                              uint16_t *residual_out, const uint16_t *gamma, float eps,
                                              const uint32_t *wq_gate, const uint16_t *s_gate,
                                              const uint32_t *wq_up, const uint16_t *s_up, uint8_t *codes,
                                              uint8_t *e8m0, int M, int N, int K, qmv_mode mode,
                                              void *workspace, size_t ws_bytes, void *stream);

/* The same MXFP4 quantisation on its own: v fp16 [M][N] (2-byte aligned) ->
 * codes uint8 [M][N/2], e8m0 uint8 [M][N/32]; N a multiple of 32,
 * M*N < 2^31. */
qmv_status qmv_quant_mxfp4(const uint16_t *v, uint8_t *codes, uint8_t *e8m0, int M, int N, void *stream);

/* Shared-prologue q/k/v ("What moved the needle", dispatch-count fusion:
 * the residual-add RMSNorm folded into the next matvec's prologue, and
 * q/k/v issued as one dispatch).  Per activation row m, the prologue of
 * qmv_int2_rmsnorm_gateup_gelu (h = fp16(x + residual), inv, xn), then three
 * independent fixed-order int2 matvecs of xn:
 *   y_q = int2 matvec (wq_q, s_q), y_k = (wq_k, s_k), y_v = (wq_v, s_v),
 * each exactly as qmv_int2 would compute it from xn (bit-exact).
 *  x, residual fp16 [M][K] (16-byte aligned); residual_out fp16 [M][K] or
 *  NULL (receives h; 16-byte aligned); gamma fp16 [K] (16-byte aligned);
 *  wq_z uint32 [N_z][K/16] (16-byte aligned); s_z fp16 [N_z]; y_z [M][N_z] in y_dtype (fp32 default, or one
 *  RNE rounding to fp16 / bf16), each N_z >= 1 and M*N_z*4 bytes < 4 GiB.
 *  K a multiple of 64, K <= 16384.  Mode: FIXED; no workspace. */
qmv_status qmv_int2_rmsnorm_qkv(const uint16_t *x, const uint16_t *residual, uint16_t *residual_out,
                                const uint16_t *gamma, float eps,
                                const uint32_t *wq_q, const uint16_t *s_q, int Nq,
                                const uint32_t *wq_k, const uint16_t *s_k, int Nk,
                                const uint32_t *wq_v, const uint16_t *s_v, int Nv,
                                void *y_q, void *y_k, void *y_v, qmv_dtype y_dtype, int M, int K,
                                qmv_mode mode, void *workspace, size_t ws_bytes, void *stream);

/* int2 lm_head + argmax in one dispatch ("The parked levers": argmax stage 1
 * and 2 merged, first maximum wins).  Logits are the fixed-order int2 matvec;
 * idx[m] is the smallest n whose logit equals the row maximum (IEEE equality,
 * so -0 == +0); maxval[m] is that logit.
 *  idx int32 [M]; maxval fp32 [M] or NULL; logits fp32 [M][N] or NULL.
 *  Needs a workspace of qmv_workspace_size(QMV_OP_INT2_ARGMAX, ...) bytes,
 *  zeroed once by qmv_workspace_init.  Mode: FIXED. */
qmv_status qmv_int2_argmax(const uint32_t *wq, const uint16_t *scale, const uint16_t *x,
                           int32_t *idx, float *maxval, float *logits, int M, int N, int K,
                           qmv_mode mode, void *workspace, size_t ws_bytes, void *stream);

/* qmv_int2_argmax without a workspace, for callers that cannot allocate
 * (code under graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, results and modes as qmv_int2_argmax; the
 * counters and keys live in a static device array of the library (3 KB per
 * GPU, kept until the process ends), whose address is taken once per device
 * on the first call there (that call also clears it with a fill kernel on
 * `stream`; every call leaves it zeroed).  Calls on one GPU share that array:
 * calls that overlap in time on one GPU race and give wrong results (keep
 * them on one stream, or ordered).  No allocation, no allocating library
 * call.  QMV_ERR_WORKSPACE if M needs more than the array holds (it holds
 * every M <= QMV_MAX_M). */
qmv_status qmv_int2_argmax_static(const uint32_t *wq, const uint16_t *scale, const uint16_t *x,
                                  int32_t *idx, float *maxval, float *logits, int M, int N, int K,
                                  qmv_mode mode, void *stream);

/* Expert-gather MXFP4 matvec ("raw-Metal loop playbook", next-target ranking
 * table: the gpt-oss MoE row, a zero-materialisation expert-gather matvec).
 * The weights of E experts sit side by side; activation row m routes to the
 * topk experts idx[m][0 .. topk); each is read in place (no gathered copy):
 *   y[m][j][n] = qmm_mxfp4 fixed-order output (m, n) computed with expert
 *                e = idx[m][j]'s rows wq[e], e8m0[e] and activation row x[m]
 * (bit-exact with qmm_mxfp4 FIXED on the slices wq[e], e8m0[e], x[m]).
 *  wq uint8 [E][N][K/2] (16-byte aligned); e8m0 uint8 [E][N][K/32];
 *  x bf16 [M][K] (16-byte aligned); idx int32 [M][topk] on the device;
 *  y [M][topk][N] in y_dtype (fp32, or one RNE rounding to fp16 / bf16).
 *  E >= 1, topk >= 1, M*topk <= 65535, one expert's N*K/2 bytes and
 *  M*topk*N*4 bytes < 4 GiB; K a multiple of 32, K <= 16384.
 *  An id outside [0, E) cannot be seen at the call (idx stays on the device):
 *  that plane y[m][j][*] is set to NaN and no memory outside wq / e8m0 is
 *  read.  Duplicate ids in a row are allowed.  Mode: FIXED; no workspace. */
qmv_status qmm_mxfp4_gather(const uint8_t *wq, const uint8_t *e8m0, int E, const uint16_t *x,
                            const int32_t *idx, int topk, void *y, qmv_dtype y_dtype, int M, int N, int K,
                            qmv_mode mode, void *workspace, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QMV_H */
