"""CPU oracle for the quantized matvec / skinny GEMM (test infrastructure).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  The product path (the HIP library and its Python
binding) never does.  The arithmetic lives in ``oracle.c``; this module only
moves numpy arrays in and out of it.

Every function takes and returns numpy arrays on the host:
  fp16 / bf16 tensors are ``np.uint16`` bit patterns, packed weights are
  ``np.uint32`` (int2, int4) or ``np.uint8`` (MXFP4 elements, E8M0 scales).
"""
import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def load(path=None):
    """Load (building first if absent) the oracle library; returns the CDLL."""
    global _lib
    if path is not None:
        return _bind(C.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = _bind(C.CDLL(_LIB_PATH))
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _bind(lib):
    vp, i64, i32, f32 = C.c_void_p, C.c_int64, C.c_int, C.c_float
    sig = {
        "orc_f16_to_f32": ([C.c_uint16], f32),
        "orc_bf16_to_f32": ([C.c_uint16], f32),
        "orc_f32_to_f16": ([f32], C.c_uint16),
        "orc_f64_to_f16": ([C.c_double], C.c_uint16),
        "orc_f32_to_bf16": ([f32], C.c_uint16),
        "orc_f64_to_bf16": ([C.c_double], C.c_uint16),
        "orc_int2_value": ([C.c_uint], i32),
        "orc_int4_value": ([C.c_uint], i32),
        "orc_e2m1_value": ([C.c_uint], f32),
        "orc_e8m0_value": ([C.c_uint8], f32),
        "orc_int2_decode_byte_lut": ([C.c_uint8, vp], None),
        "orc_int2_decode_byte_arith": ([C.c_uint8, vp], None),
        "orc_int4_decode_byte_arith": ([C.c_uint8, vp], None),
        "orc_pack_int2": ([vp, i64, i64, vp], None),
        "orc_unpack_int2": ([vp, i64, i64, vp], None),
        "orc_pack_int4": ([vp, i64, i64, vp], None),
        "orc_unpack_int4": ([vp, i64, i64, vp], None),
        "orc_pack_e2m1": ([vp, i64, i64, vp], None),
        "orc_unpack_e2m1": ([vp, i64, i64, vp], None),
        "orc_qmv_int2": ([vp, vp, vp, vp, i64, i64, i64, i32], None),
        "orc_qmv_int4": ([vp, vp, vp, vp, i64, i64, i64, i32], None),
        "orc_qmm_mxfp4": ([vp, vp, vp, vp, i64, i64, i64, i32], None),
        "orc_exp": ([f32], f32),
        "orc_gelu": ([f32], f32),
        "orc_probe_mul_add": ([f32, f32, f32], f32),
        "orc_rmsnorm_prologue": ([vp, vp, vp, f32, i64, vp, vp], f32),
        "orc_int2_rmsnorm_gateup_gelu": ([vp, vp, vp, vp, f32, vp, vp, vp, vp, vp, vp, vp,
                                          i64, i64, i64, i32], None),
        "orc_int2_argmax": ([vp, vp, vp, vp, vp, vp, i64, i64, i64, i32], None),
        "orc_quant_mxfp4_block": ([vp, vp, vp], None),
        "orc_int2_rmsnorm_gateup_gelu_mxfp4": ([vp, vp, vp, vp, f32, vp, vp, vp, vp, vp, vp, i64, i64, i64,
                                                i32], None),
        "orc_ternary_value": ([C.c_uint, i32], i32),
        "orc_pack_ternary": ([vp, i64, i64, vp], None),
        "orc_qmv_ternary": ([vp, vp, vp, vp, i64, i64, i64, i32], None),
        "orc_qmm_mxfp4_gather": ([vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32], None),
        "orc_int2_rmsnorm_qkv": ([vp, vp, vp, vp, f32, vp, vp, i64, vp, vp, i64, vp, vp, i64,
                                  vp, vp, vp, i64, i64, i32], None),
        "orc_ref64_int2": ([vp, vp, vp, vp, vp, i64, i64, i64], None),
        "orc_ref64_int4": ([vp, vp, vp, vp, vp, i64, i64, i64], None),
        "orc_ref64_mxfp4": ([vp, vp, vp, vp, vp, i64, i64, i64], None),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def default_threads():
    """Worker threads for the row-parallel oracle: OMP_NUM_THREADS if set,
    else the CPU count, never more than 16."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    n = int(env) if env.isdigit() and int(env) > 0 else (os.cpu_count() or 1)
    return max(1, min(n, 16))


# ---------------------------------------------------------------- matvecs --

def qmv_int2(wq, scale, x, threads=None, lib=None):
    """FO int2 matvec. wq uint32 [N][K/16], scale fp16 bits [N], x fp16 bits [M][K] -> fp32 [M][N]."""
    lib = lib or load()
    wq, scale, x = _c(wq, np.uint32), _c(scale, np.uint16), _c(x, np.uint16)
    N, M, K = wq.shape[0], x.shape[0], x.shape[1]
    assert wq.shape[1] * 16 == K and scale.shape == (N,) and K % 64 == 0
    y = np.empty((M, N), np.float32)
    lib.orc_qmv_int2(_p(wq), _p(scale), _p(x), _p(y), M, N, K, threads or default_threads())
    return y


def qmv_int4(wq, scales, x, threads=None, lib=None):
    """FO int4 matvec. wq uint32 [N][K/8], scales fp16 bits [N][K/32], x fp16 bits [M][K]."""
    lib = lib or load()
    wq, scales, x = _c(wq, np.uint32), _c(scales, np.uint16), _c(x, np.uint16)
    N, M, K = wq.shape[0], x.shape[0], x.shape[1]
    assert wq.shape[1] * 8 == K and scales.shape == (N, K // 32) and K % 32 == 0
    y = np.empty((M, N), np.float32)
    lib.orc_qmv_int4(_p(wq), _p(scales), _p(x), _p(y), M, N, K, threads or default_threads())
    return y


def qmm_mxfp4(wq, e8m0, x, threads=None, lib=None):
    """FO MXFP4 GEMM. wq uint8 [N][K/2], e8m0 uint8 [N][K/32], x bf16 bits [M][K]."""
    lib = lib or load()
    wq, e8m0, x = _c(wq, np.uint8), _c(e8m0, np.uint8), _c(x, np.uint16)
    N, M, K = wq.shape[0], x.shape[0], x.shape[1]
    assert wq.shape[1] * 2 == K and e8m0.shape == (N, K // 32) and K % 32 == 0
    y = np.empty((M, N), np.float32)
    lib.orc_qmm_mxfp4(_p(wq), _p(e8m0), _p(x), _p(y), M, N, K, threads or default_threads())
    return y


def quant_mxfp4(v, lib=None):
    """fp16 bits [R][32*B] -> (E2M1 codes uint8 [R][16*B], E8M0 uint8 [R][B]), one
    block per 32 consecutive values of a row."""
    lib = lib or load()
    v = _c(v, np.uint16)
    R, N = v.shape
    assert N % 32 == 0
    codes = np.empty((R, N // 2), np.uint8)
    e = np.empty((R, N // 32), np.uint8)
    for r in range(R):
        for b in range(N // 32):
            blk = np.ascontiguousarray(v[r, 32 * b:32 * b + 32])
            cb = np.empty(16, np.uint8)
            eb = np.empty(1, np.uint8)
            lib.orc_quant_mxfp4_block(_p(blk), _p(cb), _p(eb))
            codes[r, 16 * b:16 * b + 16] = cb
            e[r, b] = eb[0]
    return codes, e


def int2_rmsnorm_gateup_gelu_mxfp4(x, residual, gamma, eps, wq_gate, s_gate, wq_up, s_up,
                                   threads=None, lib=None):
    """Fused gate/up with its fp16 output quantised to MXFP4 per 32-value block.
    Returns (codes uint8 [M][N/2], e8m0 uint8 [M][N/32], residual_out fp16 bits [M][K])."""
    lib = lib or load()
    x, residual, gamma = _c(x, np.uint16), _c(residual, np.uint16), _c(gamma, np.uint16)
    wq_gate, wq_up = _c(wq_gate, np.uint32), _c(wq_up, np.uint32)
    s_gate, s_up = _c(s_gate, np.uint16), _c(s_up, np.uint16)
    (M, K), N = x.shape, wq_gate.shape[0]
    assert N % 32 == 0
    codes = np.empty((M, N // 2), np.uint8)
    e = np.empty((M, N // 32), np.uint8)
    res = np.empty((M, K), np.uint16)
    lib.orc_int2_rmsnorm_gateup_gelu_mxfp4(_p(x), _p(residual), _p(res), _p(gamma), float(eps), _p(wq_gate),
                                           _p(s_gate), _p(wq_up), _p(s_up), _p(codes), _p(e), M, N, K,
                                           threads or default_threads())
    return codes, e, res


def ternary_row_bytes(K):
    """Bytes per packed ternary row: ceil(K/80) segments of 16 bytes (80 codes)."""
    return (K + 79) // 80 * 16


def pack_ternary(v, lib=None):
    """int8 values [N][K] in {-1,0,1} -> packed uint8 [N][ternary_row_bytes(K)]."""
    lib = lib or load()
    v = _c(v, np.int8)
    N, K = v.shape
    out = np.empty((N, ternary_row_bytes(K)), np.uint8)
    lib.orc_pack_ternary(_p(v), N, K, _p(out))
    return out


def qmv_ternary(wq, scale, x, threads=None, lib=None):
    """FO ternary matvec: wq uint8 [N][ternary_row_bytes(K)], scale fp16 bits [N],
    x fp16 bits [M][K] -> y fp32 [M][N]."""
    lib = lib or load()
    wq, scale, x = _c(wq, np.uint8), _c(scale, np.uint16), _c(x, np.uint16)
    N, (M, K) = wq.shape[0], x.shape
    assert wq.shape[1] == ternary_row_bytes(K) and scale.shape == (N,)
    y = np.empty((M, N), np.float32)
    lib.orc_qmv_ternary(_p(wq), _p(scale), _p(x), _p(y), M, N, K, threads or default_threads())
    return y


def qmm_mxfp4_gather(wq, e8m0, x, idx, threads=None, lib=None):
    """Expert-gather FO MXFP4 matvec. wq uint8 [E][N][K/2], e8m0 uint8 [E][N][K/32],
    x bf16 bits [M][K], idx int32 [M][topk] in [0, E).  Returns y fp32 [M][topk][N]."""
    lib = lib or load()
    wq, e8m0, x, idx = _c(wq, np.uint8), _c(e8m0, np.uint8), _c(x, np.uint16), _c(idx, np.int32)
    E, N, M, K, topk = wq.shape[0], wq.shape[1], x.shape[0], x.shape[1], idx.shape[1]
    assert wq.shape[2] * 2 == K and e8m0.shape == (E, N, K // 32) and idx.shape[0] == M
    assert np.all((idx >= 0) & (idx < E))
    y = np.empty((M, topk, N), np.float32)
    lib.orc_qmm_mxfp4_gather(_p(wq), _p(e8m0), _p(x), _p(idx), _p(y), E, topk, M, N, K,
                             threads or default_threads())
    return y


def int2_rmsnorm_gateup_gelu(x, residual, gamma, eps, wq_gate, s_gate, wq_up, s_up,
                             threads=None, lib=None):
    """Fused prologue + dual int2 + GELU*up. Returns (out fp16 bits [M][N],
    residual_out fp16 bits [M][K], gate fp32 [M][N], up fp32 [M][N])."""
    lib = lib or load()
    x, residual, gamma = _c(x, np.uint16), _c(residual, np.uint16), _c(gamma, np.uint16)
    wq_gate, wq_up = _c(wq_gate, np.uint32), _c(wq_up, np.uint32)
    s_gate, s_up = _c(s_gate, np.uint16), _c(s_up, np.uint16)
    M, K = x.shape
    N = wq_gate.shape[0]
    out = np.empty((M, N), np.uint16)
    res_out = np.empty((M, K), np.uint16)
    g = np.empty((M, N), np.float32)
    u = np.empty((M, N), np.float32)
    lib.orc_int2_rmsnorm_gateup_gelu(_p(x), _p(residual), _p(res_out), _p(gamma), float(eps),
                                     _p(wq_gate), _p(s_gate), _p(wq_up), _p(s_up),
                                     _p(out), _p(g), _p(u), M, N, K, threads or default_threads())
    return out, res_out, g, u


def int2_rmsnorm_qkv(x, residual, gamma, eps, wq_q, s_q, wq_k, s_k, wq_v, s_v, threads=None, lib=None):
    """Shared-prologue q/k/v: residual add + RMSNorm on each row, then three int2
    fixed-order matvecs on the normalised row.  Returns (yq, yk, yv fp32 [M][N_z],
    residual_out fp16 bits [M][K])."""
    lib = lib or load()
    x, residual, gamma = _c(x, np.uint16), _c(residual, np.uint16), _c(gamma, np.uint16)
    ws = [_c(w, np.uint32) for w in (wq_q, wq_k, wq_v)]
    ss = [_c(s, np.uint16) for s in (s_q, s_k, s_v)]
    M, K = x.shape
    ys = [np.empty((M, w.shape[0]), np.float32) for w in ws]
    res_out = np.empty((M, K), np.uint16)
    lib.orc_int2_rmsnorm_qkv(_p(x), _p(residual), _p(res_out), _p(gamma), float(eps),
                             _p(ws[0]), _p(ss[0]), ws[0].shape[0], _p(ws[1]), _p(ss[1]), ws[1].shape[0],
                             _p(ws[2]), _p(ss[2]), ws[2].shape[0], _p(ys[0]), _p(ys[1]), _p(ys[2]),
                             M, K, threads or default_threads())
    return ys[0], ys[1], ys[2], res_out


def int2_argmax(wq, scale, x, threads=None, lib=None):
    """int2 FO logits + first-max argmax. Returns (idx int32 [M], maxval fp32 [M], logits fp32 [M][N])."""
    lib = lib or load()
    wq, scale, x = _c(wq, np.uint32), _c(scale, np.uint16), _c(x, np.uint16)
    N, M, K = wq.shape[0], x.shape[0], x.shape[1]
    idx = np.empty((M,), np.int32)
    mv = np.empty((M,), np.float32)
    logits = np.empty((M, N), np.float32)
    lib.orc_int2_argmax(_p(wq), _p(scale), _p(x), _p(idx), _p(mv), _p(logits), M, N, K,
                        threads or default_threads())
    return idx, mv, logits


def rmsnorm_prologue(x, residual, gamma, eps, lib=None):
    """One activation row: returns (h fp16 bits [K], xn fp16 bits [K], inv fp32)."""
    lib = lib or load()
    x, residual, gamma = _c(x, np.uint16), _c(residual, np.uint16), _c(gamma, np.uint16)
    K = x.shape[0]
    h = np.empty((K,), np.uint16)
    xn = np.empty((K,), np.uint16)
    inv = lib.orc_rmsnorm_prologue(_p(x), _p(residual), _p(gamma), float(eps), K, _p(h), _p(xn))
    return h, xn, np.float32(inv)


# --------------------------------------------------------- fp64 references --

def _ref64(fn, wq, sc, x, N, M, K, lib):
    y = np.empty((M, N), np.float64)
    a = np.empty((M, N), np.float64)
    fn(_p(wq), _p(sc), _p(x), _p(y), _p(a), M, N, K)
    return y, a


def ref64_int2(wq, scale, x, lib=None):
    """Dequantize-then-dot in double. Returns (y, sum |scaled products|)."""
    lib = lib or load()
    wq, scale, x = _c(wq, np.uint32), _c(scale, np.uint16), _c(x, np.uint16)
    return _ref64(lib.orc_ref64_int2, wq, scale, x, wq.shape[0], x.shape[0], x.shape[1], lib)


def ref64_int4(wq, scales, x, lib=None):
    lib = lib or load()
    wq, scales, x = _c(wq, np.uint32), _c(scales, np.uint16), _c(x, np.uint16)
    return _ref64(lib.orc_ref64_int4, wq, scales, x, wq.shape[0], x.shape[0], x.shape[1], lib)


def ref64_mxfp4(wq, e8m0, x, lib=None):
    lib = lib or load()
    wq, e8m0, x = _c(wq, np.uint8), _c(e8m0, np.uint8), _c(x, np.uint16)
    return _ref64(lib.orc_ref64_mxfp4, wq, e8m0, x, wq.shape[0], x.shape[0], x.shape[1], lib)


# ------------------------------------------------------------- packing ----

def pack_int2(vals, lib=None):
    """vals int8 [N][K] in {-2,-1,0,1} -> uint32 [N][K/16]."""
    lib = lib or load()
    vals = _c(vals, np.int8)
    N, K = vals.shape
    out = np.empty((N, K // 16), np.uint32)
    lib.orc_pack_int2(_p(vals), N, K, _p(out))
    return out


def unpack_int2(wq, K, lib=None):
    lib = lib or load()
    wq = _c(wq, np.uint32)
    out = np.empty((wq.shape[0], K), np.int8)
    lib.orc_unpack_int2(_p(wq), wq.shape[0], K, _p(out))
    return out


def pack_int4(q, lib=None):
    """q uint8 [N][K] in 0..15 -> uint32 [N][K/8]."""
    lib = lib or load()
    q = _c(q, np.uint8)
    N, K = q.shape
    out = np.empty((N, K // 8), np.uint32)
    lib.orc_pack_int4(_p(q), N, K, _p(out))
    return out


def unpack_int4(wq, K, lib=None):
    lib = lib or load()
    wq = _c(wq, np.uint32)
    out = np.empty((wq.shape[0], K), np.uint8)
    lib.orc_unpack_int4(_p(wq), wq.shape[0], K, _p(out))
    return out


def pack_e2m1(nib, lib=None):
    """nib uint8 [N][K] E2M1 codes 0..15 -> uint8 [N][K/2]."""
    lib = lib or load()
    nib = _c(nib, np.uint8)
    N, K = nib.shape
    out = np.empty((N, K // 2), np.uint8)
    lib.orc_pack_e2m1(_p(nib), N, K, _p(out))
    return out


def unpack_e2m1(wq, K, lib=None):
    lib = lib or load()
    wq = _c(wq, np.uint8)
    out = np.empty((wq.shape[0], K), np.uint8)
    lib.orc_unpack_e2m1(_p(wq), wq.shape[0], K, _p(out))
    return out


def int2_decode_byte(b, how="arith", lib=None):
    lib = lib or load()
    out = (C.c_int8 * 4)()
    fn = lib.orc_int2_decode_byte_lut if how == "lut" else lib.orc_int2_decode_byte_arith
    fn(b, C.cast(out, C.c_void_p))
    return list(out)


def int4_decode_byte(b, lib=None):
    lib = lib or load()
    out = (C.c_int8 * 2)()
    lib.orc_int4_decode_byte_arith(b, C.cast(out, C.c_void_p))
    return list(out)


def f16_to_f32(h, lib=None):
    lib = lib or load()
    return np.array([lib.orc_f16_to_f32(int(v)) for v in np.ravel(h)], np.float32).reshape(np.shape(h))


def f32_to_f16(f, lib=None):
    lib = lib or load()
    return np.array([lib.orc_f32_to_f16(float(v)) for v in np.ravel(f)], np.uint16).reshape(np.shape(f))


def f32_to_bf16(f, lib=None):
    lib = lib or load()
    return np.array([lib.orc_f32_to_bf16(float(v)) for v in np.ravel(f)], np.uint16).reshape(np.shape(f))
