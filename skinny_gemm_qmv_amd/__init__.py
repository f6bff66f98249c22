"""Python binding of libqmv.so, the gfx950 quantized matvec / skinny GEMM library.

Argument marshalling only: every function checks the torch tensors it is
given (device, dtype, shape, contiguity), allocates outputs the caller did
not pass, and calls the C entry point of the same name on torch's current
HIP stream.  No arithmetic of the method happens in Python.  If the built
library is missing, importing this package raises: there is no fallback.

Tensor conventions (all on the GPU, contiguous, row-major):
  int2 weights  torch.int32 [N, K/16]  (bit patterns of uint32 words)
  int4 weights  torch.int32 [N, K/8]
  MXFP4 weights torch.uint8 [N, K/2];  E8M0 scales torch.uint8 [N, K/32]
  MXFP4 experts torch.uint8 [E, N, K/2] and [E, N, K/32]; expert ids torch.int32
  ternary       torch.uint8 [N, ternary_row_bytes(K)] (five base-3 digits per byte)
  fp16 tensors  torch.float16;  bf16 tensors torch.bfloat16
"""
import ctypes as C
import os

import torch

__all__ = [
    "qmv_int2", "qmv_int4", "qmm_mxfp4", "qmv_int2_rmsnorm_gateup_gelu", "qmv_int2_rmsnorm_qkv",
    "qmv_int2_argmax", "qmv_int2_argmax_static", "qmm_mxfp4_gather", "qmv_ternary", "ternary_row_bytes",
    "qmv_int2_rmsnorm_gateup_gelu_mxfp4", "qmv_quant_mxfp4", "workspace_size", "workspace_init", "fo_spec", "abi_version", "QmvError", "LIB_PATH",
    "MODES", "OPS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqmv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950) first")

_lib = C.CDLL(LIB_PATH)

MODES = {"fixed": 0, "splitk": 1, "mfma": 2}
OPS = {"int2": 0, "int4": 1, "mxfp4": 2, "int2_gateup": 3, "int2_argmax": 4, "int2_qkv": 5, "mxfp4_gather": 6, "ternary": 7, "int2_gateup_mxfp4": 8}
_DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}

_vp, _i, _sz, _f = C.c_void_p, C.c_int, C.c_size_t, C.c_float
_SIGS = {
    "qmv_abi_version": ([], _i),
    "qmv_status_string": ([_i], C.c_char_p),
    "qmv_last_hip_error": ([], C.c_char_p),
    "qmv_fo_spec": ([_vp, _vp, _vp], None),
    "qmv_workspace_size": ([_i, _i, _i, _i, _i], _sz),
    "qmv_workspace_init": ([_vp, _sz, _vp], _i),
    "qmv_int2": ([_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _sz, _vp], _i),
    "qmv_int4": ([_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _sz, _vp], _i),
    "qmm_mxfp4": ([_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _sz, _vp], _i),
    "qmv_int2_rmsnorm_gateup_gelu": ([_vp, _vp, _vp, _vp, _f, _vp, _vp, _vp, _vp, _vp,
                                      _i, _i, _i, _i, _vp, _sz, _vp], _i),
    "qmv_int2_argmax": ([_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _sz, _vp], _i),
    "qmv_int2_argmax_static": ([_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp], _i),
    "qmv_int2_rmsnorm_qkv": ([_vp, _vp, _vp, _vp, _f, _vp, _vp, _i, _vp, _vp, _i, _vp, _vp, _i,
                              _vp, _vp, _vp, _i, _i, _i, _i, _vp, _sz, _vp], _i),
    "qmv_int2_rmsnorm_gateup_gelu_mxfp4": ([_vp, _vp, _vp, _vp, _f, _vp, _vp, _vp, _vp, _vp, _vp,
                                            _i, _i, _i, _i, _vp, _sz, _vp], _i),
    "qmv_quant_mxfp4": ([_vp, _vp, _vp, _i, _i, _vp], _i),
    "qmv_ternary": ([_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _sz, _vp], _i),
    "qmm_mxfp4_gather": ([_vp, _vp, _i, _vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _vp, _sz, _vp], _i),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


class QmvError(RuntimeError):
    def __init__(self, status, where):
        msg = _lib.qmv_status_string(status).decode()
        if status == 5:
            msg += ": " + _lib.qmv_last_hip_error().decode()
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


def _check(status, where):
    if status != 0:
        raise QmvError(status, where)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _req(t, name, dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _mode(mode):
    if mode not in MODES:
        raise ValueError(f"mode must be one of {list(MODES)}")
    return MODES[mode]


def abi_version():
    return _lib.qmv_abi_version()


def fo_spec():
    """(segment_bytes, tree_kind, inner_step) of the frozen fixed order."""
    a, b, c = C.c_int(), C.c_int(), C.c_int()
    _lib.qmv_fo_spec(C.byref(a), C.byref(b), C.byref(c))
    return a.value, b.value, c.value


def workspace_size(op, M, N, K, mode="fixed"):
    return int(_lib.qmv_workspace_size(OPS[op], M, N, K, _mode(mode)))


def workspace_init(ws, stream=None):
    _check(_lib.qmv_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "qmv_workspace_init")


def _workspace(op, M, N, K, mode, workspace, stream):
    """The caller's workspace, or a temporary one allocated and zeroed on the
    stream the kernel runs on: the zero-fill is then ordered before the
    kernel, and the caching allocator hands the block to later work on that
    stream only, which runs after the kernel."""
    need = workspace_size(op, M, N, K, mode)
    if workspace is None:
        if need == 0:
            return None, 0
        s = torch.cuda.current_stream() if stream is None else stream
        with torch.cuda.stream(s):
            workspace = torch.empty(need, dtype=torch.uint8, device="cuda")
            workspace_init(workspace, stream=s)
    return workspace, workspace.numel() * workspace.element_size()


def _out(y, M, N, dtype, device):
    if y is None:
        return torch.empty((M, N), dtype=dtype, device=device)
    return _req(y, "y", dtype, (M, N))


def _matvec(fn, name, wq, sc, x, y, y_dtype, mode, workspace, stream, op):
    M, K = x.shape
    N = wq.shape[0]
    y = _out(y, M, N, y_dtype, x.device)
    ws, wsb = _workspace(op, M, N, K, mode, workspace, stream)
    _check(fn(_ptr(wq), _ptr(sc), _ptr(x), _ptr(y), _DTYPES[y_dtype], M, N, K, _mode(mode),
              _ptr(ws), wsb, _stream(stream)), name)
    return y


def qmv_int2(wq, scale, x, y=None, y_dtype=torch.float32, mode="fixed", workspace=None, stream=None):
    """y[M,N] = x[M,K] . dequant_int2(wq)^T (see qmv.h).  wq int32 [N,K/16], scale fp16 [N]."""
    M, K = x.shape
    N = wq.shape[0]
    _req(wq, "wq", torch.int32, (N, K // 16))
    _req(scale, "scale", torch.float16, (N,))
    _req(x, "x", torch.float16, (M, K))
    return _matvec(_lib.qmv_int2, "qmv_int2", wq, scale, x, y, y_dtype, mode, workspace, stream, "int2")


def qmv_int4(wq, scales, x, y=None, y_dtype=torch.float32, mode="fixed", workspace=None, stream=None):
    """int4 (q-8) with group-32 fp16 scales.  wq int32 [N,K/8], scales fp16 [N,K/32]."""
    M, K = x.shape
    N = wq.shape[0]
    _req(wq, "wq", torch.int32, (N, K // 8))
    _req(scales, "scales", torch.float16, (N, K // 32))
    _req(x, "x", torch.float16, (M, K))
    return _matvec(_lib.qmv_int4, "qmv_int4", wq, scales, x, y, y_dtype, mode, workspace, stream, "int4")


def qmm_mxfp4(wq, e8m0, x, y=None, y_dtype=torch.float32, mode="fixed", workspace=None, stream=None):
    """MXFP4 GEMM.  wq uint8 [N,K/2], e8m0 uint8 [N,K/32], x bf16 [M,K]."""
    M, K = x.shape
    N = wq.shape[0]
    _req(wq, "wq", torch.uint8, (N, K // 2))
    _req(e8m0, "e8m0", torch.uint8, (N, K // 32))
    _req(x, "x", torch.bfloat16, (M, K))
    return _matvec(_lib.qmm_mxfp4, "qmm_mxfp4", wq, e8m0, x, y, y_dtype, mode, workspace, stream, "mxfp4")


def qmv_int2_rmsnorm_gateup_gelu(x, residual, gamma, eps, wq_gate, s_gate, wq_up, s_up, out=None,
                                 residual_out=None, mode="fixed", workspace=None, stream=None):
    """out = fp16(GELU(gate) * up) with the residual-add RMSNorm prologue (see qmv.h)."""
    M, K = x.shape
    N = wq_gate.shape[0]
    _req(x, "x", torch.float16, (M, K))
    _req(residual, "residual", torch.float16, (M, K))
    _req(gamma, "gamma", torch.float16, (K,))
    _req(wq_gate, "wq_gate", torch.int32, (N, K // 16))
    _req(wq_up, "wq_up", torch.int32, (N, K // 16))
    _req(s_gate, "s_gate", torch.float16, (N,))
    _req(s_up, "s_up", torch.float16, (N,))
    out = _out(out, M, N, torch.float16, x.device)
    if residual_out is not None:
        _req(residual_out, "residual_out", torch.float16, (M, K))
    ws, wsb = _workspace("int2_gateup", M, N, K, mode, workspace, stream)
    _check(_lib.qmv_int2_rmsnorm_gateup_gelu(
        _ptr(x), _ptr(residual), _ptr(residual_out), _ptr(gamma), float(eps), _ptr(wq_gate),
        _ptr(s_gate), _ptr(wq_up), _ptr(s_up), _ptr(out), M, N, K, _mode(mode), _ptr(ws), wsb,
        _stream(stream)), "qmv_int2_rmsnorm_gateup_gelu")
    return out


def qmv_int2_rmsnorm_gateup_gelu_mxfp4(x, residual, gamma, eps, wq_gate, s_gate, wq_up, s_up, codes=None,
                                       e8m0=None, residual_out=None, mode="fixed", workspace=None,
                                       stream=None):
    """The fused gate/up output quantised to MXFP4 in the same dispatch (see qmv.h).
    Returns (codes uint8 [M, N/2], e8m0 uint8 [M, N/32]).  A workspace (uint8,
    workspace_size("int2_gateup_mxfp4", ...) bytes, zeroed once with workspace_init)
    may be passed to avoid a per-call allocation."""
    M, K = x.shape
    N = wq_gate.shape[0]
    _req(x, "x", torch.float16, (M, K))
    _req(residual, "residual", torch.float16, (M, K))
    _req(gamma, "gamma", torch.float16, (K,))
    _req(wq_gate, "wq_gate", torch.int32, (N, K // 16))
    _req(wq_up, "wq_up", torch.int32, (N, K // 16))
    _req(s_gate, "s_gate", torch.float16, (N,))
    _req(s_up, "s_up", torch.float16, (N,))
    codes = torch.empty((M, N // 2), dtype=torch.uint8, device=x.device) if codes is None else \
        _req(codes, "codes", torch.uint8, (M, N // 2))
    e8m0 = torch.empty((M, N // 32), dtype=torch.uint8, device=x.device) if e8m0 is None else \
        _req(e8m0, "e8m0", torch.uint8, (M, N // 32))
    if residual_out is not None:
        _req(residual_out, "residual_out", torch.float16, (M, K))
    ws, wsb = _workspace("int2_gateup_mxfp4", M, N, K, mode, workspace, stream)
    _check(_lib.qmv_int2_rmsnorm_gateup_gelu_mxfp4(
        _ptr(x), _ptr(residual), _ptr(residual_out), _ptr(gamma), float(eps), _ptr(wq_gate),
        _ptr(s_gate), _ptr(wq_up), _ptr(s_up), _ptr(codes), _ptr(e8m0), M, N, K, _mode(mode), _ptr(ws), wsb,
        _stream(stream)), "qmv_int2_rmsnorm_gateup_gelu_mxfp4")
    return codes, e8m0


def qmv_quant_mxfp4(v, codes=None, e8m0=None, stream=None):
    """fp16 [M, N] -> MXFP4 (codes uint8 [M, N/2], e8m0 uint8 [M, N/32]) per 32-value block."""
    M, N = v.shape
    _req(v, "v", torch.float16, (M, N))
    codes = torch.empty((M, N // 2), dtype=torch.uint8, device=v.device) if codes is None else \
        _req(codes, "codes", torch.uint8, (M, N // 2))
    e8m0 = torch.empty((M, N // 32), dtype=torch.uint8, device=v.device) if e8m0 is None else \
        _req(e8m0, "e8m0", torch.uint8, (M, N // 32))
    _check(_lib.qmv_quant_mxfp4(_ptr(v), _ptr(codes), _ptr(e8m0), M, N, _stream(stream)), "qmv_quant_mxfp4")
    return codes, e8m0


def qmv_int2_rmsnorm_qkv(x, residual, gamma, eps, wq_q, s_q, wq_k, s_k, wq_v, s_v, y_q=None, y_k=None,
                         y_v=None, y_dtype=torch.float32, residual_out=None, mode="fixed", stream=None):
    """(y_q, y_k, y_v): three int2 matvecs of the residual-add RMSNorm of x (see qmv.h)."""
    M, K = x.shape
    _req(x, "x", torch.float16, (M, K))
    _req(residual, "residual", torch.float16, (M, K))
    _req(gamma, "gamma", torch.float16, (K,))
    ys = []
    for name, w, s, y in (("q", wq_q, s_q, y_q), ("k", wq_k, s_k, y_k), ("v", wq_v, s_v, y_v)):
        N = w.shape[0]
        _req(w, "wq_" + name, torch.int32, (N, K // 16))
        _req(s, "s_" + name, torch.float16, (N,))
        ys.append(_out(y, M, N, y_dtype, x.device))
    if residual_out is not None:
        _req(residual_out, "residual_out", torch.float16, (M, K))
    _check(_lib.qmv_int2_rmsnorm_qkv(
        _ptr(x), _ptr(residual), _ptr(residual_out), _ptr(gamma), float(eps),
        _ptr(wq_q), _ptr(s_q), wq_q.shape[0], _ptr(wq_k), _ptr(s_k), wq_k.shape[0],
        _ptr(wq_v), _ptr(s_v), wq_v.shape[0], _ptr(ys[0]), _ptr(ys[1]), _ptr(ys[2]),
        _DTYPES[y_dtype], M, K, _mode(mode), None, 0, _stream(stream)), "qmv_int2_rmsnorm_qkv")
    return ys[0], ys[1], ys[2]


def ternary_row_bytes(K):
    """Bytes of one packed ternary row: ceil(K/80) segments of 16 bytes."""
    return (K + 79) // 80 * 16


def qmv_ternary(wq, scale, x, y=None, y_dtype=torch.float32, mode="fixed", stream=None):
    """Ternary matvec (see qmv.h).  wq uint8 [N, ternary_row_bytes(K)], scale fp16 [N],
    x fp16 [M, K]."""
    M, K = x.shape
    N = wq.shape[0]
    _req(wq, "wq", torch.uint8, (N, ternary_row_bytes(K)))
    _req(scale, "scale", torch.float16, (N,))
    _req(x, "x", torch.float16, (M, K))
    return _matvec(_lib.qmv_ternary, "qmv_ternary", wq, scale, x, y, y_dtype, mode, None, stream, "ternary")


def qmm_mxfp4_gather(wq, e8m0, x, idx, y=None, y_dtype=torch.float32, mode="fixed", stream=None):
    """Expert-gather MXFP4 matvec (see qmv.h).  wq uint8 [E,N,K/2], e8m0 uint8 [E,N,K/32],
    x bf16 [M,K], idx int32 [M,topk].  Returns y [M,topk,N]."""
    M, K = x.shape
    E, N = wq.shape[0], wq.shape[1]
    topk = idx.shape[1] if idx.dim() == 2 else -1
    _req(wq, "wq", torch.uint8, (E, N, K // 2))
    _req(e8m0, "e8m0", torch.uint8, (E, N, K // 32))
    _req(x, "x", torch.bfloat16, (M, K))
    _req(idx, "idx", torch.int32, (M, topk))
    if y is None:
        y = torch.empty((M, topk, N), dtype=y_dtype, device=x.device)
    else:
        _req(y, "y", y_dtype, (M, topk, N))
    _check(_lib.qmm_mxfp4_gather(_ptr(wq), _ptr(e8m0), E, _ptr(x), _ptr(idx), topk, _ptr(y),
                                 _DTYPES[y_dtype], M, N, K, _mode(mode), None, 0, _stream(stream)),
           "qmm_mxfp4_gather")
    return y


def qmv_int2_argmax(wq, scale, x, idx=None, maxval=None, logits=None, want_maxval=True,
                    want_logits=False, mode="fixed", workspace=None, stream=None):
    """int2 lm_head logits + first-max argmax.  Returns (idx int32 [M], maxval fp32 [M] or
    None, logits fp32 [M,N] or None).  A workspace (uint8, qmv_workspace_size bytes,
    zeroed once with workspace_init) may be passed to avoid a per-call allocation."""
    M, K = x.shape
    N = wq.shape[0]
    _req(wq, "wq", torch.int32, (N, K // 16))
    _req(scale, "scale", torch.float16, (N,))
    _req(x, "x", torch.float16, (M, K))
    dev = x.device
    idx = torch.empty(M, dtype=torch.int32, device=dev) if idx is None else _req(idx, "idx", torch.int32, (M,))
    if maxval is None and want_maxval:
        maxval = torch.empty(M, dtype=torch.float32, device=dev)
    if logits is None and want_logits:
        logits = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws, wsb = _workspace("int2_argmax", M, N, K, mode, workspace, stream)
    _check(_lib.qmv_int2_argmax(_ptr(wq), _ptr(scale), _ptr(x), _ptr(idx), _ptr(maxval),
                                _ptr(logits), M, N, K, _mode(mode), _ptr(ws), wsb, _stream(stream)),
           "qmv_int2_argmax")
    return idx, maxval, logits


def qmv_int2_argmax_static(wq, scale, x, idx, maxval=None, logits=None, mode="fixed", stream=None):
    """qmv_int2_argmax with the library's static scratch instead of a workspace
    (see qmv.h); allocates nothing, so every output is the caller's:
    idx int32 [M], maxval fp32 [M] or None, logits fp32 [M,N] or None."""
    M, K = x.shape
    N = wq.shape[0]
    _req(wq, "wq", torch.int32, (N, K // 16))
    _req(scale, "scale", torch.float16, (N,))
    _req(x, "x", torch.float16, (M, K))
    _req(idx, "idx", torch.int32, (M,))
    if maxval is not None:
        _req(maxval, "maxval", torch.float32, (M,))
    if logits is not None:
        _req(logits, "logits", torch.float32, (M, N))
    _check(_lib.qmv_int2_argmax_static(_ptr(wq), _ptr(scale), _ptr(x), _ptr(idx), _ptr(maxval), _ptr(logits),
                                       M, N, K, _mode(mode), _stream(stream)), "qmv_int2_argmax_static")
    return idx, maxval, logits
