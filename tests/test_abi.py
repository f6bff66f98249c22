"""The C ABI library on a host without a GPU: it loads, exports every entry
point include/qmv.h declares, and its argument validation returns the
documented status codes.  Every call below fails validation before any HIP
call, so no GPU is touched."""
import ctypes as C
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmv.h")

q = pytest.importorskip("skinny_gemm_qmv_amd")

OK, INVALID, ALIGN, WS, UNSUP = 0, 1, 2, 3, 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmv_\w+|qmm_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("qmv_int2", "qmv_int4", "qmm_mxfp4", "qmv_int2_rmsnorm_gateup_gelu",
                 "qmv_int2_argmax", "qmv_int2_rmsnorm_qkv", "qmm_mxfp4_gather", "qmv_ternary", "qmv_int2_rmsnorm_gateup_gelu_mxfp4", "qmv_quant_mxfp4", "qmv_workspace_size", "qmv_workspace_init",
                 "qmv_status_string", "qmv_last_hip_error", "qmv_abi_version", "qmv_fo_spec"):
        assert want in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", q.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\w+)$", out, flags=re.M))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    lib = C.CDLL(q.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n)


def test_version_and_spec():
    assert q.abi_version() == 1
    assert q.fo_spec() == (16, 1, 1)
    for s in range(6):
        assert q._lib.qmv_status_string(s)


P = C.c_void_p


def _mv(fn, wq=16, sc=16, x=16, y=16, dt=0, M=1, N=64, K=64, mode=0, ws=None, wsb=0):
    return fn(P(wq) if wq else None, P(sc) if sc else None, P(x) if x else None,
              P(y) if y else None, dt, M, N, K, mode, P(ws) if ws else None, wsb, None)


@pytest.mark.parametrize("name,kmul", [("qmv_int2", 64), ("qmv_int4", 32), ("qmm_mxfp4", 32)])
def test_matvec_validation(name, kmul):
    fn = getattr(q._lib, name)
    assert _mv(fn, wq=0) == INVALID
    assert _mv(fn, sc=0) == INVALID
    assert _mv(fn, x=0) == INVALID
    assert _mv(fn, y=0) == INVALID
    assert _mv(fn, M=0) == INVALID
    assert _mv(fn, M=257) == INVALID
    assert _mv(fn, N=0) == INVALID
    assert _mv(fn, K=kmul + kmul // 2) == INVALID
    assert _mv(fn, K=0) == INVALID
    assert _mv(fn, K=16384 + kmul) == INVALID
    assert _mv(fn, dt=3) == INVALID
    assert _mv(fn, mode=7) == INVALID
    assert _mv(fn, wq=24) == ALIGN
    assert _mv(fn, x=40) == ALIGN
    assert _mv(fn, y=18) == ALIGN          # fp32 output needs 4-byte alignment
    # the output is addressed with 32-bit byte offsets: M*N*4 must stay below 4 GiB
    assert _mv(fn, M=256, N=1 << 22, K=kmul) == UNSUP
    if name != "qmm_mxfp4":
        assert _mv(fn, mode=2) == UNSUP       # matrix-core mode only for MXFP4
    else:
        assert _mv(fn, mode=2, M=16) == UNSUP  # MXFP4 matrix cores need M >= 32


def test_gateup_validation():
    fn = q._lib.qmv_int2_rmsnorm_gateup_gelu
    args = [P(16)] * 4 + [C.c_float(1e-6)] + [P(16)] * 5

    def call(args, M=1, N=64, K=64, mode=0):
        return fn(*args, M, N, K, mode, None, 0, None)
    a = list(args); a[0] = None
    assert call(a) == INVALID
    a = list(args); a[2] = None       # residual_out is optional: must not be the failure
    a[5] = None
    assert call(a) == INVALID
    assert call(args, K=96) == INVALID
    assert call(args, M=300) == INVALID
    a = list(args); a[4] = C.c_float(-1.0)
    assert call(a) == INVALID
    a = list(args); a[0] = P(18)
    assert call(a) == ALIGN
    # the prologue reads gamma and writes residual_out as 16-byte vectors
    a = list(args); a[3] = P(18)
    assert call(a) == ALIGN
    a = list(args); a[2] = P(34)
    assert call(a) == ALIGN
    assert call(args, mode=2) == UNSUP    # matrix-core mode never applies to int2
    assert call(args, M=256, N=1 << 23) == UNSUP  # fp16 output of M*N*2 >= 4 GiB (32-bit offsets)


def test_qkv_validation():
    fn = q._lib.qmv_int2_rmsnorm_qkv

    def call(ptrs=None, Ns=(64, 64, 64), dt=0, M=1, K=64, mode=0, eps=1e-6):
        p = ptrs or {}
        a = [P(p.get(i, 16)) if p.get(i, 16) else None for i in range(4)]  # x, residual, residual_out, gamma
        w = [P(p.get(4 + i, 16)) if p.get(4 + i, 16) else None for i in range(6)]  # wq/s for q, k, v
        y = [P(p.get(10 + i, 16)) if p.get(10 + i, 16) else None for i in range(3)]
        return fn(a[0], a[1], a[2], a[3], C.c_float(eps), w[0], w[1], Ns[0], w[2], w[3], Ns[1],
                  w[4], w[5], Ns[2], y[0], y[1], y[2], dt, M, K, mode, None, 0, None)
    assert call({0: 0}) == INVALID
    assert call({12: 0}) == INVALID
    assert call(Ns=(64, 0, 64)) == INVALID
    assert call(K=96) == INVALID
    assert call(M=257) == INVALID
    assert call(dt=3) == INVALID
    assert call(eps=-1.0) == INVALID
    assert call({6: 24}) == ALIGN
    assert call({10: 18}) == ALIGN
    assert call({3: 18}) == ALIGN          # gamma: 16-byte vectors
    assert call({2: 40}) == ALIGN          # residual_out: 16-byte vectors
    assert call(mode=1) == UNSUP
    assert call(M=256, Ns=(64, 1 << 22, 64)) == UNSUP  # y_k of M*N*4 >= 4 GiB


def test_gather_validation():
    fn = q._lib.qmm_mxfp4_gather

    def call(wq=16, sc=16, E=8, x=16, idx=16, topk=4, y=16, dt=0, M=1, N=64, K=64, mode=0):
        p = [P(v) if v else None for v in (wq, sc, x, idx, y)]
        return fn(p[0], p[1], E, p[2], p[3], topk, p[4], dt, M, N, K, mode, None, 0, None)
    for kw in ({"wq": 0}, {"sc": 0}, {"x": 0}, {"idx": 0}, {"y": 0}, {"E": 0}, {"topk": 0},
               {"K": 48}, {"K": 16416}, {"M": 0}, {"M": 257}, {"N": 0}, {"dt": 3}):
        assert call(**kw) == INVALID, kw
    assert call(wq=24) == ALIGN
    assert call(x=8) == ALIGN
    assert call(idx=18) == ALIGN
    assert call(y=18) == ALIGN
    assert call(mode=1) == UNSUP
    assert call(mode=2) == UNSUP
    assert call(M=256, topk=256) == UNSUP          # M*topk planes > 65535 (grid.y)
    assert call(M=64, topk=64, N=1 << 18) == UNSUP  # M*topk*N*4 >= 4 GiB
    assert call(N=1 << 19, K=16384) == UNSUP        # one expert >= 4 GiB


def test_ternary_validation():
    fn = q._lib.qmv_ternary
    assert _mv(fn, wq=0) == INVALID
    assert _mv(fn, K=12) == INVALID        # K a multiple of 8
    assert _mv(fn, K=16392) == INVALID
    assert _mv(fn, M=257) == INVALID
    assert _mv(fn, dt=5) == INVALID
    assert _mv(fn, wq=24) == ALIGN
    assert _mv(fn, x=8) == ALIGN
    assert _mv(fn, mode=1) == UNSUP
    assert _mv(fn, mode=2) == UNSUP
    assert _mv(fn, N=1 << 22, K=16384) == UNSUP  # packed weights >= 4 GiB


def test_gateup_mxfp4_validation():
    fn = q._lib.qmv_int2_rmsnorm_gateup_gelu_mxfp4

    def call(ptrs=None, M=1, N=64, K=64, mode=0, eps=1e-6, ws=None, wsb=0):
        p = ptrs or {}
        a = [P(p.get(i, 16)) if p.get(i, 16) else None for i in range(10)]
        # x, residual, residual_out, gamma, wq_gate, s_gate, wq_up, s_up, codes, e8m0
        return fn(a[0], a[1], a[2], a[3], C.c_float(eps), a[4], a[5], a[6], a[7], a[8], a[9], M, N, K, mode,
                  P(ws) if ws else None, wsb, None)
    assert call({0: 0}) == INVALID
    assert call({8: 0}) == INVALID
    assert call(N=48) == INVALID           # N a multiple of 32
    assert call(K=96) == INVALID
    assert call(eps=-1.0) == INVALID
    assert call({4: 24}) == ALIGN
    assert call({3: 18}) == ALIGN          # gamma: 16-byte vectors
    assert call({2: 40}) == ALIGN          # residual_out: 16-byte vectors
    assert call(mode=1) == UNSUP
    assert call() == WS                    # workspace required
    need = q._lib.qmv_workspace_size(8, 1, 64, 64, 0)
    assert need == 256 + 64 * 2
    assert call(ws=256, wsb=need - 2) == WS
    assert call(ws=272, wsb=need) == ALIGN
    assert q._lib.qmv_workspace_size(8, 1, 48, 64, 0) == 0


def test_quant_mxfp4_validation():
    fn = q._lib.qmv_quant_mxfp4
    assert fn(None, P(16), P(16), 1, 64, None) == INVALID
    assert fn(P(16), P(16), P(16), 1, 48, None) == INVALID
    assert fn(P(16), P(16), P(16), 0, 64, None) == INVALID
    assert fn(P(17), P(16), P(16), 1, 64, None) == ALIGN
    assert fn(P(16), P(16), P(16), 1 << 16, 1 << 15, None) == UNSUP


def test_argmax_validation():
    fn = q._lib.qmv_int2_argmax

    def call(wq=16, sc=16, x=16, idx=16, mv=None, lg=None, M=1, N=64, K=64, mode=0, ws=None, wsb=0):
        return fn(P(wq) if wq else None, P(sc) if sc else None, P(x) if x else None,
                  P(idx) if idx else None, P(mv) if mv else None, P(lg) if lg else None,
                  M, N, K, mode, P(ws) if ws else None, wsb, None)
    assert call(idx=0) == INVALID
    assert call(K=100) == INVALID
    assert call(mode=2) == UNSUP
    assert call() == WS                  # no workspace
    need = q.workspace_size("int2_argmax", 1, 64, 64)
    assert need > 0
    assert call(ws=256, wsb=need - 1) == WS
    assert call(ws=128, wsb=need) == ALIGN
    # completion counters plus one 64-bit key per activation row
    assert q.workspace_size("int2_argmax", 256, 262144, 1536) >= 1024 + 8 * 256
    assert q.workspace_size("int2_argmax", 256, 64, 64) > q.workspace_size("int2_argmax", 1, 64, 64)
    assert q.workspace_size("int2", 1, 64, 64) == 0


def test_workspace_init_validation():
    assert q._lib.qmv_workspace_init(None, 0, None) == OK
    assert q._lib.qmv_workspace_init(None, 256, None) == INVALID
    assert q._lib.qmv_workspace_init(P(128), 256, None) == ALIGN
    assert q._lib.qmv_workspace_init(P(256), 6, None) == ALIGN


def test_splitk_workspace_size_and_validation():
    # several K splits for a short-N int2 matvec: [splits][M][N] fp32 partials
    need = q.workspace_size("int2", 1, 2048, 1536, "splitk")
    assert need > 0 and need % (2048 * 4) == 0 and need // (2048 * 4) in (2, 4, 8, 16)
    assert q.workspace_size("int2", 3, 2048, 1536, "splitk") == 3 * need
    # enough rows for the whole GPU: one split, no workspace (fixed-order kernel)
    assert q.workspace_size("int2", 1, 70000, 1536, "splitk") == 0
    assert q.workspace_size("int4", 1, 16384, 4096, "splitk") == 0
    assert q.workspace_size("int2", 1, 2048, 1536, "fixed") == 0
    fn = q._lib.qmv_int2
    assert _mv(fn, M=1, N=2048, K=1536, mode=1) == WS
    assert _mv(fn, M=1, N=2048, K=1536, mode=1, ws=4096, wsb=need - 4) == WS
    assert _mv(fn, M=1, N=2048, K=1536, mode=1, ws=4096 + 16, wsb=need) == ALIGN


MEASURE_HEADER = os.path.join(ROOT, "include", "qmv_measure.h")
MEASURE_LIB = os.path.join(ROOT, "skinny_gemm_qmv_amd", "libqmv_measure.so")


def test_measure_library_exports_its_header():
    """The benchmark's reference kernels (streaming read, empty kernel): every
    function include/qmv_measure.h declares is exported, and the streaming
    read rejects bad arguments before touching the GPU."""
    if not os.path.exists(MEASURE_LIB):
        pytest.skip("libqmv_measure.so not built")
    text = re.sub(r"/\*.*?\*/", "", open(MEASURE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(qmv_measure_\w+)\s*\(", text)))
    assert names == ["qmv_measure_empty", "qmv_measure_stream_read"]
    out = subprocess.run(["nm", "-D", "--defined-only", MEASURE_LIB], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\w+)$", out, flags=re.M))
    assert all(n in exported for n in names)
    lib = C.CDLL(MEASURE_LIB)
    fn = lib.qmv_measure_stream_read
    fn.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int, C.c_void_p]
    assert fn(None, 4096, P(256), 0, None) == 1
    assert fn(P(256), 4096, None, 0, None) == 1
    assert fn(P(256), 0, P(256), 0, None) == 1
    assert fn(P(256), 4100, P(256), 0, None) == 1      # not a multiple of 16 bytes
    assert fn(P(264), 4096, P(256), 0, None) == 1      # source not 16-byte aligned
