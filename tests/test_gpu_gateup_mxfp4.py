"""GPU: the fused activation-and-quantize entry point
(qmv_int2_rmsnorm_gateup_gelu_mxfp4) and the standalone MXFP4 quantiser
(qmv_quant_mxfp4) against the oracle, bit for bit.

The fused call must give exactly the MXFP4 quantisation of the fused gate/up
fp16 output (codes and E8M0 bytes), for one and several activation rows,
several lane layouts, a single block, and repeated calls on one workspace
(the per-block counters must come back to zero).  The quantiser alone is
checked on blocks with planted rounding ties, values at and past the clamp,
signed zeros, subnormals and all-zero blocks."""
import numpy as np
import pytest
import torch

import oracle
import oracle_pins
import synth
from gpu_util import dev

pytestmark = pytest.mark.gpu

q = pytest.importorskip("skinny_gemm_qmv_amd")


def args(d):
    return (dev(d["x"], "f16"), dev(d["residual"], "f16"), dev(d["gamma"], "f16"), d["eps"],
            dev(d["wq_gate"], "u32"), dev(d["s_gate"], "f16"), dev(d["wq_up"], "u32"), dev(d["s_up"], "f16"))


def oargs(d):
    return (d["x"], d["residual"], d["gamma"], d["eps"], d["wq_gate"], d["s_gate"], d["wq_up"], d["s_up"])


@pytest.mark.parametrize("M,N,K", [
    (1, 8192, 1536),   # the fused workload
    (3, 96, 1536),
    (2, 4096, 4096),
    (5, 64, 64),
    (1, 32, 1536),     # one block
    (4, 320, 1536),    # several rows per workgroup
    (9, 160, 2048),
    (1, 1024, 4096),   # 64 segments per row: eight lanes x eight segments
    (1, 96, 8192),     # 128 segments: the counter fallback
    (3, 64, 6144),
])
def test_gateup_mxfp4_bit_exact(M, N, K):
    d = synth.fused_inputs(M, N, K, salt=N + K)
    res = torch.empty((M, K), dtype=torch.float16, device="cuda")
    codes, e8 = q.qmv_int2_rmsnorm_gateup_gelu_mxfp4(*args(d), residual_out=res)
    torch.cuda.synchronize()
    wc, we, wres = oracle.int2_rmsnorm_gateup_gelu_mxfp4(*oargs(d))
    assert np.array_equal(e8.cpu().numpy(), we), f"E8M0 M={M} N={N} K={K}"
    assert np.array_equal(codes.cpu().numpy(), wc), f"codes M={M} N={N} K={K}"
    assert np.array_equal(res.cpu().view(torch.int16).numpy().view(np.uint16), wres)


def test_gateup_mxfp4_equals_quantised_fused_output():
    d = synth.fused_inputs(2, 2048, 1536, salt=8)
    codes, e8 = q.qmv_int2_rmsnorm_gateup_gelu_mxfp4(*args(d))
    out = q.qmv_int2_rmsnorm_gateup_gelu(*args(d))
    c2, e2 = q.qmv_quant_mxfp4(out)
    torch.cuda.synchronize()
    assert torch.equal(codes, c2) and torch.equal(e8, e2)


def test_gateup_mxfp4_workspace_reuse():
    M, N, K = 3, 1024, 1536
    need = q.workspace_size("int2_gateup_mxfp4", M, N, K)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    q.workspace_init(ws)
    first = None
    for salt in (1, 1, 2, 1):
        d = synth.fused_inputs(M, N, K, salt=salt)
        codes, e8 = q.qmv_int2_rmsnorm_gateup_gelu_mxfp4(*args(d), workspace=ws)
        torch.cuda.synchronize()
        wc, we, _ = oracle.int2_rmsnorm_gateup_gelu_mxfp4(*oargs(d))
        assert np.array_equal(codes.cpu().numpy(), wc) and np.array_equal(e8.cpu().numpy(), we), salt
        cnt_bytes = (M * (N // 32) * 4 + 255) // 256 * 256
        assert int(ws[:cnt_bytes].count_nonzero()) == 0  # every block counter back at zero
        if salt == 1:
            first = codes.cpu() if first is None else first
            assert torch.equal(codes.cpu(), first)


def test_quant_mxfp4_planted_cases():
    g = np.random.default_rng(72)
    v = oracle_pins._mx_blocks(g, 600).reshape(20, 30 * 32)
    codes, e8 = q.qmv_quant_mxfp4(torch.from_numpy(v.view(np.float16)).cuda())
    torch.cuda.synchronize()
    wc, we = oracle.quant_mxfp4(v)
    assert np.array_equal(e8.cpu().numpy(), we)
    bad = np.flatnonzero(codes.cpu().numpy().ravel() != wc.ravel())
    assert bad.size == 0, (bad[:8], codes.cpu().numpy().ravel()[bad[:8]], wc.ravel()[bad[:8]])


def test_quant_mxfp4_every_fp16_value():
    # every finite fp16 pattern, in blocks whose maximum is set by a planted
    # value, so each pattern is rounded at several block exponents
    allv = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    fin = allv[np.isfinite(allv.view(np.float16))]
    g = np.random.default_rng(73)
    fin = fin[g.permutation(fin.size)]
    nb = fin.size // 31
    blocks = fin[:nb * 31].reshape(nb, 31)
    tops = synth.f16_bits(np.ldexp(1.0, g.integers(-10, 13, nb)) * g.choice([4.0, 6.0, 7.5], nb))
    v = np.concatenate([tops[:, None], blocks], axis=1)
    v = v[: (v.shape[0] // 16) * 16].reshape(-1, 16 * 32)
    codes, e8 = q.qmv_quant_mxfp4(torch.from_numpy(np.ascontiguousarray(v).view(np.float16)).cuda())
    torch.cuda.synchronize()
    wc, we = oracle.quant_mxfp4(v)
    assert np.array_equal(e8.cpu().numpy(), we)
    assert np.array_equal(codes.cpu().numpy(), wc)
