"""GPU: the shared-prologue q/k/v entry point (qmv_int2_rmsnorm_qkv) against the
oracle, bit for bit.

One dispatch computes the residual-add RMSNorm of each activation row and the
three int2 fixed-order matvecs q, k, v of the normalised row.  Every output
must equal the oracle's composition exactly, for row counts that differ per
matrix (workgroups are shared out between q, k and v), ragged shapes, several
activation rows, every lane layout the K range selects, and the three output
dtypes; residual_out must hold h = fp16(x + residual)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, bits, dev

pytestmark = pytest.mark.gpu

q = pytest.importorskip("skinny_gemm_qmv_amd")


def run(d, y_dtype=torch.float32, residual_out=None):
    ys = q.qmv_int2_rmsnorm_qkv(dev(d["x"], "f16"), dev(d["residual"], "f16"), dev(d["gamma"], "f16"),
                                d["eps"], dev(d["wq_q"], "u32"), dev(d["s_q"], "f16"), dev(d["wq_k"], "u32"),
                                dev(d["s_k"], "f16"), dev(d["wq_v"], "u32"), dev(d["s_v"], "f16"),
                                y_dtype=y_dtype, residual_out=residual_out)
    torch.cuda.synchronize()
    return ys


def reference(d):
    return oracle.int2_rmsnorm_qkv(d["x"], d["residual"], d["gamma"], d["eps"], d["wq_q"], d["s_q"],
                                   d["wq_k"], d["s_k"], d["wq_v"], d["s_v"])


@pytest.mark.parametrize("M,Nq,Nk,Nv,K", [
    (1, 2048, 512, 512, 1536),   # the q/k/v benchmark shape
    (1, 1000, 17, 300, 640),     # ragged, very unequal row counts
    (3, 257, 64, 129, 2048),
    (2, 48, 48, 48, 64),         # one segment per row
    (1, 4096, 1024, 1024, 4096),
    (1, 70, 33, 5, 16384),
])
def test_qkv_bit_exact(M, Nq, Nk, Nv, K):
    d = synth.qkv_inputs(M, Nq, Nk, Nv, K, salt=Nq + K)
    res_out = torch.empty((M, K), dtype=torch.float16, device="cuda")
    ys = run(d, residual_out=res_out)
    want = reference(d)
    for z, y, w in zip("qkv", ys, want[:3]):
        assert_bits_equal(bits(y), w.view(np.uint32), f"y_{z} M={M} N=({Nq},{Nk},{Nv}) K={K}")
    assert_bits_equal(bits(res_out), want[3], "residual_out")


@pytest.mark.parametrize("y_dtype", [torch.float16, torch.bfloat16])
def test_qkv_low_precision_outputs(y_dtype):
    d = synth.qkv_inputs(2, 300, 100, 100, 1536, salt=5)
    y32 = run(d)
    ys = run(d, y_dtype)
    for a, b in zip(ys, y32):
        # one round-to-nearest-even of the fp32 result
        assert torch.equal(a.cpu(), b.cpu().to(y_dtype))


def test_qkv_rows_equal_single_row_calls():
    d = synth.qkv_inputs(4, 200, 64, 64, 1536, salt=9)
    ys = run(d)
    for m in range(4):
        dm = dict(d)
        dm["x"], dm["residual"] = d["x"][m:m + 1], d["residual"][m:m + 1]
        y1 = run(dm)
        for a, b in zip(ys, y1):
            assert np.array_equal(bits(a)[m:m + 1], bits(b))
