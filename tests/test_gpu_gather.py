"""GPU: the expert-gather MXFP4 matvec (qmm_mxfp4_gather) against the oracle,
bit for bit.

Each output plane y[m][j] is the fixed-order MXFP4 matvec of activation row m
with expert idx[m][j], read in place from the [E][N][K/2] expert array.  The
cases cover the gpt-oss-sized decode shape, ragged N, one segment per row,
the longest K, many planes (up to 132 over 32 experts), duplicate ids in a
row and across rows, the three output dtypes, and ids outside
[0, E) (their plane is NaN, the others are untouched by it)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, bits, dev

pytestmark = pytest.mark.gpu

q = pytest.importorskip("skinny_gemm_qmv_amd")


def run(d, idx=None, y_dtype=torch.float32):
    ids = torch.from_numpy(np.ascontiguousarray(d["idx"] if idx is None else idx, np.int32)).cuda()
    y = q.qmm_mxfp4_gather(dev(d["wq"], "u8"), dev(d["e8m0"], "u8"), dev(d["x"], "bf16"), ids,
                           y_dtype=y_dtype)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("M,E,topk,N,K", [
    (1, 32, 4, 5760, 2880),   # gpt-oss-sized MoE projection, one decode token
    (3, 8, 2, 300, 1024),     # ragged N
    (2, 4, 4, 64, 32),        # one segment per row
    (1, 3, 3, 1000, 16384),   # longest K
    (16, 16, 4, 200, 512),    # 64 planes
    (4, 2, 2, 129, 2880),     # more picks than experts: every expert used twice
    (64, 8, 2, 96, 256),      # ~16 planes per expert
    (33, 32, 4, 640, 2880),   # 132 planes over 32 experts
    (9, 5, 3, 70, 6144),      # long K, several planes per expert
])
def test_gather_bit_exact(M, E, topk, N, K):
    d = synth.expert_inputs(M, E, topk, N, K, salt=N + K)
    y = run(d)
    want = oracle.qmm_mxfp4_gather(d["wq"], d["e8m0"], d["x"], d["idx"])
    assert_bits_equal(bits(y), want.view(np.uint32), f"M={M} E={E} topk={topk} N={N} K={K}")


def test_gather_duplicate_ids():
    d = synth.expert_inputs(3, 6, 4, 250, 640, salt=3)
    idx = np.array([[2, 2, 5, 2], [0, 5, 0, 1], [4, 4, 4, 4]], np.int32)
    y = bits(run(d, idx))
    want = oracle.qmm_mxfp4_gather(d["wq"], d["e8m0"], d["x"], idx)
    assert_bits_equal(y, want.view(np.uint32), "duplicate ids")
    assert np.array_equal(y[0, 0], y[0, 1]) and np.array_equal(y[2, 0], y[2, 3])


def test_gather_matches_plain_mxfp4_on_the_expert_slice():
    d = synth.expert_inputs(2, 5, 3, 700, 1536, salt=11)
    y = bits(run(d))
    for m in range(2):
        for j in range(3):
            e = int(d["idx"][m, j])
            y1 = q.qmm_mxfp4(dev(d["wq"][e], "u8"), dev(d["e8m0"][e], "u8"), dev(d["x"][m:m + 1], "bf16"))
            assert np.array_equal(y[m, j], bits(y1)[0])


@pytest.mark.parametrize("y_dtype", [torch.float16, torch.bfloat16])
def test_gather_low_precision_outputs(y_dtype):
    d = synth.expert_inputs(2, 8, 4, 333, 2880, salt=7)
    y32 = run(d)
    y = run(d, y_dtype=y_dtype)
    # one round-to-nearest-even of the fp32 result
    assert torch.equal(y.cpu(), y32.cpu().to(y_dtype))


def test_gather_out_of_range_ids_give_nan_planes():
    E = 4
    d = synth.expert_inputs(2, E, 3, 300, 512, salt=13)
    idx = np.array([[1, -1, E], [2**31 - 1, 3, 0]], np.int32)
    y = bits(run(d, idx)).view(np.float32)
    bad = (idx < 0) | (idx >= E)
    assert np.all(np.isnan(y[bad]))
    good = oracle.qmm_mxfp4_gather(d["wq"], d["e8m0"], d["x"], np.where(bad, 0, idx).astype(np.int32))
    assert_bits_equal(y[~bad].view(np.uint32), good[~bad].view(np.uint32), "valid planes")
