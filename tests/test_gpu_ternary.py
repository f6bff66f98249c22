"""GPU: the ternary matvec (qmv_ternary) against the oracle, bit for bit.

Five base-3 digits per byte, rows of 80-code segments padded to whole
segments.  The cases cover the 8B-class decoder shape, K values in every
lane-layout bucket (1 to 205 segments per row) with ragged last segments,
several activation rows, the three output dtypes, and that digits past K are
never used."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, bits, dev

pytestmark = pytest.mark.gpu

q = pytest.importorskip("skinny_gemm_qmv_amd")


def run(d, y_dtype=torch.float32, wq=None):
    y = q.qmv_ternary(dev(d["wq"] if wq is None else wq, "u8"), dev(d["scale"], "f16"), dev(d["x"], "f16"),
                      y_dtype=y_dtype)
    torch.cuda.synchronize()
    return y


def reference(d):
    return oracle.qmv_ternary(d["wq"], d["scale"], d["x"])


@pytest.mark.parametrize("M,N,K", [
    (1, 16384, 4096),   # 8B-class decoder projection
    (1, 1000, 80),      # one full segment
    (1, 300, 88),       # ragged: 80 + 8
    (2, 64, 16),        # one short segment
    (3, 257, 2560),
    (1, 70, 16384),     # longest K (205 segments)
    (5, 130, 1000),
    (16, 300, 4096),    # four-row chunks
    (7, 100, 16384),    # ragged chunk at the longest K (two-row chunks)
])
def test_ternary_bit_exact(M, N, K):
    d = synth.ternary_inputs(M, N, K, salt=N + K)
    assert_bits_equal(bits(run(d)), reference(d).view(np.uint32), f"ternary M={M} N={N} K={K}")


# K in every lane-layout bucket (segments per row 1..8, ..16, ..24, ..32, ..64,
# ..96, ..128, ..192, ..256), mostly with a ragged last segment
K_TERN = [16, 600, 1000, 1840, 2560, 4096, 7000, 9600, 12000, 16384]


def test_ternary_every_lane_layout():
    for i, K in enumerate(K_TERN):
        for M, N in ((1, 65), (2, 63)):
            d = synth.ternary_inputs(M, N, K, salt=200 + i)
            assert_bits_equal(bits(run(d)), reference(d).view(np.uint32), f"ternary M={M} N={N} K={K}")


@pytest.mark.parametrize("y_dtype", [torch.float16, torch.bfloat16])
def test_ternary_low_precision_outputs(y_dtype):
    d = synth.ternary_inputs(3, 777, 1536, salt=9)
    assert torch.equal(run(d, y_dtype).cpu(), run(d).cpu().to(y_dtype))


def test_ternary_digits_past_k_unused():
    K = 4096  # 52 segments, 64 padding digits in the last one
    d = synth.ternary_inputs(1, 2000, K, salt=4)
    g = np.random.default_rng(5)
    wq2 = d["wq"].copy()
    full = -(-K // 5)
    wq2[:, full:] = g.integers(0, 243, (2000, wq2.shape[1] - full))
    r = K % 5
    if r:
        lo = wq2[:, K // 5].astype(np.int64) % 3 ** r
        wq2[:, K // 5] = (lo + 3 ** r * g.integers(0, 3 ** (5 - r), 2000)).astype(np.uint8)
    assert np.array_equal(bits(run(d)), bits(run(d, wq=wq2)))


def test_ternary_rows_equal_single_row_calls():
    d = synth.ternary_inputs(4, 500, 4096, salt=6)
    y = bits(run(d))
    for m in range(4):
        dm = dict(d)
        dm["x"] = d["x"][m:m + 1]
        assert np.array_equal(y[m], bits(run(dm))[0])
