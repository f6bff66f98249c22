"""GPU: the matrix-core mode of qmm_mxfp4 (M >= 32) against the oracle.

This mode sums in the matrix cores' order, so it is held to the tolerance
class instead of bit equality:
  * relative L2 error <= 2e-3 against the fixed-order oracle, over the whole
    output and over every activation row separately;
  * elementwise, |y - exact| <= gamma_K * sum_k |w_k x_k| with
    gamma_K = K u / (1 - K u), u = 2^-24: the classical bound for any order of
    fp32 summation of K exact products (weights dequantize exactly to bf16, so
    every product is exact).  The exact value and sum |w x| come from the
    oracle's fp64 reference.
The elementwise bound catches a single wrong output, which a global L2 norm
over millions of outputs would not."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import bits, dev, rel_l2

pytestmark = pytest.mark.gpu

q = pytest.importorskip("skinny_gemm_qmv_amd")

TOL = 2e-3


def gpu_mfma(d, y_dtype=torch.float32):
    y = q.qmm_mxfp4(dev(d["wq"], "u8"), dev(d["e8m0"], "u8"), dev(d["x"], "bf16"), y_dtype=y_dtype,
                    mode="mfma")
    torch.cuda.synchronize()
    return y


def check_close(y, d, rows=None, what=""):
    """y: float64 [M, n] for the weight rows `rows` (all rows if None)."""
    wq, e8 = d["wq"], d["e8m0"]
    if rows is not None:
        wq, e8 = wq[rows], e8[rows]
    K = d["x"].shape[1]
    fo = oracle.qmm_mxfp4(wq, e8, d["x"]).astype(np.float64)
    exact, mag = oracle.ref64_mxfp4(wq, e8, d["x"])
    u = 2.0 ** -24
    gamma = K * u / (1.0 - K * u)
    err = np.abs(y - exact)
    bound = gamma * mag + 1e-38
    bad = np.argwhere(err > bound)
    assert bad.size == 0, f"{what}: {len(bad)} outputs outside the summation bound, first {bad[0]}: " \
                          f"got {y[tuple(bad[0])]!r}, exact {exact[tuple(bad[0])]!r}"
    r = rel_l2(y, fo)
    assert r <= TOL, (what, r)
    for m in range(y.shape[0]):
        assert rel_l2(y[m], fo[m]) <= TOL, (what, m)
    return r


@pytest.mark.parametrize("M", [64, 256])
def test_workload5_mfma_sampled_rows(M):
    """Full MXFP4 workload (N=21504, K=5376) in the launch shape the benchmark
    times; the oracle checks a sample of weight rows against every output
    column of the sample."""
    d = synth.mxfp4_inputs(M, 21504, 5376, workload=5)
    y = gpu_mfma(d)
    g = np.random.default_rng(100 + M)
    rows = np.unique(np.concatenate([[0, 1, 15, 16, 21487, 21503], g.choice(21504, 250, replace=False)]))
    yc = y.cpu().numpy().astype(np.float64)[:, rows]
    check_close(yc, d, rows, f"mxfp4 mfma M={M}")


@pytest.mark.parametrize("M,N,K", [
    (32, 16, 32),        # one tile, one block of 32
    (33, 17, 160),       # ragged M, ragged N, K with a partial 128-chunk (5 blocks)
    (47, 257, 1024),
    (64, 1000, 544),
    (100, 4100, 1024),   # grid of 256 workgroups with unequal tile counts
    (128, 1000, 4096),
    (129, 300, 96),
    (192, 700, 5376),
    (255, 64, 8192),
    (256, 2049, 512),
    (32, 40000, 256),    # more tiles than 256 workgroups x 8: extra workgroups
    # K a multiple of 128: one 16-byte scale load per tile covers four chunks
    (32, 17, 128),       # the last row's scale group runs past the end of the scales
    (40, 33, 384),       # 33 x 12 scale bytes: the last group straddles the end
    (64, 1, 1152),       # a single weight row
])
def test_mfma_shapes(M, N, K):
    d = synth.mxfp4_inputs(M, N, K, salt=M + N + K)
    y = gpu_mfma(d).cpu().numpy().astype(np.float64)
    check_close(y, d, None, f"M={M} N={N} K={K}")


@pytest.mark.parametrize("y_dtype", [torch.float16, torch.bfloat16])
def test_mfma_low_precision_outputs(y_dtype):
    d = synth.mxfp4_inputs(64, 515, 1024, salt=9)
    y32 = gpu_mfma(d)
    y = gpu_mfma(d, y_dtype)
    # one round-to-nearest-even of the fp32 result
    assert torch.equal(y.cpu(), y32.cpu().to(y_dtype))


def test_mfma_deterministic_and_scale_range():
    d = synth.mxfp4_inputs(96, 600, 2048, salt=21, exp_range=(-40, 40))
    a = bits(gpu_mfma(d))
    for _ in range(5):
        b = bits(gpu_mfma(d))
        assert np.array_equal(a, b)
    check_close(a.view(np.float32).astype(np.float64), d, None, "wide exponent range")


def test_mfma_rejects_narrow_batches():
    d = synth.mxfp4_inputs(31, 64, 64, salt=1)
    with pytest.raises(q.QmvError):
        gpu_mfma(d)


def test_mfma_exact_on_integer_inputs():
    """Integer activations in [-8, 8] and block scales 2^0 / 2^1: every product
    and every partial sum is exact in fp32 (multiples of 0.5 below 2^20), so
    the matrix cores must give the exact result bit for bit."""
    g = np.random.default_rng(7)
    M, N, K = 96, 1000, 5376
    d = dict(wq=synth.raw_bytes(g, (N, K // 2)),
             e8m0=(127 + g.integers(0, 2, (N, K // 32))).astype(np.uint8),
             x=synth.bf16_bits(g.integers(-8, 9, (M, K)).astype(np.float64)))
    y = gpu_mfma(d).cpu().numpy().astype(np.float64)
    exact, _ = oracle.ref64_mxfp4(d["wq"], d["e8m0"], d["x"])
    assert np.array_equal(y, exact)
