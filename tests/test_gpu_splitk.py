"""GPU: the split-K mode of qmv_int2 / qmv_int4 / qmm_mxfp4 against the oracle.

Split-K sums each K range separately and adds the partial sums in a second
kernel, so it belongs to the tolerance class:
  * relative L2 error <= 2e-3 against the fixed-order oracle, over the whole
    output and over every activation row;
  * elementwise |y - exact| <= gamma_n * sum_k |w_k x_k| (u = 2^-24,
    gamma_n = n u / (1 - n u), n = K + 8 roundings on the longest path: the
    products are exact; segment scales, split partials, the final sum and the
    int2 row scale each add a rounding), with the exact value and sum |w x|
    from the oracle's fp64 reference;
  * bit-identical results on repeated calls (the partials are summed in a
    fixed split order).
Shapes include ones where the library picks several splits (small N), a
ragged last split (segment count not divisible by the split count) and one
large enough that it keeps a single split (then the fixed-order kernel runs)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import bits, dev, rel_l2

pytestmark = pytest.mark.gpu

q = pytest.importorskip("skinny_gemm_qmv_amd")

TOL = 2e-3


def run(fmt, d, mode):
    if fmt == "int2":
        y = q.qmv_int2(dev(d["wq"], "u32"), dev(d["scale"], "f16"), dev(d["x"], "f16"), mode=mode)
    elif fmt == "int4":
        y = q.qmv_int4(dev(d["wq"], "u32"), dev(d["scales"], "f16"), dev(d["x"], "f16"), mode=mode)
    else:
        y = q.qmm_mxfp4(dev(d["wq"], "u8"), dev(d["e8m0"], "u8"), dev(d["x"], "bf16"), mode=mode)
    torch.cuda.synchronize()
    return y


def references(fmt, d):
    if fmt == "int2":
        fo = oracle.qmv_int2(d["wq"], d["scale"], d["x"])
        exact, mag = oracle.ref64_int2(d["wq"], d["scale"], d["x"])
    elif fmt == "int4":
        fo = oracle.qmv_int4(d["wq"], d["scales"], d["x"])
        exact, mag = oracle.ref64_int4(d["wq"], d["scales"], d["x"])
    else:
        fo = oracle.qmm_mxfp4(d["wq"], d["e8m0"], d["x"])
        exact, mag = oracle.ref64_mxfp4(d["wq"], d["e8m0"], d["x"])
    return fo.astype(np.float64), exact, mag


def inputs(fmt, M, N, K, salt):
    if fmt == "int2":
        return synth.int2_inputs(M, N, K, salt=salt)
    if fmt == "int4":
        return synth.int4_inputs(M, N, K, salt=salt)
    return synth.mxfp4_inputs(M, N, K, salt=salt)


CASES = [
    ("int2", 1, 2048, 1536),     # the int2 matvec workload: 4 splits
    ("int2", 3, 1000, 4096),
    ("int2", 2, 300, 16384),
    ("int2", 1, 70000, 1536),    # enough rows: one split, fixed-order kernel
    ("int4", 1, 1024, 4096),
    ("int4", 2, 333, 1184),      # 37 segments: ragged last split
    ("int4", 16, 500, 2048),
    ("int4", 1, 2048, 16384),
    ("mxfp4", 1, 1024, 5376),
    ("mxfp4", 16, 3000, 5376),
    ("mxfp4", 64, 700, 2048),
]


@pytest.mark.parametrize("fmt,M,N,K", CASES)
def test_splitk_within_tolerance(fmt, M, N, K):
    d = inputs(fmt, M, N, K, salt=7 + M + K)
    y = run(fmt, d, "splitk")
    fo, exact, mag = references(fmt, d)
    yd = y.cpu().numpy().astype(np.float64)
    u = 2.0 ** -24
    n = K + 8
    gamma = n * u / (1.0 - n * u)
    bad = np.argwhere(np.abs(yd - exact) > gamma * mag + 1e-38)
    assert bad.size == 0, (fmt, M, N, K, len(bad), bad[0])
    assert rel_l2(yd, fo) <= TOL
    for m in range(M):
        assert rel_l2(yd[m], fo[m]) <= TOL, (fmt, M, N, K, m)
    b0 = bits(y)
    for _ in range(3):
        assert np.array_equal(bits(run(fmt, d, "splitk")), b0)


def test_splitk_caller_workspace_reused():
    """A caller-provided workspace serves consecutive calls of different shapes."""
    d1 = inputs("int2", 1, 2048, 1536, salt=3)
    d2 = inputs("int2", 2, 1500, 4096, salt=4)
    need = max(q.workspace_size("int2", 1, 2048, 1536, "splitk"), q.workspace_size("int2", 2, 1500, 4096, "splitk"))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for d in (d1, d2, d1):
        y = q.qmv_int2(dev(d["wq"], "u32"), dev(d["scale"], "f16"), dev(d["x"], "f16"), mode="splitk", workspace=ws)
        torch.cuda.synchronize()
        fo, _, _ = references("int2", d)
        assert rel_l2(y.cpu().numpy(), fo) <= TOL


def _integer_inputs(fmt, M, N, K, seed):
    """Integer activations in [-8, 8] and power-of-two scales chosen so that
    every partial sum in any order is exactly representable in fp32 (the
    bound on |sum| over the resolution of the terms stays below 2^24)."""
    g = np.random.default_rng(seed)
    if fmt == "mxfp4":
        x = synth.bf16_bits(g.integers(-8, 9, (M, K)).astype(np.float64))
        return dict(wq=synth.raw_bytes(g, (N, K // 2)), x=x,
                    e8m0=(127 + g.integers(0, 2, (N, K // 32))).astype(np.uint8))
    x = synth.f16_bits(g.integers(-8, 9, (M, K)).astype(np.float64))
    if fmt == "int2":
        return dict(wq=synth.raw_words(g, (N, K // 16)), x=x,
                    scale=synth.f16_bits(np.ldexp(1.0, g.integers(-4, 3, N))))
    return dict(wq=synth.raw_words(g, (N, K // 8)), x=x,
                scales=synth.f16_bits(np.ldexp(1.0, g.integers(-2, 2, (N, K // 32)))))


@pytest.mark.parametrize("fmt,M,N,K", [("int2", 2, 1000, 4096), ("int4", 3, 777, 4096), ("mxfp4", 5, 600, 5376)])
def test_splitk_exact_on_integer_inputs(fmt, M, N, K):
    """With every partial sum exact, split-K must equal the exact result bit
    for bit whatever its summation order."""
    d = _integer_inputs(fmt, M, N, K, seed={"int2": 11, "int4": 12, "mxfp4": 13}[fmt])
    assert q.workspace_size(fmt, M, N, K, "splitk") > 0  # really split
    y = run(fmt, d, "splitk")
    _, exact, _ = references(fmt, d)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), exact)
