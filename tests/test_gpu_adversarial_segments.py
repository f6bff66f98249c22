"""GPU parity of the one-column int2 / int4 kernels on adversarial activations.

Within a 16-byte segment every partial sum of the fixed order is a multiple
of Q, the finest quantum among the segment's fp16 activations; whether a step
can round depends on how the sums compare with 2^24 Q.  These inputs sit on
that edge: segments whose activation sums are exactly at (A + B) max(P, N) =
2^24 Q - 1 and a few quanta past it (P, N the sums of positive values and of
negative magnitudes, codes in [-B, A]), met by rows of extreme codes (all
+1 / -2 / -1 / 0 for int2; all +7 / -8 / 0 for int4) that push the partial
sums to their largest magnitudes, mixed with Gaussian, tiny-valued, integer
and signed-zero segments in every lane layout, ragged N, and the argmax
kernel on the same inputs.  Every output must be the oracle's bits.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, bits, dev

pytestmark = pytest.mark.gpu

q = pytest.importorskip("skinny_gemm_qmv_amd")

F16 = np.float16


def fp16_of_multiple(X):
    """x = X * 2^-24 as fp16 bits (X must make it exactly representable)."""
    v = np.float64(X) * 2.0 ** -24
    h = np.array([v], np.float64).astype(F16)
    assert float(h[0]) == v, X
    return int(h.view(np.uint16)[0])


def representable_floor(X):
    """Largest Y <= X with Y * 2^-24 exactly representable in fp16."""
    if X < 2048:
        return int(X)
    step = 1 << (int(X).bit_length() - 11)
    return (int(X) // step) * step


def edge_segment(L, target, sign, rng):
    """L activations, all of one sign, with quantum Q = 2^-24 (one value is
    2^-24) and sum of magnitudes exactly target * Q."""
    big = representable_floor((target - 1 - 1000) // (L - 2))
    rest = target - 1 - (L - 2) * big
    assert 0 < rest < 2048, (target, big, rest)
    X = np.array([1, rest] + [big] * (L - 2), np.int64)
    rng.shuffle(X)
    h = np.array([fp16_of_multiple(v) for v in X], np.uint16)
    if sign < 0:
        h |= 0x8000
    return h


def gauss_segment(L, rng):
    return rng.standard_normal(L).astype(F16).view(np.uint16)


def tiny_segment(L, rng):
    v = rng.standard_normal(L)
    v[rng.integers(0, L, 2)] *= 2.0 ** -14  # a couple of very small values: ordinary step
    return v.astype(F16).view(np.uint16)


def int_segment(L, rng):
    return rng.integers(-8, 9, L).astype(F16).view(np.uint16)


def zero_segment(L, rng, neg=False):
    return np.full(L, 0x8000 if neg else 0, np.uint16)


def x_row(L, nseg, kinds, rng):
    parts = []
    for j in range(nseg):
        k = kinds[j % len(kinds)]
        if k == "gauss":
            parts.append(gauss_segment(L, rng))
        elif k == "tiny":
            parts.append(tiny_segment(L, rng))
        elif k == "int":
            parts.append(int_segment(L, rng))
        elif k == "zero":
            parts.append(zero_segment(L, rng))
        elif k == "negzero":
            parts.append(zero_segment(L, rng, True))
        else:  # ("edge", target_offset, sign)
            _, off, sign = k
            thr = (1 << 24) // (3 if L == 64 else 15)  # largest max(P, N) below 2^24 Q / (A + B)
            if (3 if L == 64 else 15) * thr == (1 << 24):
                thr -= 1
            parts.append(edge_segment(L, thr + off, sign, rng))
    return np.concatenate(parts)


def int2_rows(N, K, rng):
    """Rows of extreme codes (all +1, all -2, all -1, all 0) then random."""
    wq = rng.integers(0, 2 ** 32, size=(N, K // 16), dtype=np.uint64).astype(np.uint32)
    for r, word in enumerate((0x55555555, 0xAAAAAAAA, 0xFFFFFFFF, 0x00000000)):
        if r < N:
            wq[r] = word
    return wq


def int4_rows(N, K, rng):
    """Rows of extreme codes (all 15 -> +7, all 0 -> -8, all 8 -> 0) then random."""
    wq = rng.integers(0, 2 ** 32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    for r, word in enumerate((0xFFFFFFFF, 0x00000000, 0x88888888)):
        if r < N:
            wq[r] = word
    return wq


# at the edge and past it: at +2 quanta, code-biased partial sums of the
# all-maximal-code rows are odd multiples of Q above 2^24 Q, which binary32
# cannot hold (a summation that relied on exactness there would come out one
# quantum off)
EDGE = [("edge", 0, 1), ("edge", 2, 1), ("edge", 0, -1), ("edge", 2, -1), ("edge", 1, 1), ("edge", 3, -1)]


def run_int2(x, wq, scale):
    N = wq.shape[0]
    K = x.shape[-1]
    y = q.qmv_int2(dev(wq, "u32"), dev(scale, "f16"), dev(x.reshape(1, K), "f16"))
    torch.cuda.synchronize()
    assert_bits_equal(bits(y), oracle.qmv_int2(wq, scale, x.reshape(1, K)).view(np.uint32), f"int2 N={N} K={K}")


def run_int4(x, wq, scales):
    N = wq.shape[0]
    K = x.shape[-1]
    y = q.qmv_int4(dev(wq, "u32"), dev(scales, "f16"), dev(x.reshape(1, K), "f16"))
    torch.cuda.synchronize()
    assert_bits_equal(bits(y), oracle.qmv_int4(wq, scales, x.reshape(1, K)).view(np.uint32), f"int4 N={N} K={K}")


# every int2 lane layout with two or more slots per lane: K = 1536 (8 lanes x
# 3), 6144 (32 x 3), 8192 (32 x 4), 12288 (64 x 3), 16384 (64 x 4); N large
# enough that every wave runs several units
ROWS = {1536: 131072, 6144: 65536, 8192: 16384, 12288: 32768, 16384: 8192}


@pytest.mark.parametrize("K", [1536, 6144, 8192, 12288, 16384])
def test_int2_threshold_segments(K):
    rng = np.random.default_rng(K)
    nseg = K // 64
    N = ROWS[K]
    x = x_row(64, nseg, EDGE + ["gauss", "tiny", "int", "zero", "negzero", "gauss"], rng)
    wq = int2_rows(N, K, rng)
    scale = np.full(N, 0x3C00, np.uint16)  # 1.0: the raw sums
    scale[8:] = synth.f16_bits(rng.uniform(0.01, 0.05, N - 8))
    run_int2(x, wq, scale)


@pytest.mark.parametrize("K", [4096, 8192, 16384])
def test_int4_threshold_segments(K):
    rng = np.random.default_rng(K + 1)
    nseg = K // 32
    N = {4096: 32768, 8192: 16384, 16384: 8192}[K]
    x = x_row(32, nseg, EDGE + ["gauss", "tiny", "int", "zero", "negzero"], rng)
    wq = int4_rows(N, K, rng)
    scales = np.full((N, K // 32), 0x3C00, np.uint16)
    scales[8:] = synth.f16_bits(rng.uniform(0.005, 0.02, (N - 8, K // 32)))
    run_int4(x, wq, scales)


@pytest.mark.parametrize("kinds", [["int"], ["tiny"], ["gauss"], ["zero"], ["negzero", "int"],
                                   [("edge", 2, 1)], [("edge", 0, -1)]],
                         ids=["integers", "tiny-values", "gauss", "zeros", "negzero+int", "past-edge",
                              "at-edge"])
def test_uniform_segment_kinds(kinds):
    rng = np.random.default_rng(7)
    K, N = 1536, 131071  # ragged N
    x = x_row(64, K // 64, kinds, rng)
    wq = int2_rows(N, K, rng)
    scale = synth.f16_bits(rng.uniform(0.01, 0.05, N))
    run_int2(x, wq, scale)
    x4 = x_row(32, 4096 // 32, kinds, rng)
    N = 40001
    wq4 = int4_rows(N, 4096, rng)
    sc4 = synth.f16_bits(rng.uniform(0.005, 0.02, (N, 128)))
    run_int4(x4, wq4, sc4)


@pytest.mark.parametrize("seed", range(4))
def test_random_segment_mixes(seed):
    """Random mixes of segment kinds over the lanes' slots."""
    rng = np.random.default_rng(100 + seed)
    kinds = ["gauss", "tiny", "int", "zero", ("edge", 0, 1), ("edge", 2, -1)]
    for K in (1536, 8192):
        nseg = K // 64
        pick = [kinds[i] for i in rng.integers(0, len(kinds), nseg)]
        x = x_row(64, nseg, pick, rng)
        N = int(rng.integers(100000, 140000) if K == 1536 else rng.integers(3000, 40000))
        wq = int2_rows(N, K, rng)
        run_int2(x, wq, synth.f16_bits(rng.uniform(0.01, 0.05, N)))
    nseg = 128
    pick = [kinds[i] for i in rng.integers(0, len(kinds), nseg)]
    x4 = x_row(32, nseg, pick, rng)
    N = int(rng.integers(30000, 60000))
    run_int4(x4, int4_rows(N, 4096, rng), synth.f16_bits(rng.uniform(0.005, 0.02, (N, 128))))


def test_argmax_threshold_segments():
    rng = np.random.default_rng(11)
    K, N = 1536, 262144
    x = x_row(64, K // 64, EDGE + ["gauss", "tiny", "int", "zero"], rng)
    wq = int2_rows(N, K, rng)
    scale = synth.f16_bits(rng.uniform(0.01, 0.05, N))
    idx, mv, lg = q.qmv_int2_argmax(dev(wq, "u32"), dev(scale, "f16"), dev(x.reshape(1, K), "f16"),
                                    want_logits=True)
    torch.cuda.synchronize()
    ri, rm, rl = oracle.int2_argmax(wq, scale, x.reshape(1, K))
    assert_bits_equal(bits(lg), rl.view(np.uint32).reshape(1, N), "logits")
    assert int(idx.cpu()[0]) == int(ri[0])
    assert_bits_equal(bits(mv), rm.view(np.uint32), "max")
