"""Seeded synthetic inputs for the quantized matvec / skinny GEMM workloads.

This module only draws random tensors with the shapes and value
distributions of the workloads; it contains none of the method's arithmetic
(no decoding, no products, no sums).  Both the HIP path (through the tests
and the benchmark) and the CPU oracle consume exactly these host buffers.

Conventions:
  * fp16 / bf16 tensors are returned as ``np.uint16`` bit patterns; every
    draw is made in float64 and rounded once, to nearest-even;
  * packed int2 / int4 weights are ``np.uint32`` words of raw uniform random
    bits: since every 2-bit (4-bit) field pattern is one code, uniform bits
    are exactly uniform codes ({-2,-1,0,1} for int2, 0..15 for int4);
  * MXFP4 elements are raw uniform random bytes (uniform over the 16 E2M1
    code points) and E8M0 scales are 127 + an integer uniform in [-8, 2].

Workloads (the shapes the benchmark and the parity tests use):
  1  int2 matvec        M=1,  N=2048,   K=1536, scale ~U(0.01,0.05)
  2  int4 skinny GEMM   M in {1,4,8,16}, N=16384, K=4096, group-32 scales ~U(0.005,0.02)
  3  fused RMSNorm -> int2 gate/up -> GELU*up   M=1, N=8192 (x2), K=1536
  4  int2 lm_head + argmax   M in {1,4}, N=262144, K=1536
  5  MXFP4 GEMM         M in {1,16,64,256}, N=21504, K=5376, x bf16
  6  fused RMSNorm -> int2 q/k/v   M=1, N=2048+512+512, K=1536
  7  MXFP4 expert gather  M=1, E=32 experts, topk=4, N=5760, K=2880 (a gpt-oss-sized
                          MoE up/gate projection; ids drawn uniformly without repeats)
  8  ternary matvec     M=1, N=16384, K=4096 (an 8B-class decoder projection), five
                          base-3 digits per byte, per-row fp16 scales ~U(0.01,0.05)
"""
import numpy as np

WORKLOADS = {
    1: dict(name="int2 matvec", fmt="int2", N=2048, K=1536, Ms=(1,)),
    2: dict(name="int4 skinny GEMM", fmt="int4", N=16384, K=4096, Ms=(1, 4, 8, 16)),
    3: dict(name="fused rmsnorm gate/up gelu", fmt="fused", N=8192, K=1536, Ms=(1,)),
    4: dict(name="int2 lm_head argmax", fmt="argmax", N=262144, K=1536, Ms=(1, 4)),
    5: dict(name="mxfp4 GEMM", fmt="mxfp4", N=21504, K=5376, Ms=(1, 16, 64, 256)),
}


def rng(workload, M, salt=0):
    """The generator for one workload and batch width (PCG64, fixed seed words)."""
    return np.random.Generator(np.random.PCG64([int(workload), int(M), int(salt)]))


def f16_bits(a):
    """float64 array -> fp16 bit patterns (one round-to-nearest-even)."""
    return np.asarray(a, np.float64).astype(np.float16).view(np.uint16)


def bf16_bits(a):
    """float64 array -> bf16 bit patterns (one round-to-nearest-even, normal range)."""
    a = np.asarray(a, np.float64)
    m, e = np.frexp(a)                       # a = m * 2^e, |m| in [0.5, 1)
    q = np.ldexp(np.rint(m * 256.0), e - 8)  # 8 significant bits, ties to even
    return (q.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def raw_words(g, shape):
    return g.integers(0, 2**32, size=shape, dtype=np.uint64).astype(np.uint32)


def raw_bytes(g, shape):
    return g.integers(0, 256, size=shape, dtype=np.uint16).astype(np.uint8)


def int2_inputs(M, N, K, workload=1, salt=0, scale_range=(0.01, 0.05)):
    """Packed int2 weights [N][K/16], per-row fp16 scales [N], fp16 x [M][K]."""
    g = rng(workload, M, salt)
    wq = raw_words(g, (N, K // 16))
    scale = f16_bits(g.uniform(*scale_range, size=N))
    x = f16_bits(g.standard_normal((M, K)))
    return dict(wq=wq, scale=scale, x=x)


def int4_inputs(M, N, K, workload=2, salt=0, scale_range=(0.005, 0.02)):
    """Packed int4 weights [N][K/8], group-32 fp16 scales [N][K/32], fp16 x [M][K]."""
    g = rng(workload, M, salt)
    wq = raw_words(g, (N, K // 8))
    scales = f16_bits(g.uniform(*scale_range, size=(N, K // 32)))
    x = f16_bits(g.standard_normal((M, K)))
    return dict(wq=wq, scales=scales, x=x)


def fused_inputs(M, N, K, workload=3, salt=0):
    """x, residual fp16 [M][K] ~N(0,1); gamma fp16 [K] ~N(1,0.1); gate/up int2 [N][K/16]
    with fp16 per-row scales ~U(0.01,0.05); eps = 1e-6."""
    g = rng(workload, M, salt)
    wq_gate = raw_words(g, (N, K // 16))
    wq_up = raw_words(g, (N, K // 16))
    s_gate = f16_bits(g.uniform(0.01, 0.05, size=N))
    s_up = f16_bits(g.uniform(0.01, 0.05, size=N))
    x = f16_bits(g.standard_normal((M, K)))
    residual = f16_bits(g.standard_normal((M, K)))
    gamma = f16_bits(g.normal(1.0, 0.1, size=K))
    return dict(x=x, residual=residual, gamma=gamma, eps=1e-6,
                wq_gate=wq_gate, s_gate=s_gate, wq_up=wq_up, s_up=s_up)


def qkv_inputs(M, Nq, Nk, Nv, K, workload=6, salt=0):
    """x, residual fp16 [M][K] ~N(0,1); gamma fp16 [K] ~N(1,0.1); q/k/v int2 [N_z][K/16]
    with fp16 per-row scales ~U(0.01,0.05); eps = 1e-6 (the fused workload's recipe with
    three output matrices)."""
    g = rng(workload, M, salt)
    out = {}
    for z, n in (("q", Nq), ("k", Nk), ("v", Nv)):
        out["wq_" + z] = raw_words(g, (n, K // 16))
        out["s_" + z] = f16_bits(g.uniform(0.01, 0.05, size=n))
    out["x"] = f16_bits(g.standard_normal((M, K)))
    out["residual"] = f16_bits(g.standard_normal((M, K)))
    out["gamma"] = f16_bits(g.normal(1.0, 0.1, size=K))
    out["eps"] = 1e-6
    return out


def argmax_inputs(M, N, K, workload=4, salt=0):
    return int2_inputs(M, N, K, workload=workload, salt=salt)


def ternary_inputs(M, N, K, workload=8, salt=0, scale_range=(0.01, 0.05)):
    """Packed ternary rows uint8 [N][ceil(K/80)*16] with every byte uniform over the 243
    base-3 codes (five independent digits, each uniform over {0,1,2}; digits past K
    drawn the same way), per-row fp16 scales, fp16 x [M][K] ~N(0,1)."""
    g = rng(workload, M, salt)
    wq = g.integers(0, 243, size=(N, (K + 79) // 80 * 16), dtype=np.uint16).astype(np.uint8)
    scale = f16_bits(g.uniform(*scale_range, size=N))
    x = f16_bits(g.standard_normal((M, K)))
    return dict(wq=wq, scale=scale, x=x)


def expert_inputs(M, E, topk, N, K, workload=7, salt=0, exp_range=(-8, 2)):
    """E experts of MXFP4 weights (the MXFP4 recipe: E2M1 nibbles uniform, E8M0 = 127 +
    U{-8..2}) [E][N][K/2] + [E][N][K/32], bf16 x [M][K] ~N(0,1), and for each row topk
    distinct expert ids drawn uniformly (int32 [M][topk])."""
    g = rng(workload, M, salt)
    wq = raw_bytes(g, (E, N, K // 2))
    e8m0 = (127 + g.integers(exp_range[0], exp_range[1] + 1, size=(E, N, K // 32))).astype(np.uint8)
    x = bf16_bits(g.standard_normal((M, K)))
    idx = np.stack([g.permutation(E)[:topk] for _ in range(M)]).astype(np.int32)
    return dict(wq=wq, e8m0=e8m0, x=x, idx=idx)


def mxfp4_inputs(M, N, K, workload=5, salt=0, exp_range=(-8, 2)):
    """E2M1 elements uint8 [N][K/2], E8M0 scales uint8 [N][K/32], bf16 x [M][K]."""
    g = rng(workload, M, salt)
    wq = raw_bytes(g, (N, K // 2))
    e8m0 = (127 + g.integers(exp_range[0], exp_range[1] + 1, size=(N, K // 32))).astype(np.uint8)
    x = bf16_bits(g.standard_normal((M, K)))
    return dict(wq=wq, e8m0=e8m0, x=x)
