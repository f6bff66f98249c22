"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle on
the same seeded host buffers.  Fixed-order mode must match bit for bit.

Workloads 1-5 run at their full sizes (the launch configuration the
benchmark times); the largest MXFP4 batch widths are compared on sampled
rows (rows are independent, so the oracle computes the sample exactly)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, bits, dev

pytestmark = pytest.mark.gpu

q = pytest.importorskip("skinny_gemm_qmv_amd")


def gpu_int2(d, y_dtype=torch.float32):
    return q.qmv_int2(dev(d["wq"], "u32"), dev(d["scale"], "f16"), dev(d["x"], "f16"), y_dtype=y_dtype)


def gpu_int4(d, y_dtype=torch.float32):
    return q.qmv_int4(dev(d["wq"], "u32"), dev(d["scales"], "f16"), dev(d["x"], "f16"), y_dtype=y_dtype)


def gpu_mxfp4(d, y_dtype=torch.float32):
    return q.qmm_mxfp4(dev(d["wq"], "u8"), dev(d["e8m0"], "u8"), dev(d["x"], "bf16"), y_dtype=y_dtype)


def orc(fmt, d):
    if fmt == "int2":
        return oracle.qmv_int2(d["wq"], d["scale"], d["x"])
    if fmt == "int4":
        return oracle.qmv_int4(d["wq"], d["scales"], d["x"])
    return oracle.qmm_mxfp4(d["wq"], d["e8m0"], d["x"])


def inputs(fmt, M, N, K, salt=0):
    if fmt == "int2":
        return synth.int2_inputs(M, N, K, salt=salt)
    if fmt == "int4":
        return synth.int4_inputs(M, N, K, salt=salt)
    return synth.mxfp4_inputs(M, N, K, salt=salt)


GPU = {"int2": gpu_int2, "int4": gpu_int4, "mxfp4": gpu_mxfp4}


def check(fmt, d, y_dtype=torch.float32):
    y = GPU[fmt](d, y_dtype)
    torch.cuda.synchronize()
    ref = orc(fmt, d)
    if y_dtype == torch.float32:
        assert_bits_equal(bits(y), ref.view(np.uint32), fmt)
    elif y_dtype == torch.float16:
        assert_bits_equal(bits(y), oracle.f32_to_f16(ref), fmt + " f16 out")
    else:
        assert_bits_equal(bits(y), oracle.f32_to_bf16(ref), fmt + " bf16 out")


# ----------------------------------------------------------- workloads ----

def test_workload1_int2_matvec():
    check("int2", synth.int2_inputs(1, 2048, 1536, workload=1))


@pytest.mark.parametrize("M", [1, 4, 8, 16])
def test_workload2_int4(M):
    check("int4", synth.int4_inputs(M, 16384, 4096, workload=2))


def test_workload3_fused_gateup():
    d = synth.fused_inputs(1, 8192, 1536, workload=3)
    res_out = torch.empty((1, 1536), dtype=torch.float16, device="cuda")
    out = q.qmv_int2_rmsnorm_gateup_gelu(
        dev(d["x"], "f16"), dev(d["residual"], "f16"), dev(d["gamma"], "f16"), d["eps"],
        dev(d["wq_gate"], "u32"), dev(d["s_gate"], "f16"), dev(d["wq_up"], "u32"),
        dev(d["s_up"], "f16"), residual_out=res_out)
    torch.cuda.synchronize()
    o, r, _, _ = oracle.int2_rmsnorm_gateup_gelu(d["x"], d["residual"], d["gamma"], d["eps"],
                                                 d["wq_gate"], d["s_gate"], d["wq_up"], d["s_up"])
    assert_bits_equal(bits(out), o, "fused out")
    assert_bits_equal(bits(res_out), r, "residual_out")


def _argmax_gpu(d, want_logits=True, ws=None):
    return q.qmv_int2_argmax(dev(d["wq"], "u32"), dev(d["scale"], "f16"), dev(d["x"], "f16"),
                             want_logits=want_logits, workspace=ws)


@pytest.mark.parametrize("M", [1, 4])
def test_workload4_lm_head_argmax(M):
    d = synth.argmax_inputs(M, 262144, 1536, workload=4)
    idx, mv, lg = _argmax_gpu(d)
    torch.cuda.synchronize()
    ri, rm, rl = oracle.int2_argmax(d["wq"], d["scale"], d["x"])
    assert_bits_equal(bits(lg), rl.view(np.uint32), "logits")
    assert np.array_equal(idx.cpu().numpy(), ri)
    assert_bits_equal(bits(mv), rm.view(np.uint32), "maxval")


@pytest.mark.parametrize("M", [1, 16])
def test_workload5_mxfp4_full(M):
    check("mxfp4", synth.mxfp4_inputs(M, 21504, 5376, workload=5))


@pytest.mark.parametrize("M", [64, 256])
def test_workload5_mxfp4_sampled_rows(M):
    d = synth.mxfp4_inputs(M, 21504, 5376, workload=5)
    y = gpu_mxfp4(d)
    torch.cuda.synchronize()
    g = np.random.default_rng(M)
    rows = np.unique(np.concatenate([[0, 1, 21503], g.choice(21504, 189, replace=False)]))
    ref = oracle.qmm_mxfp4(d["wq"][rows], d["e8m0"][rows], d["x"])
    assert_bits_equal(bits(y)[:, rows], ref.view(np.uint32), f"mxfp4 M={M} sampled rows")


# ------------------------------------------------- shapes and lane layouts ----

# K values covering every lane layout (segments per row: 1..8, ..16, ..24, ..32,
# ..64, ..96, ..128, ..192, ..256, ..512) with ragged segment counts inside buckets.
K_INT2 = [64, 320, 704, 1344, 1536, 1792, 2048, 3456, 4096, 5056, 6144, 7488, 8192, 9280, 12288, 16000, 16384]
K_32 = [32, 160, 512, 544, 768, 992, 2016, 2112, 2880, 3072, 4096, 5376, 6144, 8000, 8192, 12352, 16384]


@pytest.mark.parametrize("fmt", ["int2", "int4", "mxfp4"])
def test_every_lane_layout(fmt):
    Ks = K_INT2 if fmt == "int2" else K_32
    for i, K in enumerate(Ks):
        for M, N in ((1, 65), (3, 63), (5, 130)):
            check(fmt, inputs(fmt, M, N, K, salt=100 + i))


@pytest.mark.parametrize("fmt", ["int2", "int4", "mxfp4"])
def test_batch_widths_and_ragged_rows(fmt):
    K = 1536 if fmt == "int2" else 2048
    for M in (1, 2, 3, 4, 5, 7, 8, 15, 16, 17, 31, 32, 33, 64, 255, 256):
        for N in (1, 63, 65, 1000):
            if M * N > 40000:
                continue
            check(fmt, inputs(fmt, M, N, K, salt=M * 7 + N))


@pytest.mark.parametrize("fmt", ["int2", "int4", "mxfp4"])
def test_wide_m_large_n(fmt):
    K = 1536 if fmt == "int2" else 4096
    check(fmt, inputs(fmt, 256, 3000, K, salt=5))


@pytest.mark.parametrize("fmt", ["int2", "int4", "mxfp4"])
@pytest.mark.parametrize("y_dtype", [torch.float16, torch.bfloat16])
def test_low_precision_outputs(fmt, y_dtype):
    check(fmt, inputs(fmt, 3, 777, 1536 if fmt == "int2" else 1024, salt=9), y_dtype)


# ------------------------------------------------------------ invariance ----

@pytest.mark.parametrize("fmt", ["int2", "int4", "mxfp4"])
def test_batch_row_equals_single_row_call(fmt):
    """Row m of an M-wide call equals the M = 1 call on row m (different
    kernels: register-resident vs LDS-resident activations)."""
    K = 1536 if fmt == "int2" else 4096
    d = inputs(fmt, 6, 2000, K, salt=3)
    y = bits(GPU[fmt](d))
    for m in range(6):
        dm = dict(d)
        dm["x"] = d["x"][m:m + 1]
        assert_bits_equal(bits(GPU[fmt](dm))[0], y[m], f"{fmt} row {m}")


def test_run_to_run_determinism():
    d = synth.argmax_inputs(1, 262144, 1536, workload=4)
    wq, sc, x = dev(d["wq"], "u32"), dev(d["scale"], "f16"), dev(d["x"], "f16")
    ws = torch.empty(q.workspace_size("int2_argmax", 1, 262144, 1536), dtype=torch.uint8, device="cuda")
    q.workspace_init(ws)
    first_y = bits(q.qmv_int2(wq, sc, x))
    first_i, first_m, _ = q.qmv_int2_argmax(wq, sc, x, workspace=ws)
    first_i, first_m = first_i.cpu().numpy(), bits(first_m)
    for _ in range(100):
        assert np.array_equal(bits(q.qmv_int2(wq, sc, x)), first_y)
        i, m, _ = q.qmv_int2_argmax(wq, sc, x, workspace=ws)
        assert np.array_equal(i.cpu().numpy(), first_i) and np.array_equal(bits(m), first_m)


# ------------------------------------------------------------ edge cases ----

def test_int2_large_activations():
    """|x| near the fp16 maximum: c * x = -2 * 60000 overflows fp16 but the
    fixed order forms the product in fp32."""
    d = synth.int2_inputs(2, 513, 1536, salt=11)
    g = np.random.default_rng(1)
    d["x"] = synth.f16_bits(g.choice([-60000.0, 60000.0, 65504.0, -65504.0, 1.5], size=(2, 1536)))
    check("int2", d)


@pytest.mark.parametrize("fmt", ["int2", "int4"])
def test_subnormal_activations(fmt):
    d = inputs(fmt, 2, 300, 1536, salt=12)
    g = np.random.default_rng(2)
    d["x"] = synth.f16_bits(g.standard_normal((2, 1536)) * 2.0 ** -18)  # mostly fp16 subnormals
    check(fmt, d)


def test_mxfp4_negative_zero_codes_and_scale_extremes():
    d = synth.mxfp4_inputs(2, 257, 1024, salt=13)
    d["wq"][:, :8] = 0x88  # -0, -0
    d["e8m0"][::2, :] = 1
    d["e8m0"][1::2, :] = 254
    d["x"][:, :64] = synth.bf16_bits(np.full((2, 64), 1e-30))
    check("mxfp4", d)


def test_argmax_ties_and_zeros():
    N, K = 262144, 1536
    d = synth.argmax_inputs(1, N, K, salt=14)
    ri, _, _ = oracle.int2_argmax(d["wq"], d["scale"], d["x"])
    best = int(ri[0])
    ws = torch.empty(q.workspace_size("int2_argmax", 1, N, K), dtype=torch.uint8, device="cuda")
    q.workspace_init(ws)
    for dup in (N - 1, 0, best + 1 if best + 1 < N else best - 1):
        d2 = dict(d)
        d2["wq"] = d["wq"].copy()
        d2["scale"] = d["scale"].copy()
        d2["wq"][dup] = d["wq"][best]
        d2["scale"][dup] = d["scale"][best]
        idx, mv, _ = _argmax_gpu(d2, want_logits=False, ws=ws)
        ri2, rm2, _ = oracle.int2_argmax(d2["wq"], d2["scale"], d2["x"])
        assert int(idx.cpu()[0]) == int(ri2[0]) == min(dup, best)
        assert_bits_equal(bits(mv), rm2.view(np.uint32), "maxval")
    # all logits zero; every other row with a negative scale gives -0
    z = dict(d)
    z["wq"] = np.zeros_like(d["wq"])
    z["scale"] = synth.f16_bits(np.where(np.arange(N) % 2 == 0, -0.03, 0.03))
    idx, mv, lg = _argmax_gpu(z, ws=ws)
    ri, rm, rl = oracle.int2_argmax(z["wq"], z["scale"], z["x"])
    assert int(idx.cpu()[0]) == int(ri[0]) == 0
    assert_bits_equal(bits(mv), rm.view(np.uint32), "maxval of zeros")
    assert_bits_equal(bits(lg), rl.view(np.uint32), "zero logits")


def test_argmax_workspace_reuse_across_shapes():
    """The completion counter resets itself: consecutive calls with one
    workspace and different inputs are each correct."""
    ws = torch.empty(q.workspace_size("int2_argmax", 4, 262144, 1536), dtype=torch.uint8, device="cuda")
    q.workspace_init(ws)
    for M, N, salt in ((4, 262144, 1), (1, 5000, 2), (3, 70000, 3), (4, 262144, 4)):
        d = synth.argmax_inputs(M, N, 1536, salt=salt)
        idx, mv, _ = _argmax_gpu(d, want_logits=False, ws=ws)
        ri, rm, _ = oracle.int2_argmax(d["wq"], d["scale"], d["x"])
        assert np.array_equal(idx.cpu().numpy(), ri)
        assert_bits_equal(bits(mv), rm.view(np.uint32), "maxval")


def test_fused_shapes_and_unfused_composition():
    for M, N, K, salt in ((1, 1000, 1536, 1), (3, 517, 1536, 2), (2, 64, 4096, 3), (5, 300, 64, 4),
                          (1, 129, 16384, 5), (2, 33, 16384, 6)):
        d = synth.fused_inputs(M, N, K, salt=salt)
        res_out = torch.empty((M, K), dtype=torch.float16, device="cuda")
        out = q.qmv_int2_rmsnorm_gateup_gelu(
            dev(d["x"], "f16"), dev(d["residual"], "f16"), dev(d["gamma"], "f16"), d["eps"],
            dev(d["wq_gate"], "u32"), dev(d["s_gate"], "f16"), dev(d["wq_up"], "u32"),
            dev(d["s_up"], "f16"), residual_out=res_out)
        o, r, g, u = oracle.int2_rmsnorm_gateup_gelu(d["x"], d["residual"], d["gamma"], d["eps"],
                                                     d["wq_gate"], d["s_gate"], d["wq_up"], d["s_up"])
        assert_bits_equal(bits(out), o, f"fused M={M} N={N} K={K}")
        assert_bits_equal(bits(res_out), r, "residual_out")
        # the unfused int2 kernel on the normalised activations gives the same gate logits
        xn = np.stack([oracle.rmsnorm_prologue(d["x"][m], d["residual"][m], d["gamma"], d["eps"])[1]
                       for m in range(M)])
        yg = q.qmv_int2(dev(d["wq_gate"], "u32"), dev(d["s_gate"], "f16"), dev(xn, "f16"))
        assert_bits_equal(bits(yg), g.view(np.uint32), "unfused gate")
