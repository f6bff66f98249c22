"""Calls on a stream that is not the current one.  The workspace-using paths
(the argmax, the fused gate/up with MXFP4 quantisation, split-K) allocate and
zero their temporary workspace on the stream the kernel runs on.  The side
stream is held busy first by a bounded spin, so work issued on the current
stream instead would run ahead of the kernel it has to precede; each result
must equal the same call on the current stream bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, bits, dev

pytestmark = pytest.mark.gpu

q = pytest.importorskip("skinny_gemm_qmv_amd")

SPIN = 2_000_000  # GPU cycles (about a millisecond)


def on_side_stream(call):
    s = torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s):
            torch.cuda._sleep(SPIN)
        outs.append(call(s))
    s.synchronize()
    torch.cuda.synchronize()
    return outs


def test_argmax_on_a_side_stream():
    d = synth.argmax_inputs(2, 65536, 1536, salt=5)
    wq, sc, x = dev(d["wq"], "u32"), dev(d["scale"], "f16"), dev(d["x"], "f16")
    ri, rm, rl = q.qmv_int2_argmax(wq, sc, x, want_logits=True)
    torch.cuda.synchronize()
    for i, m, lg in on_side_stream(lambda s: q.qmv_int2_argmax(wq, sc, x, want_logits=True, stream=s)):
        assert_bits_equal(bits(i), bits(ri), "idx")
        assert_bits_equal(bits(m), bits(rm), "maxval")
        assert_bits_equal(bits(lg), bits(rl), "logits")
    oi, _, _ = oracle.int2_argmax(d["wq"], d["scale"], d["x"])
    assert np.array_equal(ri.cpu().numpy(), oi)


def test_gateup_mxfp4_on_a_side_stream():
    M, N, K = 2, 1024, 1536
    d = synth.fused_inputs(M, N, K, salt=11)
    a = (dev(d["x"], "f16"), dev(d["residual"], "f16"), dev(d["gamma"], "f16"), d["eps"],
         dev(d["wq_gate"], "u32"), dev(d["s_gate"], "f16"), dev(d["wq_up"], "u32"), dev(d["s_up"], "f16"))
    wc, we, _ = oracle.int2_rmsnorm_gateup_gelu_mxfp4(d["x"], d["residual"], d["gamma"], d["eps"], d["wq_gate"],
                                                      d["s_gate"], d["wq_up"], d["s_up"])
    for codes, e8 in on_side_stream(lambda s: q.qmv_int2_rmsnorm_gateup_gelu_mxfp4(*a, stream=s)):
        assert np.array_equal(codes.cpu().numpy(), wc)
        assert np.array_equal(e8.cpu().numpy(), we)


def test_splitk_on_a_side_stream():
    d = synth.int2_inputs(1, 2048, 1536, salt=3)
    wq, sc, x = dev(d["wq"], "u32"), dev(d["scale"], "f16"), dev(d["x"], "f16")
    ref = q.qmv_int2(wq, sc, x, mode="splitk")
    torch.cuda.synchronize()
    for y in on_side_stream(lambda s: q.qmv_int2(wq, sc, x, mode="splitk", stream=s)):
        assert_bits_equal(bits(y), bits(ref), "split-K y")
