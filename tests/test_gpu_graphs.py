"""GPU: the entry points captured into a HIP graph and replayed.

The benchmark times graph replays, and callers may capture these calls, so
every replay must give the eager result bit for bit — including the entry
points that keep state in their workspace between calls (the argmax keys and
completion counter, the per-block counters of the quantising gate/up), which
must come back to zero after each replay.  Each replay is followed by eager
work and a synchronisation before its outputs are compared."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import bits, dev

pytestmark = pytest.mark.gpu

q = pytest.importorskip("skinny_gemm_qmv_amd")


def capture(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    return g


def replay_and_check(g, outputs, want, noise):
    for rep in range(4):
        for o in outputs:
            o.fill_(0x55 if o.dtype == torch.uint8 else 7)  # eager work between replays
        g.replay()
        noise()
        torch.cuda.synchronize()
        for o, w in zip(outputs, want):
            assert np.array_equal(bits(o), w), f"replay {rep}"


def test_graph_int4_argmax_and_gather():
    d4 = synth.int4_inputs(1, 4096, 4096, workload=2, salt=1)
    wq4, sc4, x4 = dev(d4["wq"], "u32"), dev(d4["scales"], "f16"), dev(d4["x"], "f16")
    y4 = torch.empty((1, 4096), device="cuda")
    da = synth.argmax_inputs(2, 65536, 1536, salt=2)
    wqa, sca, xa = dev(da["wq"], "u32"), dev(da["scale"], "f16"), dev(da["x"], "f16")
    idx = torch.empty(2, dtype=torch.int32, device="cuda")
    mv = torch.empty(2, dtype=torch.float32, device="cuda")
    ws = torch.empty(q.workspace_size("int2_argmax", 2, 65536, 1536), dtype=torch.uint8, device="cuda")
    q.workspace_init(ws)
    dg = synth.expert_inputs(1, 8, 4, 640, 2880, salt=3)
    wg, eg, xg = dev(dg["wq"], "u8"), dev(dg["e8m0"], "u8"), dev(dg["x"], "bf16")
    ids = torch.from_numpy(dg["idx"]).cuda()
    yg = torch.empty((1, 4, 640), device="cuda")

    def calls():
        q.qmv_int4(wq4, sc4, x4, y=y4)
        q.qmv_int2_argmax(wqa, sca, xa, idx=idx, maxval=mv, workspace=ws)
        q.qmm_mxfp4_gather(wg, eg, xg, ids, y=yg)

    calls()
    torch.cuda.synchronize()
    outs = [y4, idx, mv, yg]
    want = [bits(o) for o in outs]
    g = capture(calls)
    replay_and_check(g, outs, want, lambda: torch.ones(1 << 20, device="cuda").sum())
    assert int(ws.count_nonzero()) == 0


def test_graph_fused_quantise():
    d = synth.fused_inputs(1, 2048, 1536, salt=4)
    a = (dev(d["x"], "f16"), dev(d["residual"], "f16"), dev(d["gamma"], "f16"), d["eps"],
         dev(d["wq_gate"], "u32"), dev(d["s_gate"], "f16"), dev(d["wq_up"], "u32"), dev(d["s_up"], "f16"))
    codes = torch.empty((1, 1024), dtype=torch.uint8, device="cuda")
    e8 = torch.empty((1, 64), dtype=torch.uint8, device="cuda")
    for K in (1536,):
        ws = torch.empty(q.workspace_size("int2_gateup_mxfp4", 1, 2048, K), dtype=torch.uint8, device="cuda")
        q.workspace_init(ws)

        def calls():
            q.qmv_int2_rmsnorm_gateup_gelu_mxfp4(*a, codes=codes, e8m0=e8, workspace=ws)

        calls()
        torch.cuda.synchronize()
        want = [bits(codes), bits(e8)]
        g = capture(calls)
        replay_and_check(g, [codes, e8], want, lambda: torch.ones(1 << 20, device="cuda").sum())
        cnt = (2048 // 32 * 4 + 255) // 256 * 256
        assert int(ws[:cnt].count_nonzero()) == 0


def test_graph_fused_quantise_counter_fallback():
    # 128 segments per row: the arrival-counter path
    d = synth.fused_inputs(1, 256, 8192, salt=5)
    a = (dev(d["x"], "f16"), dev(d["residual"], "f16"), dev(d["gamma"], "f16"), d["eps"],
         dev(d["wq_gate"], "u32"), dev(d["s_gate"], "f16"), dev(d["wq_up"], "u32"), dev(d["s_up"], "f16"))
    codes = torch.empty((1, 128), dtype=torch.uint8, device="cuda")
    e8 = torch.empty((1, 8), dtype=torch.uint8, device="cuda")
    ws = torch.empty(q.workspace_size("int2_gateup_mxfp4", 1, 256, 8192), dtype=torch.uint8, device="cuda")
    q.workspace_init(ws)

    def calls():
        q.qmv_int2_rmsnorm_gateup_gelu_mxfp4(*a, codes=codes, e8m0=e8, workspace=ws)

    calls()
    torch.cuda.synchronize()
    want = [bits(codes), bits(e8)]
    g = capture(calls)
    replay_and_check(g, [codes, e8], want, lambda: torch.ones(1 << 20, device="cuda").sum())
    assert int(ws[:256].count_nonzero()) == 0
