#!/usr/bin/env python3
"""Benchmark of the quantized matvec / skinny GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one fixed-order library call (the whole hot path: activation
staging, weight stream, decode, multiply-accumulate, segment scales, the
fixed tree, epilogue) on one batch of synthetic input already resident in
HBM.  The headline workload is the largest single-GPU M=1 stream of the
workload set: the int2 lm_head N=262144, K=1536 (per-row fp16 scales, fp16
activations, 101 MB of weights) with the single-pass first-max argmax; its
metric is effective weight GB/s: algorithmic bytes (packed weights + scales
+ activations + outputs written) per call divided by the time per call.

Measurement:
  * cold weights: the calls rotate over enough copies of the weights
    (>= 1 GiB) that no call finds its weights in the 256 MB last-level cache;
    the timed calls continue the rotation where the warmup calls stopped;
  * the W warmup calls (default 500, so the clocks have settled under load)
    and the K timed calls are each captured once in a HIP
    graph (torch.cuda.CUDAGraph) and replayed, so host launch cost stays out
    of the timed region; HIP events bracket the timed replay on the stream
    the kernels run on;
  * the spread of single calls (p10 / median / p90) comes from events
    recorded between eagerly issued calls while the host runs ahead of the
    GPU (a GPU-side sleep is queued first);
  * the clean-stream ceiling (a plain 16-byte streaming read of 1 GiB and of
    the headline's own weight bytes) and the dispatch floor (empty kernels)
    are measured in the same process, from libqmv_measure.so;
  * rank 0 prints one JSON line with the roofline of the dominant kernel and
    the CPU oracle timed on the host on the same buffers, plus the oracle's
    time for every workload at T threads and at one thread.
Only the CPU-baseline legs use the oracle.
"""
import argparse
import ctypes
import hashlib
import importlib.util
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
FP32_VALU_FMA_PER_S = 78.6e12 / 2  # binary32 FMA rate without packed math (256 CU x 64 lanes x 2.4 GHz)
BF16_MFMA_PEAK = 2.5e15     # dense bf16 matrix-core rate
MXFP4_MFMA_PEAK = 10.1e15   # dense MXFP4 rate, for comparison only
COLD_BYTES = 1 << 30
PROFILES = os.path.join(ROOT, "profiles")
# the product library's sources: stored counter readings describe these
DIGEST_FILES = ("qmv_api.hip", "qmv_fo.hip", "qmv_mfma.hip", "qmv_device.hpp", "qmv_internal.hpp")

HEAD_N, HEAD_K = 262144, 1536
HEAD_LABEL = "int2 lm_head+argmax N=262144 K=1536 M=1"
HEAD_TRAFFIC = "int2_argmax_n262144_k1536_m1_traffic.json"
EXTRA_STEPS = 200  # timed calls per extra workload (the headline times exactly --steps)
# The pages' figure for the same metric on the same workload (the int2 lm_head
# matvec, K = 1536, a vocab-sized stream of about 100 MB): 40.6 GB/s effective,
# DRAM-bound, measured on another machine (Apple A19, Metal) -- context for
# vs_baseline, not a target ("Gemma4 raw-Metal loop on A19", "What moved the
# needle").
PAGES_LM_HEAD_GBS = 40.6


def effective_gbps(bytes_per_call, seconds_per_call):
    """Effective bandwidth: algorithmic bytes moved per call times calls per second."""
    return bytes_per_call / seconds_per_call / 1e9


def strip_comments(src):
    """C/C++ source text without its comments (string and character literals
    kept), every run of whitespace folded to one space."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def build_flags():
    """The product library's compile flags (the build script's FLAGS), without
    include paths, which differ between checkouts."""
    spec = importlib.util.spec_from_file_location("_qmv_build", os.path.join(ROOT, "skinny_gemm_qmv_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return [f for f in mod.FLAGS if not f.startswith("-I")]


def source_digest():
    """Digest of what the product library is built from -- its HIP sources and
    public header with comments left out, and its compile flags -- to tell
    whether stored counter readings still describe the kernels being timed."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "skinny_gemm_qmv_amd", "csrc")
    paths = [os.path.join(csrc, name) for name in DIGEST_FILES] + [os.path.join(ROOT, "include", "qmv.h")]
    for path in paths:
        with open(path, encoding="utf-8") as f:
            h.update(os.path.basename(path).encode() + strip_comments(f.read()).encode())
    h.update(" ".join(build_flags()).encode())
    return h.hexdigest()[:16]


def argmax_bytes(M, N=HEAD_N, K=HEAD_K):
    """int2 lm_head + argmax: packed weights, row scales, activations, and
    the index and maximum written per activation row."""
    return N * K // 4 + N * 2 + M * K * 2 + 8 * M


def gather_bytes(ids, E, N, K, M, topk):
    """Expert gather: the distinct experts a call reads (each once), the
    activations, the ids and the planes written."""
    eb = N * K // 2 + N * (K // 32)
    distinct = len(set(int(e) for e in ids.ravel() if 0 <= e < E))
    return distinct * eb + M * K * 2 + M * topk * 4 + M * topk * N * 4


def parse(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    # about 16 ms of load before the timed calls: on MI355X the headline's
    # time per call settles only after several ms of sustained load (200
    # calls measured 35-37 us after 20 warmup calls, 32.2 us after 500)
    p.add_argument("--warmup", type=int, default=500)
    p.add_argument("--no-extra", action="store_true", help="skip the sweep over the other workloads")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle legs")
    p.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling and dispatch floor")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="CPU time budget of the headline oracle baseline")
    p.add_argument("--cpu-config-seconds", type=float, default=0.25,
                   help="single-thread oracle time aimed at per workload in the per-workload CPU table")
    p.add_argument("--only", default="", help="run one workload by label and print its line (profiling)")
    p.add_argument("--copy-calib", action="store_true",
                   help="run a plain 256 MiB device copy (counter calibration) and exit")
    return p.parse_args(argv)


def graph_of(calls):
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls[0]()  # library/stream warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    return g


def time_graph(g):
    import torch
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3  # seconds


def dev(a, kind):
    """Host numpy buffer -> GPU tensor in the binding's conventions."""
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if kind == "u32":
        return torch.from_numpy(a.view(np.int32)).cuda()
    if kind == "f16":
        return torch.from_numpy(a.view(np.float16)).cuda()
    if kind == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def rotating(t, copies):
    return [t] + [t.clone() for _ in range(copies - 1)]


def run_case(make_call, steps, warmup, min_warm_s=0.0):
    """make_call(i) -> callable for step i.  The warmup calls are steps
    0 .. W-1 and the timed calls W .. W+K-1, so a rotation over weight copies
    continues past the warmup instead of re-reading what it just read.  With
    min_warm_s > 0 the warmup graph is replayed until that much GPU time has
    passed (each replay ends at step W-1, so the rotation still continues
    into the timed calls): the clocks settle only after several ms of load.
    Returns seconds per timed call."""
    wg = graph_of([make_call(i) for i in range(warmup)]) if warmup > 0 else None
    tg = graph_of([make_call(warmup + i) for i in range(steps)])
    if wg is not None:
        warm = time_graph(wg)
        while warm < min_warm_s:
            warm += time_graph(wg)
    return time_graph(tg) / steps


def per_call_spread(make_call, n, first):
    """p10 / median / p90 of single calls (microseconds): events recorded
    between calls issued eagerly while the GPU works through a queued sleep,
    so the host is ahead and the calls run back to back."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    calls = [make_call(first + i) for i in range(n)]
    torch.cuda.synchronize()
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(100_000_000)  # ~40 ms of GPU time while the host queues
    evs[0].record()
    for i, c in enumerate(calls):
        c()
        evs[i + 1].record()
    torch.cuda.synchronize()
    d = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n))
    return {"p10": round(d[n // 10], 3), "p50": round(d[n // 2], 3), "p90": round(d[(9 * n) // 10], 3),
            "calls": n}


def argmax_case(M, cold=True):
    import torch
    import skinny_gemm_qmv_amd as q
    import synth
    N, K = HEAD_N, HEAD_K
    d = synth.argmax_inputs(M, N, K, workload=4)
    wb = N * K // 4 + N * 2
    copies = max(1, -(-COLD_BYTES // wb)) if cold else 1
    wq = rotating(dev(d["wq"], "u32"), copies)
    sc = rotating(dev(d["scale"], "f16"), copies)
    x = dev(d["x"], "f16")
    idx = torch.empty(M, dtype=torch.int32, device="cuda")
    mv = torch.empty(M, dtype=torch.float32, device="cuda")
    ws = torch.empty(q.workspace_size("int2_argmax", M, N, K), dtype=torch.uint8, device="cuda")
    q.workspace_init(ws)

    def make(i):
        return lambda: q.qmv_int2_argmax(wq[i % copies], sc[i % copies], x, idx=idx, maxval=mv, workspace=ws)
    return make, argmax_bytes(M), d, copies, wq


def int4_case(M, cold=True):
    import torch
    import skinny_gemm_qmv_amd as q
    import synth
    N, K = 16384, 4096
    d = synth.int4_inputs(M, N, K, workload=2)
    wbytes = N * K // 2 + N * (K // 32) * 2
    copies = max(1, -(-COLD_BYTES // wbytes)) if cold else 1
    wq = rotating(dev(d["wq"], "u32"), copies)
    sc = rotating(dev(d["scales"], "f16"), copies)
    x = dev(d["x"], "f16")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nbytes = wbytes + M * K * 2 + M * N * 4
    return (lambda i: (lambda: q.qmv_int4(wq[i % copies], sc[i % copies], x, y=y))), nbytes, d, copies


def sweep_cases():
    """(label, builder) for the other workloads; builder() -> (make_call, bytes, flops, bound)."""
    import numpy as np
    import torch
    import skinny_gemm_qmv_amd as q
    import synth

    def int2_c1(mode="fixed"):
        def b():
            d = synth.int2_inputs(1, 2048, 1536, workload=1)
            wb = 2048 * 1536 // 4 + 2048 * 2
            cp = -(-COLD_BYTES // wb)
            wq, sc = rotating(dev(d["wq"], "u32"), cp), rotating(dev(d["scale"], "f16"), cp)
            x = dev(d["x"], "f16")
            y = torch.empty((1, 2048), device="cuda")
            need = q.workspace_size("int2", 1, 2048, 1536, mode)
            ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
            return (lambda i: (lambda: q.qmv_int2(wq[i % cp], sc[i % cp], x, y=y, mode=mode, workspace=ws))), \
                wb + 3072 + 8192, 2 * 2048 * 1536, "hbm"
        return b

    def int4_m(M):
        def b():
            mk, nb, _, _ = int4_case(M)
            fl = 2 * M * 16384 * 4096
            return mk, nb, fl, "hbm" if M == 1 else "alu"
        return b

    def int4_hot():
        mk, nb, _, _ = int4_case(1, cold=False)
        return mk, nb, 2 * 16384 * 4096, "hbm"

    def fused_c3():
        d = synth.fused_inputs(1, 8192, 1536, workload=3)
        wb = 2 * (8192 * 1536 // 4 + 8192 * 2)
        cp = -(-COLD_BYTES // wb)
        wg, sg = rotating(dev(d["wq_gate"], "u32"), cp), rotating(dev(d["s_gate"], "f16"), cp)
        wu, su = rotating(dev(d["wq_up"], "u32"), cp), rotating(dev(d["s_up"], "f16"), cp)
        x, r, gm = dev(d["x"], "f16"), dev(d["residual"], "f16"), dev(d["gamma"], "f16")
        out = torch.empty((1, 8192), dtype=torch.float16, device="cuda")
        ro = torch.empty((1, 1536), dtype=torch.float16, device="cuda")
        nb = wb + 3 * 1536 * 2 + 1536 * 2 + 8192 * 2
        return (lambda i: (lambda: q.qmv_int2_rmsnorm_gateup_gelu(
            x, r, gm, 1e-6, wg[i % cp], sg[i % cp], wu[i % cp], su[i % cp], out=out,
            residual_out=ro))), nb, 2 * 2 * 8192 * 1536, "hbm"

    def fused_quant_f4():
        # the fused workload with its output quantised to MXFP4 in the same
        # dispatch (codes + E8M0 instead of fp16)
        d = synth.fused_inputs(1, 8192, 1536, workload=3)
        wb = 2 * (8192 * 1536 // 4 + 8192 * 2)
        cp = -(-COLD_BYTES // wb)
        wg, sg = rotating(dev(d["wq_gate"], "u32"), cp), rotating(dev(d["s_gate"], "f16"), cp)
        wu, su = rotating(dev(d["wq_up"], "u32"), cp), rotating(dev(d["s_up"], "f16"), cp)
        x, r, gm = dev(d["x"], "f16"), dev(d["residual"], "f16"), dev(d["gamma"], "f16")
        codes = torch.empty((1, 4096), dtype=torch.uint8, device="cuda")
        e8 = torch.empty((1, 256), dtype=torch.uint8, device="cuda")
        ro = torch.empty((1, 1536), dtype=torch.float16, device="cuda")
        ws = torch.empty(q.workspace_size("int2_gateup_mxfp4", 1, 8192, 1536), dtype=torch.uint8, device="cuda")
        q.workspace_init(ws)
        nb = wb + 3 * 1536 * 2 + 1536 * 2 + 4096 + 256
        return (lambda i: (lambda: q.qmv_int2_rmsnorm_gateup_gelu_mxfp4(
            x, r, gm, 1e-6, wg[i % cp], sg[i % cp], wu[i % cp], su[i % cp], codes=codes, e8m0=e8,
            residual_out=ro, workspace=ws))), nb, 2 * 2 * 8192 * 1536, "hbm"

    def qkv_f1():
        # q/k/v shapes of a K=1536 decoder layer: 8 query heads and 2 key/value
        # heads of 256 (synthetic int2 weights, the fused workload's recipe)
        Nq, Nk, Nv, K = 2048, 512, 512, 1536
        d = synth.qkv_inputs(1, Nq, Nk, Nv, K)
        wb = (Nq + Nk + Nv) * (K // 4 + 2)
        cp = -(-COLD_BYTES // wb)
        ws = {z: rotating(dev(d["wq_" + z], "u32"), cp) for z in "qkv"}
        ss = {z: rotating(dev(d["s_" + z], "f16"), cp) for z in "qkv"}
        x, r, gm = dev(d["x"], "f16"), dev(d["residual"], "f16"), dev(d["gamma"], "f16")
        ys = [torch.empty((1, n), device="cuda") for n in (Nq, Nk, Nv)]
        ro = torch.empty((1, K), dtype=torch.float16, device="cuda")
        nb = wb + 3 * K * 2 + K * 2 + (Nq + Nk + Nv) * 4
        return (lambda i: (lambda: q.qmv_int2_rmsnorm_qkv(
            x, r, gm, 1e-6, ws["q"][i % cp], ss["q"][i % cp], ws["k"][i % cp], ss["k"][i % cp],
            ws["v"][i % cp], ss["v"][i % cp], y_q=ys[0], y_k=ys[1], y_v=ys[2], residual_out=ro))), \
            nb, 2 * (Nq + Nk + Nv) * K, "hbm"

    def gather_f2(M):
        # a gpt-oss-sized MoE projection: 32 MXFP4 experts of N=5760, K=2880,
        # each activation row routed to 4 of them; every step picks other
        # experts (a fresh id draw) from enough copies of the expert array that
        # the weights are read cold.  Bytes count each distinct expert of a
        # call once (repeats within a call are served by the caches).
        def b():
            E, topk, N, K = 32, 4, 5760, 2880
            d = synth.expert_inputs(M, E, topk, N, K)
            eb = N * K // 2 + N * (K // 32)
            cp = -(-COLD_BYTES // (E * eb))
            wq, e = rotating(dev(d["wq"], "u8"), cp), rotating(dev(d["e8m0"], "u8"), cp)
            x = dev(d["x"], "bf16")
            g = synth.rng(7, M, 1)
            draws = [np.stack([g.permutation(E)[:topk] for _ in range(M)]).astype(np.int32) for _ in range(8)]
            ids = [torch.from_numpy(a).cuda() for a in draws]
            nb = statistics.mean(gather_bytes(a, E, N, K, M, topk) for a in draws)
            y = torch.empty((M, topk, N), device="cuda")
            return (lambda i: (lambda: q.qmm_mxfp4_gather(wq[i % cp], e[i % cp], x, ids[i % 8], y=y))), \
                nb, 2 * M * topk * N * K, "hbm"
        return b

    def ternary_m(M):
        # an 8B-class decoder projection with ternary weights (five base-3
        # digits per byte, rows of 52 segments of 80 codes)
        def b():
            N, K = 16384, 4096
            d = synth.ternary_inputs(M, N, K, workload=8)
            wb = N * ((K + 79) // 80 * 16) + N * 2
            cp = -(-COLD_BYTES // wb)
            wq, sc = rotating(dev(d["wq"], "u8"), cp), rotating(dev(d["scale"], "f16"), cp)
            x = dev(d["x"], "f16")
            y = torch.empty((M, N), device="cuda")
            return (lambda i: (lambda: q.qmv_ternary(wq[i % cp], sc[i % cp], x, y=y))), \
                wb + M * K * 2 + M * N * 4, 2 * M * N * K, "hbm"
        return b

    def argmax_c4(M, cold=True):
        def b():
            mk, nb, _, _, _ = argmax_case(M, cold)
            return mk, nb, 2 * M * HEAD_N * HEAD_K, "hbm" if M == 1 else "alu"
        return b

    def mxfp4_m(M, mode="fixed"):
        def b():
            d = synth.mxfp4_inputs(M, 21504, 5376, workload=5)
            wb = 21504 * 5376 // 2 + 21504 * 168
            cp = -(-COLD_BYTES // wb)
            wq, e = rotating(dev(d["wq"], "u8"), cp), rotating(dev(d["e8m0"], "u8"), cp)
            x = dev(d["x"], "bf16")
            y = torch.empty((M, 21504), device="cuda")
            if mode == "mfma":
                # the bf16 matrix-core rate binds once the arithmetic intensity
                # (2M flops per 0.53 weight bytes) passes its ridge (~312 flop/B)
                bound = "hbm" if M <= 64 else "mfma"
            else:
                bound = "hbm" if M == 1 else "alu"
            return (lambda i: (lambda: q.qmm_mxfp4(wq[i % cp], e[i % cp], x, y=y, mode=mode))), \
                wb + M * 5376 * 2 + M * 21504 * 4, 2 * M * 21504 * 5376, bound
        return b

    return [
        ("int2 lm_head+argmax N=262144 K=1536 M=1 hot (one weight copy, cache-resident)", argmax_c4(1, False)),
        ("int2 lm_head+argmax N=262144 K=1536 M=4", argmax_c4(4)),
        ("int4 N=16384 K=4096 M=1", int4_m(1)),
        ("int4 N=16384 K=4096 M=1 hot (one weight copy, cache-resident)", int4_hot),
        ("int4 N=16384 K=4096 M=4", int4_m(4)),
        ("int4 N=16384 K=4096 M=8", int4_m(8)),
        ("int4 N=16384 K=4096 M=16", int4_m(16)),
        ("int2 N=2048 K=1536 M=1", int2_c1()),
        ("int2 N=2048 K=1536 M=1 split-K", int2_c1("splitk")),
        ("fused rmsnorm+int2 gate/up+gelu N=2x8192 K=1536 M=1", fused_c3),
        ("fused rmsnorm+int2 gate/up+gelu+mxfp4 quantise N=2x8192 K=1536 M=1", fused_quant_f4),
        ("fused rmsnorm+int2 q/k/v N=2048+512+512 K=1536 M=1", qkv_f1),
        ("mxfp4 expert gather E=32 top-4 N=5760 K=2880 M=1", gather_f2(1)),
        ("mxfp4 expert gather E=32 top-4 N=5760 K=2880 M=16", gather_f2(16)),
        ("ternary N=16384 K=4096 M=1", ternary_m(1)),
        ("mxfp4 N=21504 K=5376 M=1", mxfp4_m(1)),
        ("mxfp4 N=21504 K=5376 M=16", mxfp4_m(16)),
        ("mxfp4 N=21504 K=5376 M=64", mxfp4_m(64)),
        ("mxfp4 N=21504 K=5376 M=256", mxfp4_m(256)),
        ("mxfp4 N=21504 K=5376 M=64 matrix cores", mxfp4_m(64, "mfma")),
        ("mxfp4 N=21504 K=5376 M=256 matrix cores", mxfp4_m(256, "mfma")),
    ]


def roof_fraction(bound, nbytes, flops, sec):
    gbs = effective_gbps(nbytes, sec)
    if bound == "hbm":
        return gbs / HBM_PEAK_GBS
    if bound == "mfma":
        return flops / sec / BF16_MFMA_PEAK
    # fixed-order arithmetic: one binary32 FMA per (code, activation column)
    return (flops / 2 / sec) / FP32_VALU_FMA_PER_S


def stored_traffic(label_file, digest):
    path = os.path.join(PROFILES, label_file)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


def _measure_lib():
    path = os.path.join(ROOT, "skinny_gemm_qmv_amd", "libqmv_measure.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.qmv_measure_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                            ctypes.c_void_p]
    lib.qmv_measure_stream_read.restype = ctypes.c_int
    lib.qmv_measure_empty.argtypes = [ctypes.c_void_p]
    lib.qmv_measure_empty.restype = ctypes.c_int
    return lib


def ceilings(head_copies, steps):
    """The clean-stream ceiling and the dispatch floor on this GPU: a plain
    16-byte streaming read of 1 GiB (four rotating buffers, cold) and of the
    headline's own weight bytes (rotating over its copies), and back-to-back
    empty kernels, each replayed from a graph."""
    import torch
    lib = _measure_lib()
    if lib is None:
        return None
    sink = torch.empty(8192, dtype=torch.int32, device="cuda")

    def st():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def read(t, nbytes):
        def c():
            if lib.qmv_measure_stream_read(ctypes.c_void_p(t.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                           0, st()) != 0:
                raise RuntimeError("qmv_measure_stream_read failed")
        return c

    out = {"command": "python3 bench.py (ceiling leg, libqmv_measure.so)"}
    big = [torch.empty(COLD_BYTES, dtype=torch.uint8, device="cuda") for _ in range(4)]
    for b in big:
        b.fill_(1)
    s = run_case(lambda i: read(big[i % 4], COLD_BYTES), 8, 4)
    out["stream_read_1GiB_GBs"] = round(effective_gbps(COLD_BYTES, s), 1)
    del big
    torch.cuda.empty_cache()
    hb = head_copies[0].numel() * 4
    s = run_case(lambda i: read(head_copies[i % len(head_copies)], hb), max(20, steps // 4), 5)
    out["stream_read_headline_bytes_GBs"] = round(effective_gbps(hb, s), 1)
    out["stream_read_headline_bytes_us"] = round(s * 1e6, 3)

    def empty():
        if lib.qmv_measure_empty(st()) != 0:
            raise RuntimeError("qmv_measure_empty failed")
    s = run_case(lambda i: empty, 200, 20)
    out["dispatch_floor_us"] = round(s * 1e6, 3)
    return out


def cpu_baseline(d, seconds):
    """The oracle's lm_head + argmax on the same host buffers: median call
    time over as many full calls as fit the budget (at least three)."""
    import oracle
    threads = oracle.default_threads()
    times = []
    t_end = time.perf_counter() + seconds
    while True:
        t0 = time.perf_counter()
        oracle.int2_argmax(d["wq"], d["scale"], d["x"], threads=threads)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() > t_end and len(times) >= 3:
            break
    return statistics.median(times), threads, len(times)


def cpu_per_config(target_seconds):
    """The oracle per workload at T threads and at one thread, as in the
    baseline plan: each timed on the first R rows of the workload's own host
    buffers (R sized so one single-thread call takes about target_seconds;
    rows are independent, so the time scales with R), median of three calls
    after one warm-up, reported per full call."""
    import oracle
    import synth
    T = oracle.default_threads()

    def med(fn, reps=3):
        fn()
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return statistics.median(ts)

    def sized(per_rows, N):
        # per_rows(r, threads) runs the oracle on the first r rows
        r0 = min(N, 256)
        t0 = time.perf_counter()
        per_rows(r0, 1)
        t_row = max((time.perf_counter() - t0) / r0, 1e-9)
        r = int(min(N, max(r0, target_seconds / t_row)))
        r = max(r, min(N, 4 * T))
        t1 = med(lambda: per_rows(r, 1))
        tT = med(lambda: per_rows(r, T))
        return r, t1 * N / r, tT * N / r

    rows = []

    def add(label, nbytes, per_rows, N, flops=None):
        r, t1, tT = sized(per_rows, N)
        rec = {"workload": label, "rows_timed": r, "rows": N,
               "us_per_call_1_thread": round(t1 * 1e6, 1), "us_per_call_T_threads": round(tT * 1e6, 1),
               "GB/s_T_threads": round(effective_gbps(nbytes, tT), 3)}
        if flops is not None:
            rec["TFLOP/s_T_threads"] = round(flops / tT / 1e12, 5)
        rows.append(rec)

    d = synth.int2_inputs(1, 2048, 1536, workload=1)
    add("int2 N=2048 K=1536 M=1", 2048 * 386 + 3072 + 8192,
        lambda r, t: oracle.qmv_int2(d["wq"][:r], d["scale"][:r], d["x"], threads=t), 2048)
    for M in (1, 4, 8, 16):
        d4 = synth.int4_inputs(M, 16384, 4096, workload=2)
        add(f"int4 N=16384 K=4096 M={M}", 16384 * 2304 + M * 8192 + M * 65536,
            lambda r, t, d4=d4: oracle.qmv_int4(d4["wq"][:r], d4["scales"][:r], d4["x"], threads=t), 16384)
    d3 = synth.fused_inputs(1, 8192, 1536, workload=3)
    add("fused rmsnorm+int2 gate/up+gelu N=2x8192 K=1536 M=1", 2 * 8192 * 386 + 12288 + 16384,
        lambda r, t: oracle.int2_rmsnorm_gateup_gelu(d3["x"], d3["residual"], d3["gamma"], d3["eps"],
                                                     d3["wq_gate"][:r], d3["s_gate"][:r], d3["wq_up"][:r],
                                                     d3["s_up"][:r], threads=t), 8192)
    for M in (1, 4):
        da = synth.argmax_inputs(M, HEAD_N, HEAD_K, workload=4)
        add(f"int2 lm_head+argmax N=262144 K=1536 M={M}", argmax_bytes(M),
            lambda r, t, da=da: oracle.int2_argmax(da["wq"][:r], da["scale"][:r], da["x"], threads=t), HEAD_N)
    for M in (1, 16, 64, 256):
        d5 = synth.mxfp4_inputs(M, 21504, 5376, workload=5)
        add(f"mxfp4 N=21504 K=5376 M={M}", 21504 * 2856 + M * 10752 + M * 86016,
            lambda r, t, d5=d5: oracle.qmm_mxfp4(d5["wq"][:r], d5["e8m0"][:r], d5["x"], threads=t), 21504,
            flops=2 * M * 21504 * 5376 if M >= 64 else None)
        del d5
    return {"threads": T, "host_cpus_visible": os.cpu_count(), "rows": rows}


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)

    if args.copy_calib:
        src = torch.empty(1 << 28, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 28, "launches": 5}))
        return

    if args.only:
        if args.only == HEAD_LABEL:
            mk, nb, _, _, _ = argmax_case(1)
        else:
            found = [b for label, b in sweep_cases() if label == args.only]
            if not found:
                print(f"unknown --only label {args.only!r}", file=sys.stderr)
                sys.exit(2)
            mk, nb, _, _ = found[0]()
        sec = run_case(mk, args.steps, args.warmup)
        print(json.dumps({"label": args.only, "us": sec * 1e6, "GB/s": effective_gbps(nb, sec)}), flush=True)
        return

    make_call, nbytes, d, copies, head_wq = argmax_case(1)
    sec = run_case(make_call, args.steps, args.warmup)
    gbs = effective_gbps(nbytes, sec)
    spread = per_call_spread(make_call, max(50, min(400, args.steps)), args.warmup + args.steps)
    digest = source_digest()
    traffic = stored_traffic(HEAD_TRAFFIC, digest)

    ceil = None if args.no_ceiling else ceilings(head_wq, args.steps)
    del head_wq

    extra = []
    if not args.no_extra:
        for label, b in sweep_cases():
            mk, nb, fl, bound = b()
            # at least EXTRA_STEPS calls per timed graph, so that the graph
            # launch does not inflate the latency-floor kernels (a few us each)
            # the inputs are generated on the host first, so the GPU has idled:
            # warm up for at least 20 ms of load
            s = run_case(mk, max(EXTRA_STEPS, args.steps // 10), max(5, args.warmup // 4), min_warm_s=0.02)
            rec = {"workload": label, "us_per_call": round(s * 1e6, 3),
                   "GB/s": round(effective_gbps(nb, s), 1),
                   "TFLOP/s": round(fl / s / 1e12, 3), "bound": bound,
                   "roofline_frac": round(roof_fraction(bound, nb, fl, s), 4)}
            if "matrix cores" in label:
                rec["frac_of_bf16_mfma_peak"] = round(fl / s / BF16_MFMA_PEAK, 4)
                rec["frac_of_mxfp4_mfma_peak"] = round(fl / s / MXFP4_MFMA_PEAK, 4)
            extra.append(rec)
            del mk
            torch.cuda.empty_cache()

    cpu = None
    cpu_table = None
    if not args.no_cpu:
        med, threads, reps = cpu_baseline(d, args.cpu_seconds)
        cpu = {"value": round(effective_gbps(nbytes, med), 3), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"full int2 lm_head+argmax N=262144 K=1536 M=1 call on the same host buffers, median "
                         f"of {reps} calls ({med * 1e3:.1f} ms each), {threads} threads, {os.cpu_count()} host "
                         f"CPUs visible"}
        cpu_table = cpu_per_config(args.cpu_config_seconds)

    line = {
        "metric": "effective weight GB/s per qmv call at M=1 (int2 lm_head + argmax, N=262144 K=1536)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(gbs / PAGES_LM_HEAD_GBS, 2),
        "baseline": {"value": PAGES_LM_HEAD_GBS, "unit": "GB/s", "hardware": "Apple A19 (Metal)",
                     "workload": "int2 lm_head matvec, K=1536, vocab-sized (~100 MB) stream, M=1",
                     "note": "the pages' figure on another machine: context, not a target"},
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "int2 lm_head matvec N=262144, K=1536 (per-row fp16 scales, fp16 x) + single-pass "
                               "first-max argmax, M=1, fixed order, cold weights",
                   "M": 1, "N": HEAD_N, "K": HEAD_K, "weight_copies": copies,
                   "bytes_per_call": nbytes, "source_digest": digest},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic},
        "per_call_us": spread,
        "ceiling": ceil,
        "cpu_baseline": cpu,
        "cpu_per_workload": cpu_table,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
