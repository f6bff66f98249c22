#!/usr/bin/env python3
"""Benchmark of the quantized matvec / skinny GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one fixed-order library call (the whole hot path: activation
staging, weight stream, decode, multiply-accumulate, segment scales, the
fixed tree, epilogue) on one batch of synthetic input already resident in
HBM.  The headline workload is the int4 skinny GEMM N=16384, K=4096 (group-32
fp16 scales, fp16 activations) at M=1; its metric is effective weight GB/s:
algorithmic bytes (packed weights + scales + activations + outputs written)
per call divided by the time per call.

Measurement:
  * cold weights: the K timed calls rotate over enough copies of the weights
    (>= 1 GiB) that no call finds its weights in the 256 MB last-level cache;
  * the W warmup calls and the K timed calls are each captured once in a HIP
    graph (torch.cuda.CUDAGraph) and replayed, so host launch cost stays out
    of the timed region; HIP events bracket the timed replay on the stream
    the kernels run on;
  * rank 0 prints one JSON line with the roofline of the dominant kernel and
    the CPU oracle timed on the host on the same buffers.
Only the CPU-baseline leg uses the oracle.
"""
import argparse
import hashlib
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


def effective_gbps(bytes_per_call, seconds_per_call):
    """Effective bandwidth: algorithmic bytes moved per call times calls per second."""
    return bytes_per_call / seconds_per_call / 1e9


def source_digest():
    """Digest of the HIP sources, to tell whether stored counter readings
    still describe the kernels being timed."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "skinny_gemm_qmv_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--no-extra", action="store_true", help="skip the sweep over the other workloads")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--only", default="", help="run one sweep entry by label (profiling)")
    p.add_argument("--copy-calib", action="store_true",
                   help="run a plain 256 MiB device copy (counter calibration) and exit")
    return p.parse_args()


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


def run_case(make_call, steps, warmup):
    """make_call(i) -> callable for step i.  Returns seconds per call."""
    wg = graph_of([make_call(i) for i in range(warmup)]) if warmup > 0 else None
    tg = graph_of([make_call(i) for i in range(steps)])
    if wg is not None:
        time_graph(wg)
    return time_graph(tg) / steps


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
        # the weights are read cold
        def b():
            E, topk, N, K = 32, 4, 5760, 2880
            d = synth.expert_inputs(M, E, topk, N, K)
            eb = N * K // 2 + N * (K // 32)
            cp = -(-COLD_BYTES // (E * eb))
            wq, e = rotating(dev(d["wq"], "u8"), cp), rotating(dev(d["e8m0"], "u8"), cp)
            x = dev(d["x"], "bf16")
            g = synth.rng(7, M, 1)
            ids = [torch.from_numpy(np.stack([g.permutation(E)[:topk] for _ in range(M)]).astype(np.int32)).cuda()
                   for _ in range(8)]
            y = torch.empty((M, topk, N), device="cuda")
            return (lambda i: (lambda: q.qmm_mxfp4_gather(wq[i % cp], e[i % cp], x, ids[i % 8], y=y))), \
                M * topk * eb + M * K * 2 + M * topk * 4 + M * topk * N * 4, 2 * M * topk * N * K, "hbm"
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

    def argmax_c4(M):
        def b():
            d = synth.argmax_inputs(M, 262144, 1536, workload=4)
            wb = 262144 * 1536 // 4 + 262144 * 2
            cp = -(-COLD_BYTES // wb)
            wq, sc = rotating(dev(d["wq"], "u32"), cp), rotating(dev(d["scale"], "f16"), cp)
            x = dev(d["x"], "f16")
            idx = torch.empty(M, dtype=torch.int32, device="cuda")
            mv = torch.empty(M, dtype=torch.float32, device="cuda")
            ws = torch.empty(q.workspace_size("int2_argmax", M, 262144, 1536), dtype=torch.uint8, device="cuda")
            q.workspace_init(ws)
            return (lambda i: (lambda: q.qmv_int2_argmax(wq[i % cp], sc[i % cp], x, idx=idx, maxval=mv,
                                                         workspace=ws))), wb + M * 3072 + 8 * M, \
                2 * M * 262144 * 1536, "hbm" if M == 1 else "alu"
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
        ("int2 N=2048 K=1536 M=1", int2_c1()),
        ("int2 N=2048 K=1536 M=1 split-K", int2_c1("splitk")),
        ("int4 N=16384 K=4096 M=4", int4_m(4)),
        ("int4 N=16384 K=4096 M=8", int4_m(8)),
        ("int4 N=16384 K=4096 M=16", int4_m(16)),
        ("fused rmsnorm+int2 gate/up+gelu N=2x8192 K=1536 M=1", fused_c3),
        ("fused rmsnorm+int2 gate/up+gelu+mxfp4 quantise N=2x8192 K=1536 M=1", fused_quant_f4),
        ("fused rmsnorm+int2 q/k/v N=2048+512+512 K=1536 M=1", qkv_f1),
        ("mxfp4 expert gather E=32 top-4 N=5760 K=2880 M=1", gather_f2(1)),
        ("mxfp4 expert gather E=32 top-4 N=5760 K=2880 M=16", gather_f2(16)),
        ("ternary N=16384 K=4096 M=1", ternary_m(1)),
        ("int2 lm_head+argmax N=262144 K=1536 M=1", argmax_c4(1)),
        ("int2 lm_head+argmax N=262144 K=1536 M=4", argmax_c4(4)),
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


def cpu_baseline(d, seconds):
    import oracle
    threads = oracle.default_threads()
    times = []
    t_end = time.perf_counter() + seconds
    while True:
        t0 = time.perf_counter()
        oracle.qmv_int4(d["wq"], d["scales"], d["x"], threads=threads)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() > t_end and len(times) >= 3:
            break
    return statistics.median(times), threads, len(times)


def main():
    args = parse()
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
        for label, b in sweep_cases():
            if label == args.only:
                mk, nb, fl, bound = b()
                sec = run_case(mk, args.steps, args.warmup)
                print(json.dumps({"label": label, "us": sec * 1e6, "GB/s": effective_gbps(nb, sec)}))
                return
        if args.only != "int4 M=1":
            print(f"unknown --only label {args.only!r}", file=sys.stderr)
            sys.exit(2)
        mk, nb, d, copies = int4_case(1)
        sec = run_case(mk, args.steps, args.warmup)
        print(json.dumps({"label": "int4 M=1", "us": sec * 1e6, "GB/s": effective_gbps(nb, sec)}))
        return

    make_call, nbytes, d, copies = int4_case(1)
    sec = run_case(make_call, args.steps, args.warmup)
    gbs = effective_gbps(nbytes, sec)
    digest = source_digest()
    traffic = stored_traffic("int4_n16384_k4096_m1_traffic.json", digest)

    extra = []
    if not args.no_extra:
        # the headline call hot: one weight copy, re-read from the caches
        mk, nb, _, _ = int4_case(1, cold=False)
        s = run_case(mk, max(20, args.steps // 10), max(5, args.warmup // 10))
        extra.append({"workload": "int4 N=16384 K=4096 M=1 hot (one weight copy, cache-resident)",
                      "us_per_call": round(s * 1e6, 3), "GB/s": round(effective_gbps(nb, s), 1),
                      "TFLOP/s": round(2 * 16384 * 4096 / s / 1e12, 3),
                      "bound": "hbm", "roofline_frac": round(roof_fraction("hbm", nb, 0, s), 4)})
        del mk
        for label, b in sweep_cases():
            mk, nb, fl, bound = b()
            s = run_case(mk, max(20, args.steps // 10), max(5, args.warmup // 10))
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
    if not args.no_cpu:
        med, threads, reps = cpu_baseline(d, args.cpu_seconds)
        cpu = {"value": round(effective_gbps(nbytes, med), 3), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"full int4 N=16384 K=4096 M=1 call on the same host buffers, median of "
                         f"{reps} calls, {threads} threads, {os.cpu_count()} host CPUs visible"}

    line = {
        "metric": "effective weight GB/s per qmv call at M=1 (int4 N=16384 K=4096)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "int4 symmetric (q-8) skinny GEMM, N=16384, K=4096, group-32 fp16 "
                               "scales, fp16 x, M=1, fixed order, cold weights",
                   "M": 1, "N": 16384, "K": 4096, "weight_copies": copies,
                   "bytes_per_call": nbytes, "source_digest": digest},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
