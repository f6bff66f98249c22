"""Pins for the CPU oracle: checks against facts fixed by the pages, by the
format specifications and by mathematics, never against the oracle itself.

Each ``check_*`` takes a loaded oracle library (so the same checks can be
run against deliberately broken copies of the oracle) and raises
AssertionError on failure.
"""
import json
import math
import os

import numpy as np

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U32 = 2.0 ** -24  # unit roundoff of binary32


def gamma(d):
    return d * U32 / (1.0 - d * U32)


# ------------------------------------------------------------- conversions --

def check_f16_decode_all(lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = np.array([lib.orc_f16_to_f32(int(b)) for b in bits], np.float32)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _interesting_f32(g, n):
    # wide exponent sweep, fp16 halfway points, overflow and subnormal borders
    e = g.integers(-30, 20, size=n)
    m = g.uniform(1.0, 2.0, size=n)
    v = (np.ldexp(m, e) * np.where(g.random(n) < 0.5, -1.0, 1.0)).astype(np.float32)
    h = g.integers(0, 0x7C00, size=n // 4).astype(np.uint16).view(np.float16).astype(np.float64)
    halfway = (h + np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(h), 2.0 ** -24))).astype(int) - 11)
               ).astype(np.float32)
    specials = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 65536.0, 2.0 ** -24, 2.0 ** -25,
                         2.0 ** -25 * 1.5, 2.0 ** -14, 2.0 ** -14 * (1 - 2.0 ** -11), 1e-30, 1e30],
                        np.float32)
    return np.concatenate([v, halfway, specials, -specials])


def check_f32_to_f16_rne(lib):
    g = np.random.default_rng(11)
    v = _interesting_f32(g, 20000)
    ours = np.array([lib.orc_f32_to_f16(float(a)) for a in v], np.uint16)
    ref = v.astype(np.float16).view(np.uint16)  # numpy: IEEE round-to-nearest-even
    assert np.array_equal(ours, ref), np.flatnonzero(ours != ref)[:10]


def check_f64_to_f16_rne(lib):
    g = np.random.default_rng(12)
    v = np.concatenate([g.standard_normal(5000), np.ldexp(g.uniform(1, 2, 5000), g.integers(-28, 17, 5000))])
    ours = np.array([lib.orc_f64_to_f16(float(a)) for a in v], np.uint16)
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def check_f32_to_bf16_rne(lib):
    import torch
    g = np.random.default_rng(13)
    v = np.concatenate([
        (np.ldexp(g.uniform(1, 2, 20000), g.integers(-140, 127, 20000))
         * np.where(g.random(20000) < 0.5, -1, 1)).astype(np.float32),
        # exact halfway points between adjacent bf16 values
        ((g.integers(0, 0x7F00, 4000).astype(np.uint32) << 16) | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 3.3895314e38, 3.4028235e38, 1e-40, 1e-45], np.float32),
    ])
    ours = np.array([lib.orc_f32_to_bf16(float(a)) for a in v], np.uint16)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref), np.flatnonzero(ours != ref)[:10]


def check_bf16_decode(lib):
    bits = np.arange(0, 65536, 7, dtype=np.uint32)
    ours = np.array([lib.orc_bf16_to_f32(int(b)) for b in bits], np.float32)
    ref = (bits << 16).view(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# ----------------------------------------------------------------- decode --

def check_int2_decode(lib):
    import ctypes as C
    a, b = (C.c_int8 * 4)(), (C.c_int8 * 4)()
    for byte in range(256):
        lib.orc_int2_decode_byte_lut(byte, C.cast(a, C.c_void_p))
        lib.orc_int2_decode_byte_arith(byte, C.cast(b, C.c_void_p))
        assert list(a) == list(b), byte
        # two's-complement reading of each 2-bit field, low field first
        for t in range(4):
            f = (byte >> (2 * t)) & 3
            assert a[t] == (f if f < 2 else f - 4), (byte, t)
    # worked bytes: 0xE4 = fields 0,1,2,3 (low first) -> 0, 1, -2, -1
    lib.orc_int2_decode_byte_arith(0xE4, C.cast(a, C.c_void_p))
    assert list(a) == [0, 1, -2, -1]
    lib.orc_int2_decode_byte_lut(0x00, C.cast(a, C.c_void_p))
    assert list(a) == [0, 0, 0, 0]
    lib.orc_int2_decode_byte_lut(0xFF, C.cast(a, C.c_void_p))
    assert list(a) == [-1, -1, -1, -1]
    vals = sorted({lib.orc_int2_value(f) for f in range(4)})
    assert vals == [-2, -1, 0, 1]


def check_int4_decode(lib):
    import ctypes as C
    out = (C.c_int8 * 2)()
    seen = []
    for byte in range(256):
        lib.orc_int4_decode_byte_arith(byte, C.cast(out, C.c_void_p))
        lut = [lib.orc_int4_value(byte & 15), lib.orc_int4_value(byte >> 4)]
        assert list(out) == lut, byte
        seen += lut
    # symmetric code-8: every value -8..7 once per nibble position, 0 at code 8
    assert sorted(set(seen)) == list(range(-8, 8))
    assert lib.orc_int4_value(8) == 0 and lib.orc_int4_value(0) == -8 and lib.orc_int4_value(15) == 7


def check_e2m1_table(lib):
    # OCP MX v1.0 E2M1: exponent bias 1, one mantissa bit, subnormal at exponent 0
    for nib in range(16):
        s, e, m = nib >> 3, (nib >> 1) & 3, nib & 1
        mag = 0.5 * m if e == 0 else math.ldexp(1.0 + 0.5 * m, e - 1)
        want = -mag if s else mag
        got = lib.orc_e2m1_value(nib)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), nib
    for e in range(255):
        assert lib.orc_e8m0_value(e) == math.ldexp(1.0, e - 127), e
    assert math.isnan(lib.orc_e8m0_value(255))


def check_pack_roundtrip(lib):
    g = np.random.default_rng(21)
    v = g.integers(-2, 2, size=(5, 192)).astype(np.int8)
    assert np.array_equal(oracle.unpack_int2(oracle.pack_int2(v, lib), 192, lib), v)
    q = g.integers(0, 16, size=(5, 96)).astype(np.uint8)
    assert np.array_equal(oracle.unpack_int4(oracle.pack_int4(q, lib), 96, lib), q)
    nb = g.integers(0, 16, size=(5, 96)).astype(np.uint8)
    assert np.array_equal(oracle.unpack_e2m1(oracle.pack_e2m1(nb, lib), 96, lib), nb)
    # every code at every position: little-endian fields along K
    for i in range(16):
        for c in (-2, -1, 1):
            row = np.zeros((1, 16), np.int8)
            row[0, i] = c
            assert int(oracle.pack_int2(row, lib)[0, 0]) == ((c & 3) << (2 * i))
    for i in range(8):
        for q0 in (1, 7, 15):
            row = np.zeros((1, 8), np.uint8)
            row[0, i] = q0
            assert int(oracle.pack_int4(row, lib)[0, 0]) == (q0 << (4 * i))
    for k in range(2):
        row = np.zeros((1, 2), np.uint8)
        row[0, k] = 0xB
        assert int(oracle.pack_e2m1(row, lib)[0, 0]) == (0xB << (4 * k))


# --------------------------------------------------------------- products --

def check_products_exact():
    """The products the fixed order relies on are exact in binary32, so a
    fused multiply-add and a multiply-then-add give the same bits."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = h[np.isfinite(h)].astype(np.float32)
    for c in list(range(-8, 8)):
        p32 = (np.float32(c) * h).astype(np.float64)
        p64 = np.float64(c) * h.astype(np.float64)
        assert np.array_equal(p32, p64), c
    b = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    b = b[np.isfinite(b)]
    for v in (0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.5, -6.0):
        p32 = np.float32(v) * b
        p64 = np.float64(v) * b.astype(np.float64)
        ok = np.abs(p64) <= np.finfo(np.float32).max
        assert np.array_equal(p32[ok].astype(np.float64), p64[ok]), v


# --------------------------------------------------------------- FO sums ---

def _tiny_cases():
    g = np.random.default_rng(31)
    for K in (64, 128, 192, 1536):
        for M, N in ((1, 1), (2, 7), (3, 5)):
            yield g, M, N, K


def check_int2_vs_fp64(lib):
    for g, M, N, K in _tiny_cases():
        wq = synth.raw_words(g, (N, K // 16))
        sc = synth.f16_bits(g.uniform(0.01, 0.05, N))
        x = synth.f16_bits(g.standard_normal((M, K)) * 4)
        y = oracle.qmv_int2(wq, sc, x, lib=lib)
        y64, a = oracle.ref64_int2(wq, sc, x, lib=lib)
        d = 63 + math.ceil(math.log2(K // 64)) if K > 64 else 63
        bound = gamma(d) * a * (1 + U32) + U32 * np.abs(y64) + 1e-12 * a
        assert np.all(np.abs(y - y64) <= bound), (K, M, N, np.max(np.abs(y - y64) - bound))


def check_int4_vs_fp64(lib):
    for g, M, N, K in _tiny_cases():
        wq = synth.raw_words(g, (N, K // 8))
        sc = synth.f16_bits(g.uniform(0.005, 0.02, (N, K // 32)))
        x = synth.f16_bits(g.standard_normal((M, K)) * 4)
        y = oracle.qmv_int4(wq, sc, x, lib=lib)
        y64, a = oracle.ref64_int4(wq, sc, x, lib=lib)
        d = 31 + 1 + math.ceil(math.log2(K // 32))
        bound = gamma(d) * a + 1e-12 * a
        assert np.all(np.abs(y - y64) <= bound), (K, M, N, np.max(np.abs(y - y64) - bound))


def check_mxfp4_vs_fp64(lib):
    for g, M, N, K in _tiny_cases():
        wq = synth.raw_bytes(g, (N, K // 2))
        e = (127 + g.integers(-8, 3, (N, K // 32))).astype(np.uint8)
        x = synth.bf16_bits(g.standard_normal((M, K)) * 4)
        y = oracle.qmm_mxfp4(wq, e, x, lib=lib)
        y64, a = oracle.ref64_mxfp4(wq, e, x, lib=lib)
        d = 31 + 1 + math.ceil(math.log2(K // 32))
        bound = gamma(d) * a + 1e-12 * a
        assert np.all(np.abs(y - y64) <= bound), (K, M, N, np.max(np.abs(y - y64) - bound))


def check_integer_x_exact(lib):
    """Integer-valued x with power-of-two scales: every partial sum is exact,
    so any order equals the exact dot product."""
    g = np.random.default_rng(41)
    for K in (64, 192, 1536):
        M, N = 2, 6
        x = synth.f16_bits(g.integers(-8, 9, (M, K)).astype(np.float64))
        wq = synth.raw_words(g, (N, K // 16))
        sc = synth.f16_bits(np.ldexp(1.0, g.integers(-4, 3, N)))
        y = oracle.qmv_int2(wq, sc, x, lib=lib)
        y64, _ = oracle.ref64_int2(wq, sc, x, lib=lib)
        assert np.array_equal(y.astype(np.float64), y64)
        wq4 = synth.raw_words(g, (N, K // 8))
        sc4 = synth.f16_bits(np.ldexp(1.0, g.integers(-4, 3, (N, K // 32))))
        y = oracle.qmv_int4(wq4, sc4, x, lib=lib)
        y64, _ = oracle.ref64_int4(wq4, sc4, x, lib=lib)
        assert np.array_equal(y.astype(np.float64), y64)
        xb = synth.bf16_bits(g.integers(-8, 9, (M, K)).astype(np.float64))
        wq8 = synth.raw_bytes(g, (N, K // 2))
        e = (127 + g.integers(-8, 3, (N, K // 32))).astype(np.uint8)
        y = oracle.qmm_mxfp4(wq8, e, xb, lib=lib)
        y64, _ = oracle.ref64_mxfp4(wq8, e, xb, lib=lib)
        assert np.array_equal(y.astype(np.float64), y64)


def check_single_segment_sequential(lib):
    """With one segment per row the fixed order is a plain running sum in
    code order (numpy's cumulative sum in float32), then the row scale."""
    g = np.random.default_rng(51)
    x = synth.f16_bits(g.standard_normal((1, 64)) * 100)
    vals = g.integers(-2, 2, (3, 64)).astype(np.int8)
    wq = oracle.pack_int2(vals, lib)
    sc = synth.f16_bits(g.uniform(0.01, 0.05, 3))
    y = oracle.qmv_int2(wq, sc, x, lib=lib)
    xf = x.view(np.float16).astype(np.float32)[0]
    for n in range(3):
        run = np.cumsum(vals[n].astype(np.float32) * xf, dtype=np.float32)[-1]
        assert y[0, n] == np.float32(sc.view(np.float16)[n]) * run
    # int4: one group of 32, value q-8, then the group scale
    x = synth.f16_bits(g.standard_normal((1, 32)) * 100)
    q = g.integers(0, 16, (3, 32)).astype(np.uint8)
    sc = synth.f16_bits(g.uniform(0.005, 0.02, (3, 1)))
    y = oracle.qmv_int4(oracle.pack_int4(q, lib), sc, x, lib=lib)
    xf = x.view(np.float16).astype(np.float32)[0]
    for n in range(3):
        run = np.cumsum((q[n].astype(np.float32) - 8) * xf, dtype=np.float32)[-1]
        assert y[0, n] == np.float32(sc.view(np.float16)[n, 0]) * run


def _golden_row(case):
    K = case["K"]
    codes = np.zeros((1, K), np.int8)
    x = np.zeros((1, K), np.float64)
    if "segments" in case:
        for j, tag in enumerate(case["segments"]):
            base = 64 * j
            if tag in ("A", "-A"):
                codes[0, base:base + 33] = -2
                x[0, base:base + 33] = -65504.0 if tag == "A" else 65504.0
            elif tag == "s":
                codes[0, base + 1] = 1
                x[0, base + 1] = 0.125
    else:
        for ent in case["entries"]:
            k0, k1 = ent["k"]
            codes[0, k0:k1 + 1] = ent["code"]
            x[0, k0:k1 + 1] = ent["x"]
    return codes, synth.f16_bits(x)


def check_golden_order(lib):
    with open(os.path.join(GOLDEN, "fo_order_int2.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        codes, x = _golden_row(case)
        wq = oracle.pack_int2(codes, lib)
        sc = synth.f16_bits(np.array([1.0]))
        y = oracle.qmv_int2(wq, sc, x, lib=lib)
        assert y[0, 0] == np.float32(case["expected_y"]), (case["name"], y[0, 0])


def check_threads_identical(lib):
    d = synth.int2_inputs(2, 333, 1536, salt=9)
    a = oracle.qmv_int2(d["wq"], d["scale"], d["x"], threads=1, lib=lib)
    b = oracle.qmv_int2(d["wq"], d["scale"], d["x"], threads=7, lib=lib)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    d = synth.mxfp4_inputs(2, 101, 5376, salt=9)
    a = oracle.qmm_mxfp4(d["wq"], d["e8m0"], d["x"], threads=1, lib=lib)
    b = oracle.qmm_mxfp4(d["wq"], d["e8m0"], d["x"], threads=5, lib=lib)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ------------------------------------------------------------ exp / GELU ---

def _ulp32(v):
    v = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 23).astype(int))


def check_exp_accuracy(lib):
    z = np.concatenate([np.linspace(-87, 87, 200001), np.linspace(-1, 1, 20001)]).astype(np.float32)
    ours = np.array([lib.orc_exp(float(a)) for a in z], np.float64)
    ref = np.exp(z.astype(np.float64))
    err = np.abs(ours - ref) / _ulp32(ref)
    assert err.max() <= 2.0, err.max()
    assert lib.orc_exp(0.0) == 1.0


def check_gelu_accuracy(lib):
    g = np.linspace(-10, 10, 100001).astype(np.float32)
    ours = np.array([lib.orc_gelu(float(a)) for a in g], np.float64)
    gd = g.astype(np.float64)
    u = math.sqrt(2.0 / math.pi) * (gd + 0.044715 * gd ** 3)
    # g * (1 + tanh u) / 2 written as g / (1 + e^(-2u)), which double evaluates
    # without cancellation for negative g
    ref = gd / (1.0 + np.exp(-2.0 * u))
    # where -2u > 87 the definition clamps the exponent: |result| < |g| e^-87
    slack = np.where(-2.0 * u > 87.0, 2.0 * np.abs(gd) * math.exp(-87.0), 0.0)
    # the binary32 argument -2u carries ~3 roundings, so e^(-2u) is only
    # known to |2u| * 3u32 relative: the condition of the exponential
    cond = 4.0 * np.abs(2.0 * u) * U32 * np.abs(ref)
    err = (np.abs(ours - ref) - slack - cond) / _ulp32(ref)
    assert err.max() <= 8.0, err.max()
    assert lib.orc_gelu(0.0) == 0.0


# -------------------------------------------------------------- RMSNorm ----

def check_rmsnorm_vs_fp64(lib):
    for K in (64, 1536, 4096):
        d = synth.fused_inputs(1, 8, K, salt=K)
        x, r, gm = d["x"][0], d["residual"][0], d["gamma"]
        h, xn, inv = oracle.rmsnorm_prologue(x, r, gm, 1e-6, lib=lib)
        xd = x.view(np.float16).astype(np.float64)
        rd = r.view(np.float16).astype(np.float64)
        h_ref = (xd + rd).astype(np.float16)  # one rounding of the exact sum
        assert np.array_equal(h, h_ref.view(np.uint16))
        hd = h_ref.astype(np.float64)
        inv64 = 1.0 / math.sqrt(np.sum(hd * hd) / K + float(np.float32(1e-6)))
        d_ = 63 + math.ceil(math.log2(max(K // 64, 1))) + 4
        assert abs(float(inv) - inv64) <= gamma(d_) * inv64
        xn64 = hd * inv64 * gm.view(np.float16).astype(np.float64)
        got = xn.view(np.float16).astype(np.float64)
        # within one fp16 ulp (the fp32 steps are within a few binary32 ulps)
        ulp16 = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(xn64), 2.0 ** -14))).astype(int) - 10)
        assert np.all(np.abs(got - xn64) <= ulp16), np.max(np.abs(got - xn64) / ulp16)


def check_fused_composition(lib):
    d = synth.fused_inputs(2, 40, 1536, salt=3)
    out, res, g, u = oracle.int2_rmsnorm_gateup_gelu(
        d["x"], d["residual"], d["gamma"], d["eps"], d["wq_gate"], d["s_gate"], d["wq_up"],
        d["s_up"], lib=lib)
    # fp64 composition: normalise, dequantize, dot, GELU (tanh form), product
    for m in range(2):
        xd = d["x"][m].view(np.float16).astype(np.float64)
        rd = d["residual"][m].view(np.float16).astype(np.float64)
        hd = (xd + rd).astype(np.float16).astype(np.float64)
        assert np.array_equal(res[m], (xd + rd).astype(np.float16).view(np.uint16))
        xn = hd / math.sqrt(np.mean(hd * hd) + 1e-6) * d["gamma"].view(np.float16).astype(np.float64)
        xn16 = xn.astype(np.float16)
        wg = oracle.unpack_int2(d["wq_gate"], 1536, lib).astype(np.float64)
        wu = oracle.unpack_int2(d["wq_up"], 1536, lib).astype(np.float64)
        gd = (wg @ xn16.astype(np.float64)) * d["s_gate"].view(np.float16).astype(np.float64)
        ud = (wu @ xn16.astype(np.float64)) * d["s_up"].view(np.float16).astype(np.float64)
        # gate/up within a loose bound of the fp64 path (xn may differ by 1 fp16 ulp)
        assert np.max(np.abs(g[m] - gd)) <= 2e-3 * np.max(np.abs(gd)) + 1e-3
        assert np.max(np.abs(u[m] - ud)) <= 2e-3 * np.max(np.abs(ud)) + 1e-3
        gel = 0.5 * gd * (1 + np.tanh(math.sqrt(2 / math.pi) * (gd + 0.044715 * gd ** 3)))
        o = out[m].view(np.float16).astype(np.float64)
        ref = gel * ud
        assert np.max(np.abs(o - ref)) <= 5e-3 * np.max(np.abs(ref)) + 1e-3


def check_qkv_composition(lib):
    # closed form: x = 1, r = 0, gamma = 1, eps = 0 gives h = 1, sum of squares K,
    # inv = 1 and xn = 1, so y_z[n] = s_n * (sum of row n's codes), exact in fp32
    g = np.random.default_rng(71)
    M, K = 2, 640
    ns = (48, 16, 24)
    vals = [g.integers(-2, 2, (n, K)).astype(np.int8) for n in ns]
    scs = [synth.f16_bits(g.uniform(0.01, 0.05, n)) for n in ns]
    x = synth.f16_bits(np.ones((M, K)))
    r = synth.f16_bits(np.zeros((M, K)))
    gm = synth.f16_bits(np.ones(K))
    wq = [oracle.pack_int2(v, lib) for v in vals]
    yq, yk, yv, res = oracle.int2_rmsnorm_qkv(x, r, gm, 0.0, wq[0], scs[0], wq[1], scs[1], wq[2], scs[2],
                                              lib=lib)
    assert np.array_equal(res, x)
    for y, v, s in zip((yq, yk, yv), vals, scs):
        exact = s.view(np.float16).astype(np.float64) * v.astype(np.int64).sum(axis=1)
        assert np.array_equal(y, np.broadcast_to(exact.astype(np.float32), y.shape))
    # random inputs: each output within a loose bound of the fp64 composition
    d = synth.qkv_inputs(2, 40, 24, 24, 1536, salt=3)
    outs = oracle.int2_rmsnorm_qkv(d["x"], d["residual"], d["gamma"], d["eps"], d["wq_q"], d["s_q"],
                                   d["wq_k"], d["s_k"], d["wq_v"], d["s_v"], lib=lib)
    for m in range(2):
        xd = d["x"][m].view(np.float16).astype(np.float64)
        rd = d["residual"][m].view(np.float16).astype(np.float64)
        hd = (xd + rd).astype(np.float16).astype(np.float64)
        assert np.array_equal(outs[3][m], (xd + rd).astype(np.float16).view(np.uint16))
        xn = hd / math.sqrt(np.mean(hd * hd) + 1e-6) * d["gamma"].view(np.float16).astype(np.float64)
        xn16 = xn.astype(np.float16).astype(np.float64)
        for z, y in zip("qkv", outs[:3]):
            w = oracle.unpack_int2(d["wq_" + z], 1536, lib).astype(np.float64)
            yd = (w @ xn16) * d["s_" + z].view(np.float16).astype(np.float64)
            assert np.max(np.abs(y[m] - yd)) <= 2e-3 * np.max(np.abs(yd)) + 1e-3


# ------------------------------------------------------- MXFP4 quantiser --

def _mx_quant_ref(v16):
    # the conversion written another way: the block exponent from the
    # power-of-two bracket of the maximum, and the element rounding as
    # round-half-even in three fixed-step bands (step 1/2 below 2, 1 in
    # [2, 4), 2 from 4), clamped to 6
    v = v16.view(np.float16).astype(np.float64)
    amax = np.max(np.abs(v))
    if amax == 0:
        e = -127
    else:
        e = 0
        while 2.0 ** e > amax:
            e -= 1
        while 2.0 ** (e + 1) <= amax:
            e += 1
        e -= 2
    q = np.abs(v) * 2.0 ** (-e)
    r = np.where(q < 2, np.round(q * 2) / 2, np.where(q < 4, np.round(q), 2 * np.round(q / 2)))
    r = np.minimum(r, 6.0)
    mag = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    code = np.array([int(np.flatnonzero(mag == x)[0]) for x in r]) | np.where(np.signbit(v), 8, 0)
    packed = (code[0::2] | (code[1::2] << 4)).astype(np.uint8)
    return packed, np.uint8(e + 127)


def _mx_blocks(g, nblk):
    # random blocks over a wide exponent range, with exact ties and values
    # at and past the clamp planted relative to the block maximum
    blocks = []
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 7.5, 0.5, 3.0])
    for b in range(nblk):
        s = int(g.integers(-20, 12))
        top = 2.0 ** s * g.choice([4.0, 5.0, 6.0, 7.0, 7.5, 4.5])
        vals = g.uniform(-1, 1, 32) * top
        k = int(g.integers(0, 12))
        vals[1:1 + k] = g.choice(mids, k) * 2.0 ** (s - 2) * g.choice([-1, 1], k)
        vals[0] = top
        if b % 7 == 3:
            vals[:] = 0.0
            vals[5] = -0.0
        if b % 7 == 5:
            vals[:] = g.choice([-0.0, 0.0], 32)
            vals[9] = 2.0 ** -24  # smallest fp16
        g.shuffle(vals)
        blocks.append(synth.f16_bits(vals))
    return np.array(blocks)


def check_quant_mxfp4(lib):
    g = np.random.default_rng(71)
    v = _mx_blocks(g, 400)
    codes, e = oracle.quant_mxfp4(v, lib=lib)
    for i in range(v.shape[0]):
        rc, re = _mx_quant_ref(v[i])
        assert e[i, 0] == re, (i, e[i, 0], re)
        assert np.array_equal(codes[i], rc), i
    # values already on the grid of their block come back exactly
    for s in (-14, 0, 9):
        vals = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6] * 4) * np.repeat([1, -1, 1, -1], 8) * 2.0 ** s
        c, e = oracle.quant_mxfp4(synth.f16_bits(vals)[None, :], lib=lib)
        back = np.array([lib.orc_e2m1_value(int((c[0, i // 2] >> (4 * (i % 2))) & 15)) for i in range(32)])
        assert np.array_equal(back * 2.0 ** (int(e[0, 0]) - 127), vals)


def check_fused_quant_composition(lib):
    d = synth.fused_inputs(2, 96, 1536, salt=4)
    args = (d["x"], d["residual"], d["gamma"], d["eps"], d["wq_gate"], d["s_gate"], d["wq_up"], d["s_up"])
    codes, e, res = oracle.int2_rmsnorm_gateup_gelu_mxfp4(*args, lib=lib)
    out, res2, _, _ = oracle.int2_rmsnorm_gateup_gelu(*args, lib=lib)
    c2, e2 = oracle.quant_mxfp4(out, lib=lib)
    assert np.array_equal(codes, c2) and np.array_equal(e, e2) and np.array_equal(res, res2)


# ---------------------------------------------------------------- ternary --

def _ternary_table():
    # digits of every code from the encoding side: enumerate all digit tuples
    # (t0..t4) and place each at the byte sum t_i 3^i it encodes to
    import itertools
    tab = np.full((256, 5), 99, np.int64)
    for t in itertools.product(range(3), repeat=5):
        tab[sum(d * 3 ** i for i, d in enumerate(t))] = t
    return tab - 1  # weight values; rows 243..255 stay invalid (98)


def _ternary_ref64(wq, scale, x, K):
    tab = _ternary_table()
    vals = tab[wq].reshape(wq.shape[0], -1)[:, :K].astype(np.float64)  # [N][K]
    xd = x.view(np.float16).astype(np.float64)
    s = scale.view(np.float16).astype(np.float64)
    return (xd @ vals.T) * s, (np.abs(xd) @ np.abs(vals).T) * s


def check_ternary_decode(lib):
    tab = _ternary_table()
    for b in range(243):
        assert [lib.orc_ternary_value(b, i) for i in range(5)] == list(tab[b]), b
    g = np.random.default_rng(61)
    for K in (5, 80, 83, 4096):
        v = g.integers(-1, 2, (3, K)).astype(np.int8)
        wq = oracle.pack_ternary(v, lib=lib)
        assert wq.shape == (3, oracle.ternary_row_bytes(K)) and wq.max() <= 242
        got = tab[wq].reshape(3, -1)
        assert np.array_equal(got[:, :K], v) and np.all(got[:, K:] == 0)


def check_ternary_vs_fp64(lib):
    g = np.random.default_rng(62)
    for K in (16, 80, 88, 160, 600, 1536):
        for M, N in ((1, 1), (2, 7), (3, 5)):
            d = synth.ternary_inputs(M, N, K, salt=K + N)
            x = synth.f16_bits(g.standard_normal((M, K)) * 4)
            y = oracle.qmv_ternary(d["wq"], d["scale"], x, lib=lib)
            y64, a = _ternary_ref64(d["wq"], d["scale"], x, K)
            nseg = (K + 79) // 80
            dd = 80 + (math.ceil(math.log2(nseg)) if nseg > 1 else 0)
            bound = gamma(dd) * a * (1 + U32) + U32 * np.abs(y64) + 1e-12 * a
            assert np.all(np.abs(y - y64) <= bound), (K, M, N)
            if K % 80:  # digits past K are never read: redraw them, same bits
                wq2 = d["wq"].copy().astype(np.int64)
                full = -(-K // 5)  # first byte holding only digits past K
                wq2[:, full:] = g.integers(0, 243, (N, wq2.shape[1] - full))
                r = K % 5
                if r:  # the byte holding digit K: keep its low r digits
                    lo = wq2[:, K // 5] % 3 ** r
                    wq2[:, K // 5] = lo + 3 ** r * g.integers(0, 3 ** (5 - r), N)
                y2 = oracle.qmv_ternary(wq2.astype(np.uint8), d["scale"], x, lib=lib)
                assert np.array_equal(y2.view(np.uint32), y.view(np.uint32)), K


def check_ternary_closed_form(lib):
    # every weight +1 (or every weight -1) and integer x: every partial sum is
    # exact, so y = s * (+-sum x) exactly; power-of-two scales keep it exact
    g = np.random.default_rng(63)
    for K in (80, 400, 4096):
        xi = g.integers(-6, 7, (2, K))
        x = synth.f16_bits(xi.astype(np.float64))
        s = np.ldexp(1.0, g.integers(-3, 3, 4))
        for code, sign in ((242, 1), (0, -1)):
            wq = np.full((4, oracle.ternary_row_bytes(K)), code, np.uint8)
            y = oracle.qmv_ternary(wq, synth.f16_bits(s), x, lib=lib)
            want = sign * xi.sum(axis=1)[:, None] * s[None, :]
            assert np.array_equal(y.astype(np.float64), want)


def check_expert_gather(lib):
    # closed form: expert e has every element 1.0 (E2M1 code 2) and every block
    # scale 2^e; with integer x the output is exactly 2^idx * sum(x), so each
    # output names the expert it was computed from
    g = np.random.default_rng(81)
    E, M, topk, N, K = 6, 3, 4, 5, 96
    wq = np.full((E, N, K // 2), 0x22, np.uint8)
    e8 = np.broadcast_to((127 + np.arange(E, dtype=np.uint8))[:, None, None], (E, N, K // 32)).copy()
    xi = g.integers(-4, 5, (M, K))
    x = synth.bf16_bits(xi.astype(np.float64))
    idx = np.array([[5, 0, 3, 3], [1, 2, 4, 0], [0, 0, 0, 0]], np.int32)  # duplicates allowed
    y = oracle.qmm_mxfp4_gather(wq, e8, x, idx, lib=lib)
    want = np.ldexp(1.0, idx)[:, :, None] * xi.sum(axis=1)[:, None, None]
    assert np.array_equal(y, np.broadcast_to(want, y.shape).astype(np.float32))
    # random experts: within the fixed-order bound of brute-force fp64 on the selected expert
    d = synth.expert_inputs(2, 8, 3, 24, 256, salt=1)
    y = oracle.qmm_mxfp4_gather(d["wq"], d["e8m0"], d["x"], d["idx"], lib=lib)
    table = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])
    xd = d["x"].astype(np.uint32).astype(np.uint64) << np.uint64(16)
    xd = xd.astype(np.uint32).view(np.float32).astype(np.float64)
    for m in range(2):
        for j in range(3):
            e = int(d["idx"][m, j])
            nib = np.stack([d["wq"][e] & 15, d["wq"][e] >> 4], axis=-1).reshape(24, 256)
            w = table[nib] * np.repeat(np.ldexp(1.0, d["e8m0"][e].astype(int) - 127), 32, axis=1)
            exact = w @ xd[m]
            mag = np.abs(w) @ np.abs(xd[m])
            assert np.all(np.abs(y[m, j] - exact) <= gamma(32 + 3 + 1) * mag)


# --------------------------------------------------------------- argmax ----

def check_argmax_ties(lib):
    g = np.random.default_rng(61)
    K, N = 128, 50
    vals = g.integers(-2, 2, (N, K)).astype(np.int8)
    x = synth.f16_bits(g.standard_normal((1, K)))
    sc = synth.f16_bits(np.full(N, 0.03))
    _, _, logits = oracle.int2_argmax(oracle.pack_int2(vals, lib), sc, x, lib=lib)
    best = int(np.argmax(logits[0]))
    # duplicate the winning row at a higher index: the lower index must win
    v2 = vals.copy()
    v2[N - 1] = vals[best]
    idx, mv, lg = oracle.int2_argmax(oracle.pack_int2(v2, lib), sc, x, lib=lib)
    assert int(idx[0]) == min(best, N - 1) and mv[0] == lg[0, idx[0]]
    # duplicate at a lower index: that index wins
    lo = 0 if best != 0 else 1
    v3 = vals.copy()
    v3[lo] = vals[best]
    idx, _, _ = oracle.int2_argmax(oracle.pack_int2(v3, lib), sc, x, lib=lib)
    assert int(idx[0]) == min(lo, best)
    # all-zero logits, some rows with negative scale (-0 results): index 0
    z = np.zeros((N, K), np.int8)
    scz = synth.f16_bits(np.where(np.arange(N) % 2 == 0, -0.03, 0.03))
    idx, mv, lg = oracle.int2_argmax(oracle.pack_int2(z, lib), scz, x, lib=lib)
    assert np.signbit(lg[0, 0]) and int(idx[0]) == 0 and mv[0] == 0.0
    # against numpy's argmax (first occurrence) on the oracle's own logits, M = 4
    d = synth.int2_inputs(4, 3000, 256, salt=2)
    idx, mv, lg = oracle.int2_argmax(d["wq"], d["scale"], d["x"], lib=lib)
    assert np.array_equal(idx, np.argmax(lg, axis=1).astype(np.int32))
    assert np.array_equal(mv, lg.max(axis=1))


def check_no_contraction(lib):
    """The arithmetic contract: every binary32 operation rounds on its own,
    and nothing is fused unless written as fma.  (1 + 2^-12)^2 = 1 + 2^-11 +
    2^-24 is a tie between two binary32 neighbours and rounds to the even one,
    1 + 2^-11; adding -(1 + 2^-11) then gives exactly 0, while one fused
    rounding would keep the 2^-24.  Both roundings are worked out exactly
    here with rationals."""
    from fractions import Fraction as Fr
    a = 1.0 + 2.0 ** -12
    c = -(1.0 + 2.0 ** -11)
    exact = Fr(a) * Fr(a)
    lo = Fr(1) + Fr(2) ** -11            # 1 + 2^-11: last significand bit 0
    hi = lo + Fr(2) ** -23               # its upper neighbour
    assert exact - lo == hi - exact       # a tie, resolved to the even lo
    unfused = float(lo + Fr(c))
    fused = float(exact + Fr(c))
    assert unfused == 0.0 and fused == 2.0 ** -24
    got = lib.orc_probe_mul_add(a, a, c)
    assert got == unfused and math.copysign(1.0, got) == 1.0, got


ALL_CHECKS = [
    check_f16_decode_all, check_f32_to_f16_rne, check_f64_to_f16_rne, check_f32_to_bf16_rne,
    check_bf16_decode, check_int2_decode, check_int4_decode, check_e2m1_table, check_pack_roundtrip,
    check_int2_vs_fp64, check_int4_vs_fp64, check_mxfp4_vs_fp64, check_integer_x_exact,
    check_single_segment_sequential, check_golden_order, check_threads_identical,
    check_exp_accuracy, check_gelu_accuracy, check_rmsnorm_vs_fp64, check_fused_composition,
    check_qkv_composition, check_expert_gather, check_ternary_decode, check_ternary_vs_fp64,
    check_ternary_closed_form, check_quant_mxfp4, check_fused_quant_composition, check_argmax_ties,
    check_no_contraction,
]
