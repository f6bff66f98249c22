"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pins catch every one of them.  The real oracle is never modified."""
import os

import pytest

import oracle
from oracle import build as obuild
import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text to replace, replacement, extra compiler flags, pin expected to fail)
MUTANTS = [
    ("tree_sequential",
     "for (int p = 0; p < s; ++p) v[p] = v[p] + v[p + s];",
     "if (s == 1) for (int p = 1; p < p2; ++p) v[0] = v[0] + v[p];",
     (), P.check_golden_order),
    ("tree_adjacent_pairs",
     "for (int p = 0; p < s; ++p) v[p] = v[p] + v[p + s];",
     "for (int p = 0; p < s; ++p) v[p] = v[2 * p] + v[2 * p + 1];",
     (), P.check_golden_order),
    ("int2_fields_swapped",
     "static const int INT2_VALUE[4] = {0, 1, -2, -1};",
     "static const int INT2_VALUE[4] = {0, 1, -1, -2};",
     (), P.check_int2_decode),
    ("int2_unsigned",
     "static const int INT2_VALUE[4] = {0, 1, -2, -1};",
     "static const int INT2_VALUE[4] = {-2, -1, 0, 1};",
     (), P.check_int2_decode),
    ("int4_bias_off_by_one",
     "ORC_API int orc_int4_value(unsigned q) { return (int)(q & 15u) - 8; }",
     "ORC_API int orc_int4_value(unsigned q) { return (int)(q & 15u) - 7; }",
     (), P.check_int4_decode),
    ("int4_group_scale_index",
     "v[j] = orc_f16_to_f32(srow[j]) * t;",
     "v[j] = orc_f16_to_f32(srow[j ^ 1]) * t;",
     (), P.check_int4_vs_fp64),
    ("mxfp4_nibble_order_in_fo",
     "float c = orc_e2m1_value((k % 2 == 0) ? (b & 15u) : (b >> 4));",
     "float c = orc_e2m1_value((k % 2 == 1) ? (b & 15u) : (b >> 4));",
     (), P.check_mxfp4_vs_fp64),
    ("mxfp4_scale_bias",
     "return ldexpf(1.0f, (int)e - 127);",
     "return ldexpf(1.0f, (int)e - 128);",
     (), P.check_e2m1_table),
    ("int2_dropped_last_code",
     "for (int64_t k = 64 * (int64_t)j; k < 64 * (int64_t)j + 64; ++k) {\n            float c = (float)orc_int2_value",
     "for (int64_t k = 64 * (int64_t)j; k < 64 * (int64_t)j + 63; ++k) {\n            float c = (float)orc_int2_value",
     (), P.check_int2_vs_fp64),
    ("f16_subnormal_exponent",
     "v = ldexp((double)m, -24);",
     "v = ldexp((double)m, -25);",
     (), P.check_f16_decode_all),
    ("f16_round_half_up",
     "double r = nearbyint(q);            /* ties to even */",
     "double r = floor(q + 0.5);",
     (), P.check_f32_to_f16_rne),
    ("exp_dropped_term",
     "0x1.6c16c2p-10f, 0x1.a01a02p-13f};",
     "0x0p+0f, 0x0p+0f};",
     (), P.check_exp_accuracy),
    ("gelu_constant",
     "#define ORC_GELU_C 0x1.6e4e26p-5f",
     "#define ORC_GELU_C 0x1.6e4e26p-4f",
     (), P.check_gelu_accuracy),
    ("rmsnorm_mean_over_k_minus_1",
     "float ms = ss / (float)K;",
     "float ms = ss / (float)(K - 1);",
     (), P.check_rmsnorm_vs_fp64),
    ("rmsnorm_residual_not_added",
     "h_out[k] = orc_f64_to_f16((double)orc_f16_to_f32(x[k]) + (double)orc_f16_to_f32(r[k]));",
     "h_out[k] = x[k];",
     (), P.check_rmsnorm_vs_fp64),
    ("gather_ids_transposed",
     "const int64_t e = idx[m * topk + j];",
     "const int64_t e = idx[j * M + m];",
     (), P.check_expert_gather),
    ("gather_expert_stride",
     "orc_qmm_mxfp4(wq + e * N * (K / 2), e8m0 + e * N * (K / 32), x + m * K,",
     "orc_qmm_mxfp4(wq + e * N * (K / 2), e8m0 + e * (N - 1) * (K / 32), x + m * K,",
     (), P.check_expert_gather),
    ("qkv_k_not_normalised",
     "orc_qmv_int2(wq_k, s_k, xn, yk, M, Nk, K, nthreads);",
     "orc_qmv_int2(wq_k, s_k, h, yk, M, Nk, K, nthreads);",
     (), P.check_qkv_composition),
    ("ternary_digit_order_reversed",
     "for (int s = 0; s < i; ++s) d /= 3u;",
     "for (int s = 0; s < 4 - i; ++s) d /= 3u;",
     (), P.check_ternary_decode),
    ("ternary_digit_index_shifted",
     "float c = (float)orc_ternary_value(row[k / 5], (int)(k % 5));",
     "float c = (float)orc_ternary_value(row[k / 5], (int)((k + 1) % 5));",
     (), P.check_ternary_vs_fp64),
    ("mxfp4_quant_ties_to_odd",
     "if (dc < db || (dc == db && (c % 2) == 0)) best = c;",
     "if (dc < db || (dc == db && (c % 2) == 1)) best = c;",
     (), P.check_quant_mxfp4),
    ("mxfp4_quant_exponent_off_by_one",
     "shared = ex - 1 - 2;",
     "shared = ex - 2;",
     (), P.check_quant_mxfp4),
    ("mxfp4_quant_sign_dropped",
     "unsigned code = (unsigned)best | (signbit(x) ? 8u : 0u);",
     "unsigned code = (unsigned)best | (x < 0.0 ? 8u : 0u);",
     (), P.check_quant_mxfp4),
    ("argmax_last_max",
     "if (y[m * N + n] > y[m * N + best]) best = n;",
     "if (y[m * N + n] >= y[m * N + best]) best = n;",
     (), P.check_argmax_ties),
]


@pytest.mark.parametrize("name,old,new,flags,check", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new, flags, check):
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation anchor for {name} not found"
    src = tmp_path / f"oracle_{name}.c"
    src.write_text(text.replace(old, new))
    lib = oracle.load(obuild.build(str(src), str(tmp_path / f"lib_{name}.so"), flags, quiet=True))
    with pytest.raises(AssertionError):
        check(lib)


def test_unmutated_copy_passes(tmp_path):
    """The same build route with no mutation passes the same pins."""
    src = tmp_path / "oracle_copy.c"
    src.write_text(open(SRC).read())
    lib = oracle.load(obuild.build(str(src), str(tmp_path / "lib_copy.so"), (), quiet=True))
    for check in {m[4] for m in MUTANTS}:
        check(lib)


# Build-flag mutants: the same source built with flags that break the
# arithmetic contract.  Checked in a child process, because a shared object
# built with -ffast-math may switch the whole process to flush-to-zero.
FLAG_MUTANTS = [
    ("fast_math", ("-ffast-math",)),                            # FTZ/DAZ, reassociation, no signed zeros
    ("contraction_with_fma", ("-ffp-contract=fast", "-mfma")),  # a*b+c fused into one rounding
]

CHILD = r"""
import json, os, sys
sys.path[:0] = [os.environ["QMV_ROOT"], os.path.join(os.environ["QMV_ROOT"], "tests")]
import oracle, oracle_pins as P
lib = oracle.load(sys.argv[1])
failed = []
for check in P.ALL_CHECKS:
    try:
        check(lib)
    except AssertionError:
        failed.append(check.__name__)
print(json.dumps(failed))
"""


def _pins_in_child(lib_path, env_extra=None, timeout=900):
    import json
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, QMV_ROOT=root, **(env_extra or {}))
    r = subprocess.run([sys.executable, "-c", CHILD, lib_path], capture_output=True, text=True, timeout=timeout,
                       env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    return json.loads(r.stdout.strip().splitlines()[-1])


@pytest.mark.parametrize("name,flags", FLAG_MUTANTS, ids=[m[0] for m in FLAG_MUTANTS])
def test_flag_mutant_is_caught(tmp_path, name, flags):
    lib = obuild.build(SRC, str(tmp_path / f"lib_{name}.so"), flags, quiet=True)
    failed = _pins_in_child(lib)
    assert failed, f"no pin rejected the oracle built with {flags}"


def test_pins_pass_under_address_and_undefined_sanitizers(tmp_path):
    """The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
    (any report aborts) passes every pin: no out-of-bounds access, no
    undefined arithmetic anywhere the pins reach."""
    import subprocess
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                             check=True).stdout.strip()
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.skip("gcc has no AddressSanitizer runtime here")
    flags = ("-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g")
    lib = obuild.build(SRC, str(tmp_path / "lib_asan.so"), flags, quiet=True)
    env = {"LD_PRELOAD": libasan, "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}
    failed = _pins_in_child(lib, env)
    assert failed == [], failed
