"""The no-allocation argmax entry point (qmv_int2_argmax_static, scratch in
a static device array of the library) against the workspace entry point
(qmv_int2_argmax) through the C ABI: identical idx, maxval and logits bits on
two calls in a row, the first at the largest M the scratch holds, the second
smaller, which also checks that the first call left the scratch zeroed."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, bits, dev

pytestmark = pytest.mark.gpu

q = pytest.importorskip("skinny_gemm_qmv_amd")


def both(M, N, K, salt):
    d = synth.argmax_inputs(M, N, K, salt=salt)
    wq, sc, x = dev(d["wq"], "u32"), dev(d["scale"], "f16"), dev(d["x"], "f16")
    ri, rm, rl = q.qmv_int2_argmax(wq, sc, x, want_logits=True)
    idx = torch.empty(M, dtype=torch.int32, device="cuda")
    mv = torch.empty(M, dtype=torch.float32, device="cuda")
    lg = torch.empty((M, N), dtype=torch.float32, device="cuda")
    q.qmv_int2_argmax_static(wq, sc, x, idx, maxval=mv, logits=lg)
    torch.cuda.synchronize()
    assert_bits_equal(bits(idx), bits(ri), f"idx M={M} N={N}")
    assert_bits_equal(bits(mv), bits(rm), f"maxval M={M} N={N}")
    assert_bits_equal(bits(lg), bits(rl), f"logits M={M} N={N}")
    return d, idx


def test_static_scratch_matches_workspace_call_twice():
    both(256, 8192, 1536, salt=1)          # every key slot of the scratch in use
    d, idx = both(3, 2048, 1536, salt=2)   # smaller: the scratch must be back at zero
    ri, _, _ = oracle.int2_argmax(d["wq"], d["scale"], d["x"])
    assert np.array_equal(idx.cpu().numpy(), ri)


def test_static_scratch_lm_head_shape():
    both(1, 262144, 1536, salt=3)
    both(1, 262144, 1536, salt=4)


def test_static_scratch_rejects_bad_arguments():
    """Validation happens before the scratch is touched."""
    lib = q._lib
    assert lib.qmv_int2_argmax_static(None, None, None, None, None, None, 1, 64, 64, 0, None) == 1
    wq = torch.zeros((64, 4), dtype=torch.int32, device="cuda")
    sc = torch.zeros(64, dtype=torch.float16, device="cuda")
    x = torch.zeros((1, 64), dtype=torch.float16, device="cuda")
    idx = torch.zeros(1, dtype=torch.int32, device="cuda")
    P = q._ptr
    assert lib.qmv_int2_argmax_static(P(wq), P(sc), P(x), P(idx), None, None, 257, 64, 64, 0, None) == 1
    assert lib.qmv_int2_argmax_static(P(wq), P(sc), P(x), P(idx), None, None, 1, 64, 64, 1, None) == 4
