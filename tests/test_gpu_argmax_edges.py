"""GPU: the int2 lm_head + argmax at the edges of its shape range, bit for bit
against the oracle (indices, maxima and logits): the most activation rows
(256, one completion counter per row chunk), a single weight row (the index
must be 0), one-segment rows (K = 64), the longest rows (K = 16384), and row
counts that leave the last row group and the last workgroup partly empty."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, bits, dev

pytestmark = pytest.mark.gpu

q = pytest.importorskip("skinny_gemm_qmv_amd")


@pytest.mark.parametrize("M,N,K", [
    (256, 4096, 1536),   # the most activation rows
    (255, 777, 1536),    # ragged rows and row chunks
    (1, 1, 64),          # one weight row of one segment
    (3, 1, 1536),        # one weight row, several activation rows
    (7, 3, 64),
    (2, 4097, 16384),    # the longest rows, a ragged row group
    (1, 65537, 1536),    # one row past a power of two
    (64, 9000, 4096),
])
def test_argmax_edges(M, N, K):
    d = synth.argmax_inputs(M, N, K, salt=M * 31 + N + K)
    idx, mv, lg = q.qmv_int2_argmax(dev(d["wq"], "u32"), dev(d["scale"], "f16"), dev(d["x"], "f16"),
                                    want_logits=True)
    torch.cuda.synchronize()
    ri, rm, rl = oracle.int2_argmax(d["wq"], d["scale"], d["x"])
    assert_bits_equal(bits(lg), rl.view(np.uint32), f"logits M={M} N={N} K={K}")
    assert np.array_equal(idx.cpu().numpy(), ri), f"idx M={M} N={N} K={K}"
    assert_bits_equal(bits(mv), rm.view(np.uint32), f"maxval M={M} N={N} K={K}")
    if N == 1:
        assert (idx.cpu().numpy() == 0).all()


def test_argmax_without_maxval_or_logits():
    """idx alone (maxval and logits null) equals the full call's idx."""
    d = synth.argmax_inputs(5, 20000, 1536, salt=77)
    args = (dev(d["wq"], "u32"), dev(d["scale"], "f16"), dev(d["x"], "f16"))
    full, _, _ = q.qmv_int2_argmax(*args, want_logits=True)
    only, mv, lg = q.qmv_int2_argmax(*args, want_maxval=False, want_logits=False)
    torch.cuda.synchronize()
    assert mv is None and lg is None
    assert torch.equal(full, only)
