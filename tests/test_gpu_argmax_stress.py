"""GPU: many back-to-back lm_head + argmax calls of varying shape on one
workspace (and on the library's static scratch), with nothing between them
on the stream.  The single-dispatch merge (per-row 64-bit keys folded with
atomic max, a self-resetting completion counter, the last workgroup's
exchange) must give, for every call, the first maximum of the logits that
the same call wrote; the logits themselves are checked against the oracle
elsewhere."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import dev

pytestmark = pytest.mark.gpu

q = pytest.importorskip("skinny_gemm_qmv_amd")

SHAPES = [(1, 262144), (4, 262144), (1, 5000), (3, 70000), (2, 129), (1, 1), (7, 33000), (1, 131072)]


def first_max(lg):
    """Index of the first maximum per row (-0 == +0), on the host."""
    a = lg.cpu().numpy()
    return np.argmax(a, axis=1).astype(np.int32)


@pytest.mark.parametrize("static", [False, True])
def test_many_calls_in_a_row(static):
    K = 1536
    data = []
    for i, (M, N) in enumerate(SHAPES):
        d = synth.argmax_inputs(M, N, K, salt=900 + i)
        data.append((M, N, dev(d["wq"], "u32"), dev(d["scale"], "f16"), dev(d["x"], "f16")))
    ws = None
    if not static:
        ws = torch.empty(q.workspace_size("int2_argmax", 8, 262144, K), dtype=torch.uint8, device="cuda")
        q.workspace_init(ws)
    outs = []
    for rep in range(40):
        for M, N, wq, sc, x in data:
            idx = torch.empty(M, dtype=torch.int32, device="cuda")
            lg = torch.empty((M, N), dtype=torch.float32, device="cuda")
            if static:
                q.qmv_int2_argmax_static(wq, sc, x, idx, logits=lg)
            else:
                q.qmv_int2_argmax(wq, sc, x, idx=idx, logits=lg, want_maxval=False, workspace=ws)
            if rep % 8 == 0:
                outs.append((idx, lg))
    torch.cuda.synchronize()
    for idx, lg in outs:
        assert np.array_equal(idx.cpu().numpy(), first_max(lg))
    if ws is not None:
        assert int(ws.count_nonzero()) == 0  # counters and keys back at zero
