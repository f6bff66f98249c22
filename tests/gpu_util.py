"""Helpers for the GPU parity tests: host numpy buffers (from synth) onto the
GPU in the binding's tensor conventions, and bit-level comparisons."""
import numpy as np
import torch


def dev(a, kind):
    """numpy host buffer -> contiguous GPU tensor.
    kind: 'u32' packed words -> int32, 'u8', 'f16' (uint16 bits), 'bf16' (uint16 bits)."""
    a = np.ascontiguousarray(a)
    if kind == "u32":
        t = torch.from_numpy(a.view(np.int32))
    elif kind == "u8":
        t = torch.from_numpy(a)
    elif kind == "f16":
        t = torch.from_numpy(a.view(np.float16))
    elif kind == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        raise ValueError(kind)
    return t.cuda()


def bits(t):
    """GPU/CPU tensor -> numpy array of its raw bits (uint32 for 4-byte, uint16 for 2-byte)."""
    t = t.detach().cpu().contiguous()
    if t.element_size() == 4:
        return t.view(torch.int32).numpy().view(np.uint32)
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def assert_bits_equal(got, want, what=""):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.flatnonzero(got.ravel() != want.ravel())
    if bad.size:
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} of {got.size} differ; first at flat index {i}: "
                             f"got {got.ravel()[i]:#x}, want {want.ravel()[i]:#x}")


def rel_l2(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))
