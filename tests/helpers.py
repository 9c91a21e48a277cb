"""Small helpers shared by the GPU tests (no method arithmetic here)."""

import numpy as np


def bits_u16(t):
    """A bf16 torch tensor's bit patterns as a numpy uint16 array (CPU copy)."""
    import torch

    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def host_array(t):
    """CPU numpy view of a head tensor in the form the oracle takes."""
    import torch

    if t.dtype == torch.bfloat16:
        return bits_u16(t)
    return t.detach().cpu().numpy()


def same_bits(a, b):
    """Bitwise equality of two fp32 tensors (NaN payloads included)."""
    import torch

    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


def rel_err(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    denom = np.maximum(np.abs(want), 1e-30)
    r = np.abs(got - want) / denom
    r[(got == 0) & (want == 0)] = 0.0
    return r


def say(*args):
    print(*args, flush=True)
