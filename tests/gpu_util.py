"""Host <-> device helpers for the GPU parity tests (storage-form numpy
arrays: float32 for f32, uint16 bit patterns for f16 / bf16, uint8 codes)."""
import sys

import numpy as np
import torch

TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to_dev(a, ft=None):
    a = np.ascontiguousarray(a)
    if ft is None or ft == "f32":
        return torch.from_numpy(a.copy()).cuda()
    return torch.from_numpy(a.view(np.int16).copy()).view(TORCH[ft]).cuda()


def from_dev(t):
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.int8, torch.uint8):
        return t.view(torch.uint8).numpy()
    return t.numpy()


def bits(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a.view(np.uint32)
    if a.dtype == np.int8:
        return a.view(np.uint8)
    return a


def assert_same(got, want, what):
    """Bit-for-bit equality (signed zeros included)."""
    g, w = bits(np.asarray(got)), bits(np.asarray(want))
    assert g.shape == w.shape, (what, g.shape, w.shape)
    bad = np.argwhere(g != w)
    if bad.size:
        idx = [tuple(i) for i in bad[:8]]
        msg = "%s: %d of %d differ; first %s; got %s want %s" % (
            what, len(bad), g.size, idx, [hex(int(g[i])) for i in idx], [hex(int(w[i])) for i in idx])
        raise AssertionError(msg)


def note(*a):
    print(*a, flush=True)
    sys.stdout.flush()
