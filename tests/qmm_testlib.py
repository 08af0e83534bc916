"""Helpers for the GPU parity tests: oracle-side input preparation, device
upload and the tolerance check.  Every expected value comes from the oracle
package; every input from the synth package (through the oracle quantizer
where the inputs are packed weights)."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import synth

# Tolerance of the quantized matmuls against the float64 oracle: relative L2
# error of the whole output and largest absolute error (fp32 accumulation).
REL_L2 = 1e-3
MAX_ABS = 1e-2


def say(*msg):
    """Name the case on stdout before a GPU step (flushed, so a crash still
    leaves it behind)."""
    print("[case]", *msg, flush=True)
    sys.stdout.flush()


def dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def host(t, dtype=None):
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def quantized(key, n, k, bits):
    """Seeded weight -> oracle quantization -> (w_f32, codes, words, s, b)."""
    w = synth.draw_weight(key, n, k)
    codes, s, b = oracle.quantize(w, bits)
    return w, codes, oracle.pack(codes, bits), s, b


def rel_l2(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


def assert_close(got, want, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), what
    r = rel_l2(got, want)
    m = float(np.max(np.abs(got - want))) if got.size else 0.0
    assert r <= REL_L2 and m <= MAX_ABS, f"{what}: rel_l2={r:.3e} max_abs={m:.3e}"
    return r, m


# Guard bands: an output written into the middle of a larger buffer whose
# every byte (the output region included) starts as a sentinel.  A kernel
# that writes past either end of its output changes a sentinel byte.
GUARD_BYTES = 4096
SENTINEL = 0xA5


class Guarded:
    """A device tensor of `shape` and `dtype` with GUARD_BYTES of sentinel
    bytes on either side (the tensor itself starts filled with sentinels
    too, so a kernel that leaves part of it unwritten is also caught by the
    parity check that follows)."""

    def __init__(self, shape, dtype):
        import torch
        self.shape = tuple(shape)
        numel = 1
        for d in self.shape:
            numel *= d
        esz = torch.empty((), dtype=dtype).element_size()
        self.pad = GUARD_BYTES // esz
        self.nbytes = numel * esz
        self.buf = torch.empty(2 * self.pad + numel, dtype=dtype, device="cuda")
        self.buf.view(torch.uint8).fill_(SENTINEL)
        self.t = self.buf[self.pad:self.pad + numel].view(self.shape)

    def intact(self) -> bool:
        u8 = self.buf.view(-1).view(__import__("torch").uint8)
        head = u8[:GUARD_BYTES]
        tail = u8[GUARD_BYTES + self.nbytes:]
        return bool((head == SENTINEL).all()) and bool((tail == SENTINEL).all())

    def check(self, what=""):
        assert self.intact(), f"{what}: a write landed outside the output's {self.shape} region"
