"""Guard bands around GPU output buffers.

An output tensor is carved from the middle of a larger allocation whose
whole extent is first filled with the byte 0xA5.  After a call, the bands
before and after the tensor must still hold that byte, so a kernel that
writes outside its output (or past its workspace) is caught.  The tensor
itself starts as garbage, so every element a call claims to produce must
be written for the comparisons that follow to pass.
"""
from __future__ import annotations

import math

import torch

PAD_BYTES = 4096
FILL = 0xA5


class Guarded:
    def __init__(self, shape, dtype, device="cuda"):
        esize = torch.empty((), dtype=dtype).element_size()
        self.pad = PAD_BYTES // esize
        n = int(math.prod(shape))
        self.buf = torch.empty(n + 2 * self.pad, dtype=dtype, device=device)
        self.buf.view(torch.uint8).fill_(FILL)
        self.t = self.buf[self.pad:self.pad + n].view(tuple(shape))
        self.pad_bytes = self.pad * esize

    def check(self, name: str = "buffer"):
        raw = self.buf.view(torch.uint8)
        head = raw[:self.pad_bytes]
        tail = raw[raw.numel() - self.pad_bytes:]
        assert bool((head == FILL).all()), f"{name}: write before the start of the buffer"
        assert bool((tail == FILL).all()), f"{name}: write past the end of the buffer"


def guarded(shape, dtype, device="cuda"):
    g = Guarded(shape, dtype, device)
    return g.t, g


def check_all(*pairs):
    for name, g in pairs:
        if g is not None:
            g.check(name)
