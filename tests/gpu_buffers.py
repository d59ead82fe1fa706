"""Device buffers for the GPU parity tests: NaN-poisoned outputs inside
canary guard bands, and inputs placed at chosen offsets from an aligned
boundary."""
import numpy as np
import torch

from parity import bf16_bits, to_dev

DEV = "cuda:0"
GUARD = 1024                      # elements of guard band on each side
CANARY16 = 0x5A5A
TDT = {0: torch.float32, 1: torch.bfloat16}


class Guarded:
    """A NaN-filled device tensor of `shape` inside canary guard bands,
    optionally starting `offset` elements past a 256-byte boundary."""

    def __init__(self, shape, dtype, offset=0):
        n = int(np.prod(shape))
        self.dtype, self.shape, self.n, self.off = dtype, shape, n, GUARD + offset
        self.buf = torch.empty(n + 2 * GUARD + offset + 16, dtype=dtype, device=DEV)
        raw = self.buf.view(torch.int16) if dtype == torch.bfloat16 else self.buf.view(torch.int32)
        raw.fill_(CANARY16 if dtype == torch.bfloat16 else 0x5A5A5A5A)
        self.t = self.buf[self.off:self.off + n].view(shape)
        self.t.fill_(float("nan") if dtype.is_floating_point else -7)

    def canaries_intact(self):
        raw = self.buf.view(torch.int16) if self.dtype == torch.bfloat16 else self.buf.view(torch.int32)
        pat = CANARY16 if self.dtype == torch.bfloat16 else 0x5A5A5A5A
        lo = raw[:self.off]
        hi = raw[self.off + self.n:]
        return bool((lo == pat).all()) and bool((hi == pat).all())


def upload(a, offset=0):
    """Copy a host array into a fresh device buffer starting `offset` elements
    past an aligned boundary (offset 0 gives a 256-byte aligned tensor)."""
    t = to_dev(a)
    if offset == 0:
        return t
    flat = torch.empty(t.numel() + offset + 16, dtype=t.dtype, device=DEV)
    view = flat[offset:offset + t.numel()].view(t.shape)
    view.copy_(t)
    return view


def host(t):
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.cpu().numpy()
