"""Helpers for GPU parity tests: device transfer and oracle comparison."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

TOL = {"fp32": 1e-4, "bf16": 2e-2}


def torch_dtype(dtype):
    import torch
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[dtype]


def dev(x, dtype="fp32"):
    """Host float32 array (exactly representable in dtype) -> device tensor of dtype."""
    import torch
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")
    return t.to(torch_dtype(dtype)).contiguous()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(x - ref)) / den) if den > 0 else float(np.max(np.abs(x)))


def log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ output canaries
#
# Every output a parity case checks lives inside a larger buffer whose guard
# bands before and after it hold a fixed NaN bit pattern.  After the call the
# bands must be untouched (no write past either end), and the output itself
# must hold no canary word (every element was written) - an unwritten element
# would also read as NaN and fail the numeric comparison.

GUARD_BYTES = 4096           # per side; a multiple of 16 keeps the view 16-byte aligned
_CANARY = {"float32": 0x7FC0A5A5, "bfloat16": 0x7FA5}


class Guarded:
    """A tensor view of `shape` inside a canary-filled buffer."""

    def __init__(self, shape, dtype):
        import torch
        self.dtype = dtype
        es = torch.empty((), dtype=dtype).element_size()
        self.g = GUARD_BYTES // es
        self.n = int(np.prod(shape)) if len(shape) else 1
        self.buf = torch.empty(self.n + 2 * self.g, dtype=dtype, device="cuda")
        self._ints().fill_(self._word())
        self.t = self.buf[self.g:self.g + self.n].view(shape)

    def _word(self):
        import torch
        w = _CANARY[str(self.dtype).replace("torch.", "")]
        return w - (1 << 32) if self.dtype == torch.float32 and w >= 1 << 31 else w

    def _ints(self):
        import torch
        return self.buf.view(torch.int32 if self.dtype == torch.float32 else torch.int16)

    def check(self, name):
        ints = self._ints()
        w = self._word()
        lo, hi = ints[:self.g], ints[self.g + self.n:]
        assert bool((lo == w).all()), f"{name}: write before the start of the output"
        assert bool((hi == w).all()), f"{name}: write past the end of the output"
        assert not bool((ints[self.g:self.g + self.n] == w).any()), f"{name}: output element left unwritten"


def guarded(shape, dtype):
    return Guarded(tuple(shape), dtype)
