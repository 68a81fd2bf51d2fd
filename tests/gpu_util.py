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
