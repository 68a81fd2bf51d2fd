"""Seeded synthetic inputs for the Infini-attention segment kernel.

This module is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark. It holds workload shapes, seeded random draws and the bf16
storage format only; it contains none of the method's arithmetic.

Workloads (the pages' own measurements need trained weights and datasets,
so Gaussian activations of the same shapes stand in for them):

  tiny_fp32        B=1, H=2,  d=32,  L=16,   4 segments, fp32
  fwd_200m         B=8, H=12, d=64,  L=64,  16 segments, bf16   (16 rollouts x 64)
  fwd_llama3_8b    B=4, Hq=32/Hkv=8, d=128, L=2048, 16 segments, bf16
  stream_1m        B=1, H=32, d=64,  L=2048, 512 single-segment launches, bf16
  train_llama3_8b  B=8, H=32, d=128, L=64,  16 segments, bf16, fwd + bwd

Every tensor block is drawn from its own PCG64 stream keyed by
(workload id, tensor id, batch, head, segment), so any (b, h, s) block can be
regenerated on its own, without drawing the rest of the tensor.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# Tensor ids used in the seed key.
T_Q, T_K, T_V, T_BETA, T_DO, T_M0, T_Z0, T_DMS, T_DZS = range(9)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int               # workload id (first seed word)
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    seg_len: int
    segments: int          # segments per launch
    launches: int          # sequential launches that carry the state
    dtype: str             # "fp32" or "bf16"
    qkv_scale: float       # Q/K/V ~ N(0,1) * qkv_scale
    beta_dist: str         # "normal" or "uniform4"
    backward: bool = False

    @property
    def seq_len(self) -> int:
        """Tokens per launch."""
        return self.seg_len * self.segments

    @property
    def total_tokens(self) -> int:
        return self.seq_len * self.launches

    def shapes(self):
        B, Hq, Hkv, N, d = self.batch, self.q_heads, self.kv_heads, self.seq_len, self.head_dim
        return dict(Q=(B, Hq, N, d), K=(B, Hkv, N, d), V=(B, Hkv, N, d),
                    beta=(Hq,), M=(B, Hkv, d, d), z=(B, Hkv, d))

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 1, 2, 2, 32, 16, 4, 1, "fp32", 1.0, "normal", True),
    "fwd_200m": Workload("fwd_200m", 2, 8, 12, 12, 64, 64, 16, 1, "bf16", 1.0 / math.sqrt(64), "normal"),
    "fwd_llama3_8b": Workload("fwd_llama3_8b", 3, 4, 32, 8, 128, 2048, 16, 1, "bf16",
                              1.0 / math.sqrt(128), "normal"),
    "stream_1m": Workload("stream_1m", 4, 1, 32, 32, 64, 2048, 1, 512, "bf16", 1.0 / 8, "normal"),
    "train_llama3_8b": Workload("train_llama3_8b", 5, 8, 32, 32, 128, 64, 16, 1, "bf16",
                                1.0 / math.sqrt(128), "uniform4", True),
}


def rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


# ---------------------------------------------------------------- bf16 storage

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 with round-to-nearest-even; return uint16 bits.

    Inputs must be finite (NaN/Inf are not produced by the generators)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round freshly drawn float32 values to the workload's storage format.

    Returns float32 values that are exactly representable in `dtype`."""
    if dtype == "fp32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(x32))
    raise ValueError(dtype)


# ---------------------------------------------------------------- generators

def block(w: Workload, tensor: int, b: int, h: int, s: int, launch: int = 0,
          scale: float | None = None) -> np.ndarray:
    """One (seg_len, head_dim) block of Q, K, V or dO, in storage precision (as float32)."""
    sc = w.qkv_scale if scale is None else scale
    g = rng(w.wid, tensor, launch, b, h, s)
    x = g.standard_normal((w.seg_len, w.head_dim), dtype=np.float32) * np.float32(sc)
    return storage(x, w.dtype)


def tensor(w: Workload, tensor_id: int, launch: int = 0, heads: int | None = None,
           scale: float | None = None) -> np.ndarray:
    """A full [B, H, N, d] tensor of one launch, as float32 holding storage-precision values."""
    H = heads if heads is not None else (w.q_heads if tensor_id in (T_Q, T_DO) else w.kv_heads)
    out = np.empty((w.batch, H, w.seq_len, w.head_dim), dtype=np.float32)
    L = w.seg_len
    for b in range(w.batch):
        for h in range(H):
            for s in range(w.segments):
                out[b, h, s * L:(s + 1) * L] = block(w, tensor_id, b, h, s, launch, scale)
    return out


def qkv(w: Workload, launch: int = 0):
    return tensor(w, T_Q, launch), tensor(w, T_K, launch), tensor(w, T_V, launch)


def d_out(w: Workload, launch: int = 0) -> np.ndarray:
    """Upstream gradient dO ~ N(0, 1), in storage precision."""
    return tensor(w, T_DO, launch, heads=w.q_heads, scale=1.0)


def beta(w: Workload) -> np.ndarray:
    """Per-query-head gate parameter (float32)."""
    g = rng(w.wid, T_BETA)
    if w.beta_dist == "normal":
        return g.standard_normal(w.q_heads).astype(np.float32)
    if w.beta_dist == "uniform4":
        return g.uniform(-4.0, 4.0, w.q_heads).astype(np.float32)
    raise ValueError(w.beta_dist)


def random_state(w: Workload, tokens: int = 64, seed: int = 0):
    """A consistent nonzero carried state (M0, z0), built as if from `tokens`
    earlier tokens: keys and values drawn like the workload's, then passed
    through the caller-supplied feature map.  Returned as the raw prefix
    (K_pre, V_pre) so that the caller computes the state itself."""
    g = rng(w.wid, T_M0, seed)
    shp = (w.batch, w.kv_heads, tokens, w.head_dim)
    kp = g.standard_normal(shp, dtype=np.float32) * np.float32(w.qkv_scale)
    vp = g.standard_normal(shp, dtype=np.float32) * np.float32(w.qkv_scale)
    return storage(kp, w.dtype), storage(vp, w.dtype)


def upstream_state_grads(w: Workload, seed: int = 0):
    g = rng(w.wid, T_DMS, seed)
    dM = g.standard_normal(w.shapes()["M"]).astype(np.float32) * np.float32(1e-3)
    dz = g.standard_normal(w.shapes()["z"]).astype(np.float32) * np.float32(1e-3)
    return dM, dz
