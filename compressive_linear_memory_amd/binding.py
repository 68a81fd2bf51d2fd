"""ctypes binding of libinfini (argument marshalling only).

Every step of the computation runs in the HIP library; this module checks
tensor properties, allocates outputs and workspace with torch on the GPU and
passes raw device pointers plus torch's current stream.  There is no other
implementation to fall back to: if libinfini.so is missing or fails to load,
every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libinfini.so")

INFINI_FP32, INFINI_BF16 = 0, 1
_DTYPES = {torch.float32: INFINI_FP32, torch.bfloat16: INFINI_BF16}
FEATURE_MAPS = {"elu1": 0, "taylor2": 1}


def feature_dim(head_dim: int, feature_map: str = "elu1") -> int:
    """Rows of the memory M (features per key) for a feature map."""
    return head_dim if feature_map == "elu1" else 1 + head_dim + head_dim * head_dim


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_heads", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("seg_len", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("feature_map", ctypes.c_int32)]


class InfiniError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {lib().infini_status_string(code).decode()} (status {code})")
        self.code = code


_lib = None
_P = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    """Load libinfini.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        L.infini_status_string.restype = ctypes.c_char_p
        L.infini_status_string.argtypes = [ctypes.c_int]
        L.infini_version.restype = ctypes.c_int
        L.infini_version.argtypes = []
        for fn in ("infini_fwd_workspace_bytes", "infini_bwd_workspace_bytes", "infini_decode_workspace_bytes",
                   "infini_fwd_saved_bytes"):
            getattr(L, fn).restype = ctypes.c_size_t
            getattr(L, fn).argtypes = [ctypes.POINTER(Problem)]
        L.infini_attn_fwd.restype = ctypes.c_int
        L.infini_attn_fwd.argtypes = [ctypes.POINTER(Problem)] + [_P] * 11 + [ctypes.c_size_t, _P]
        L.infini_attn_bwd.restype = ctypes.c_int
        L.infini_attn_bwd.argtypes = [ctypes.POINTER(Problem)] + [_P] * 17 + [ctypes.c_size_t, _P]
        L.infini_attn_fwd_varlen.restype = ctypes.c_int
        L.infini_attn_fwd_varlen.argtypes = [ctypes.POINTER(Problem)] + [_P] * 12 + [ctypes.c_size_t, _P]
        L.infini_attn_bwd_varlen.restype = ctypes.c_int
        L.infini_attn_bwd_varlen.argtypes = [ctypes.POINTER(Problem)] + [_P] * 18 + [ctypes.c_size_t, _P]
        L.infini_attn_bwd_saved.restype = ctypes.c_int
        L.infini_attn_bwd_saved.argtypes = [ctypes.POINTER(Problem)] + [_P] * 20 + [ctypes.c_size_t, _P]
        L.infini_fwd_path.restype = ctypes.c_char_p
        L.infini_fwd_path.argtypes = [ctypes.POINTER(Problem)]
        L.infini_fwd_memory.restype = ctypes.c_int
        L.infini_fwd_memory.argtypes = [ctypes.POINTER(Problem)] + [_P] * 7 + [ctypes.c_size_t, _P]
        L.infini_fwd_attend.restype = ctypes.c_int
        L.infini_fwd_attend.argtypes = [ctypes.POINTER(Problem)] + [_P] * 7 + [ctypes.c_size_t, _P]
        L.infini_fwd_stream_workspace_bytes.restype = ctypes.c_size_t
        L.infini_fwd_stream_workspace_bytes.argtypes = [ctypes.POINTER(Problem), ctypes.c_int, ctypes.c_int]
        L.infini_fwd_stream.restype = ctypes.c_int
        L.infini_fwd_stream.argtypes = ([ctypes.POINTER(Problem), ctypes.c_int] + [_P] * 8 +
                                        [ctypes.c_size_t, ctypes.c_int, ctypes.c_int, _P, _P, _P])
        L.infini_decode.restype = ctypes.c_int
        L.infini_decode.argtypes = [ctypes.POINTER(Problem), ctypes.c_int32] + [_P] * 12 + [ctypes.c_size_t, _P]
        L.infini_decode_noalloc.restype = ctypes.c_int
        L.infini_decode_noalloc.argtypes = [ctypes.POINTER(Problem), ctypes.c_int32] + [_P] * 12
        _lib = L
    return _lib


def problem(q: torch.Tensor, k: torch.Tensor, seg_len: int, feature_map: str = "elu1") -> Problem:
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [batch, heads, seq_len, head_dim]")
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if feature_map not in FEATURE_MAPS:
        raise ValueError(f"unknown feature map {feature_map}")
    B, Hq, N, d = q.shape
    return Problem(B, Hq, k.shape[1], N, d, int(seg_len), _DTYPES[q.dtype], FEATURE_MAPS[feature_map])


def workspace_bytes(p: Problem, backward: bool = False) -> int:
    fn = lib().infini_bwd_workspace_bytes if backward else lib().infini_fwd_workspace_bytes
    return int(fn(ctypes.byref(p)))


def saved_bytes(p: Problem) -> int:
    """Bytes of the forward's saved row statistics (its lse output)."""
    return int(lib().infini_fwd_saved_bytes(ctypes.byref(p)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(name, t, dtype, shape, device):
    if t is None:
        return
    if t.device != device or t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name}: need contiguous {dtype} {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def attn_fwd(q, k, v, beta, seg_len, M0=None, z0=None, want_lse=False, out=None, ws=None, seq_lens=None,
             feature_map="elu1"):
    """O, M_S, z_S (and lse if want_lse) of one call; see include/infini.h.

    `out` may hold preallocated (O, M_S, z_S, lse) tensors and `ws` a uint8
    workspace tensor, so that a timed loop allocates nothing.  `seq_lens`
    (int32 [batch] on the device) makes it a variable-length batch
    (infini_attn_fwd_varlen).  `feature_map` "taylor2" selects the
    second-order Taylor map: the state then has 1 + d + d^2 rows."""
    p = problem(q, k, seg_len, feature_map)
    dev = q.device
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    nf = feature_dim(d, feature_map)
    for name, t, dt, shp in (("k", k, q.dtype, (B, Hkv, N, d)), ("v", v, q.dtype, (B, Hkv, N, d)),
                             ("beta", beta, torch.float32, (Hq,)),
                             ("M0", M0, torch.float32, (B, Hkv, nf, d)), ("z0", z0, torch.float32, (B, Hkv, nf))):
        _check(name, t, dt, shp, dev)
    _check("q", q, q.dtype, q.shape, dev)
    _check("seq_lens", seq_lens, torch.int32, (B,), dev)
    if out is None:
        O = torch.empty_like(q)
        M_S = torch.empty((B, Hkv, nf, d), dtype=torch.float32, device=dev)
        z_S = torch.empty((B, Hkv, nf), dtype=torch.float32, device=dev)
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev) if want_lse else None
    else:
        O, M_S, z_S, lse = out
        for name, t, dt, shp in (("O", O, q.dtype, q.shape), ("M_S", M_S, torch.float32, (B, Hkv, nf, d)),
                                 ("z_S", z_S, torch.float32, (B, Hkv, nf)), ("lse", lse, torch.float32, (B, Hq, N))):
            _check(name, t, dt, shp, dev)
    if ws is None:
        ws = torch.empty(max(workspace_bytes(p), 1), dtype=torch.uint8, device=dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(M0), _ptr(z0), _ptr(O), _ptr(M_S), _ptr(z_S), _ptr(lse),
            _ptr(ws), ws.numel(), _stream())
    if seq_lens is None:
        rc = lib().infini_attn_fwd(ctypes.byref(p), *args)
    else:
        rc = lib().infini_attn_fwd_varlen(ctypes.byref(p), _ptr(seq_lens), *args)
    if rc != 0:
        raise InfiniError(rc, "infini_attn_fwd" if seq_lens is None else "infini_attn_fwd_varlen")
    return (O, M_S, z_S, lse) if want_lse else (O, M_S, z_S)


def attn_bwd(q, k, v, beta, seg_len, dO, M0=None, z0=None, lse=None, dM_S=None, dz_S=None,
             want_state_grads=False, ws=None, out=None, seq_lens=None, state=None):
    """dQ, dK, dV, dbeta (and dM0, dz0 if want_state_grads); see include/infini.h.

    `out` may hold preallocated (dQ, dK, dV, dbeta, dM0, dz0) tensors (dM0 and
    dz0 None unless want_state_grads).  `seq_lens` (int32 [batch] on the
    device) makes it a variable-length batch (infini_attn_bwd_varlen).
    `state` = (M_S, z_S) returned by the forward for the same inputs calls
    infini_attn_bwd_saved, which does not rebuild that state."""
    p = problem(q, k, seg_len)
    dev = q.device
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    for name, t, dt, shp in (("k", k, q.dtype, (B, Hkv, N, d)), ("v", v, q.dtype, (B, Hkv, N, d)),
                             ("dO", dO, q.dtype, (B, Hq, N, d)), ("beta", beta, torch.float32, (Hq,)),
                             ("M0", M0, torch.float32, (B, Hkv, d, d)), ("z0", z0, torch.float32, (B, Hkv, d)),
                             ("lse", lse, torch.float32, (B, Hq, N)),
                             ("dM_S", dM_S, torch.float32, (B, Hkv, d, d)),
                             ("dz_S", dz_S, torch.float32, (B, Hkv, d)),
                             ("seq_lens", seq_lens, torch.int32, (B,))):
        _check(name, t, dt, shp, dev)
    M_S, z_S = state if state is not None else (None, None)
    if state is not None:
        _check("M_S", M_S, torch.float32, (B, Hkv, d, d), dev)
        _check("z_S", z_S, torch.float32, (B, Hkv, d), dev)
    if out is None:
        dQ = torch.empty_like(q)
        dK = torch.empty_like(k)
        dV = torch.empty_like(v)
        dbeta = torch.empty((Hq,), dtype=torch.float32, device=dev)
        dM0 = torch.empty((B, Hkv, d, d), dtype=torch.float32, device=dev) if want_state_grads else None
        dz0 = torch.empty((B, Hkv, d), dtype=torch.float32, device=dev) if want_state_grads else None
    else:
        dQ, dK, dV, dbeta, dM0, dz0 = out
        for name, t, dt, shp in (("dQ", dQ, q.dtype, q.shape), ("dK", dK, q.dtype, k.shape),
                                 ("dV", dV, q.dtype, v.shape), ("dbeta", dbeta, torch.float32, (Hq,)),
                                 ("dM0", dM0, torch.float32, (B, Hkv, d, d)),
                                 ("dz0", dz0, torch.float32, (B, Hkv, d))):
            _check(name, t, dt, shp, dev)
    if ws is None:
        ws = torch.empty(max(workspace_bytes(p, backward=True), 1), dtype=torch.uint8, device=dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(M0), _ptr(z0), _ptr(lse), _ptr(dO), _ptr(dM_S),
            _ptr(dz_S), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dbeta), _ptr(dM0), _ptr(dz0), _ptr(ws), ws.numel(),
            _stream())
    if state is not None:
        rc = lib().infini_attn_bwd_saved(ctypes.byref(p), _ptr(seq_lens), *args[:6], _ptr(M_S), _ptr(z_S), *args[6:])
        name = "infini_attn_bwd_saved"
    elif seq_lens is None:
        rc = lib().infini_attn_bwd(ctypes.byref(p), *args)
        name = "infini_attn_bwd"
    else:
        rc = lib().infini_attn_bwd_varlen(ctypes.byref(p), _ptr(seq_lens), *args)
        name = "infini_attn_bwd_varlen"
    if rc != 0:
        raise InfiniError(rc, name)
    if want_state_grads:
        return dQ, dK, dV, dbeta, dM0, dz0
    return dQ, dK, dV, dbeta


def fwd_memory(p: Problem, k, v, M0, z0, M_S, z_S, ws):
    """Phase 1 of the forward (memory path only) on preallocated buffers."""
    rc = lib().infini_fwd_memory(ctypes.byref(p), _ptr(k), _ptr(v), _ptr(M0), _ptr(z0), _ptr(M_S), _ptr(z_S),
                                 _ptr(ws), ws.numel(), _stream())
    if rc != 0:
        raise InfiniError(rc, "infini_fwd_memory")


def fwd_attend(p: Problem, q, k, v, beta, O, lse, ws):
    """Phase 2 of the forward (attention, retrieval, gate) on preallocated buffers."""
    rc = lib().infini_fwd_attend(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(O), _ptr(lse),
                                 _ptr(ws), ws.numel(), _stream())
    if rc != 0:
        raise InfiniError(rc, "infini_fwd_attend")


def _event_handle(ev):
    """Raw HIP event of a torch.cuda.Event (created lazily by torch: recorded
    once here if it does not exist yet)."""
    if not ev.cuda_event:
        ev.record()
    return ev.cuda_event


class StreamCalls:
    """Marshalled arguments of one infini_fwd_stream call: a batch of calls of
    shape `p` over the given per-call tensors, so that a loop that repeats the
    batch pays the marshalling once.  The tensors must stay alive."""

    def __init__(self, p: Problem, qs, ks, vs, beta, M, z, outs, ws, n_pipe, group, mem_stream, att_streams,
                 events):
        n = len(qs)
        if not (len(ks) == len(vs) == len(outs) == n) or n < 1:
            raise ValueError("qs, ks, vs, outs: one tensor per call")
        if len(att_streams) != n_pipe or len(events) != 2 * n_pipe:
            raise ValueError("need n_pipe attention streams and 2 * n_pipe events")
        arr = lambda ts: (_P * n)(*[t.data_ptr() for t in ts])
        self._keep = (arr(qs), arr(ks), arr(vs), arr(outs),
                      (_P * n_pipe)(*[s.cuda_stream for s in att_streams]),
                      (_P * (2 * n_pipe))(*[_event_handle(e) for e in events]))
        self.args = (ctypes.byref(p), n, self._keep[0], self._keep[1], self._keep[2], _ptr(beta), _ptr(M), _ptr(z),
                     self._keep[3], _ptr(ws), ws.numel(), n_pipe, group, _P(mem_stream.cuda_stream),
                     self._keep[4], self._keep[5])
        self._p = p

    def __call__(self):
        rc = lib().infini_fwd_stream(*self.args)
        if rc != 0:
            raise InfiniError(rc, "infini_fwd_stream")


def stream_workspace_bytes(p: Problem, n_pipe: int, group: int) -> int:
    return int(lib().infini_fwd_stream_workspace_bytes(ctypes.byref(p), n_pipe, group))


def fwd_stream(p: Problem, qs, ks, vs, beta, M, z, outs, ws, n_pipe, group, mem_stream, att_streams, events):
    """infini_fwd_stream (see include/infini.h): len(qs) chained calls of shape
    p in groups of `group`, the memory phases on mem_stream and each group's
    attention phases on att_streams; M, z hold the state and are updated in
    place."""
    StreamCalls(p, qs, ks, vs, beta, M, z, outs, ws, n_pipe, group, mem_stream, att_streams, events)()


def decode(q, k, v, beta, seg_len, pos, kcache, vcache, M=None, z=None, out=None, state_out=None, ws=None):
    """Streaming decode (see include/infini.h, infini_decode): T = q.shape[2]
    new tokens at positions pos.. of the current segment.  Writes the new K/V
    rows into kcache/vcache ([B, Hkv, seg_len, d]) and returns O [B, Hq, T, d];
    when pos + T == seg_len it also returns the state after the segment,
    (O, M_next, z_next)."""
    p = problem(q, k, seg_len)
    p.seq_len = q.shape[2]
    dev = q.device
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    for name, t, dt, shp in (("k", k, q.dtype, (B, Hkv, T, d)), ("v", v, q.dtype, (B, Hkv, T, d)),
                             ("beta", beta, torch.float32, (Hq,)),
                             ("kcache", kcache, q.dtype, (B, Hkv, seg_len, d)),
                             ("vcache", vcache, q.dtype, (B, Hkv, seg_len, d)),
                             ("M", M, torch.float32, (B, Hkv, d, d)), ("z", z, torch.float32, (B, Hkv, d))):
        _check(name, t, dt, shp, dev)
    _check("q", q, q.dtype, q.shape, dev)
    closes = pos + T == seg_len
    O = torch.empty_like(q) if out is None else out
    M_next = z_next = None
    if closes:
        if state_out is None:
            M_next = torch.empty((B, Hkv, d, d), dtype=torch.float32, device=dev)
            z_next = torch.empty((B, Hkv, d), dtype=torch.float32, device=dev)
        else:
            M_next, z_next = state_out
    if ws is None:
        ws = torch.empty(max(lib().infini_decode_workspace_bytes(ctypes.byref(p)), 1), dtype=torch.uint8,
                         device=dev)
    rc = lib().infini_decode(ctypes.byref(p), int(pos), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(kcache),
                             _ptr(vcache), _ptr(M), _ptr(z), _ptr(O), _ptr(M_next), _ptr(z_next), _ptr(ws),
                             ws.numel(), _stream())
    if rc != 0:
        raise InfiniError(rc, "infini_decode")
    return (O, M_next, z_next) if closes else O


def decode_noalloc(q, k, v, beta, seg_len, pos, kcache, vcache, M=None, z=None, out=None, state_out=None):
    """infini_decode_noalloc (see include/infini.h): infini_decode with the
    library's static per-device scratch instead of a workspace.  Outputs must
    be preallocated (out, and state_out when the call completes the segment)
    for the call to allocate nothing."""
    p = problem(q, k, seg_len)
    p.seq_len = q.shape[2]
    dev = q.device
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    for name, t, dt, shp in (("k", k, q.dtype, (B, Hkv, T, d)), ("v", v, q.dtype, (B, Hkv, T, d)),
                             ("beta", beta, torch.float32, (Hq,)),
                             ("kcache", kcache, q.dtype, (B, Hkv, seg_len, d)),
                             ("vcache", vcache, q.dtype, (B, Hkv, seg_len, d)),
                             ("M", M, torch.float32, (B, Hkv, d, d)), ("z", z, torch.float32, (B, Hkv, d)),
                             ("out", out, q.dtype, (B, Hq, T, d))):
        _check(name, t, dt, shp, dev)
    _check("q", q, q.dtype, q.shape, dev)
    closes = pos + T == seg_len
    O = torch.empty_like(q) if out is None else out
    M_next = z_next = None
    if closes:
        if state_out is None:
            M_next = torch.empty((B, Hkv, d, d), dtype=torch.float32, device=dev)
            z_next = torch.empty((B, Hkv, d), dtype=torch.float32, device=dev)
        else:
            M_next, z_next = state_out
    rc = lib().infini_decode_noalloc(ctypes.byref(p), int(pos), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                     _ptr(kcache), _ptr(vcache), _ptr(M), _ptr(z), _ptr(O), _ptr(M_next),
                                     _ptr(z_next), _stream())
    if rc != 0:
        raise InfiniError(rc, "infini_decode_noalloc")
    return (O, M_next, z_next) if closes else O


def fwd_path(p: Problem) -> str:
    """Kernel family the forward runs for this problem."""
    r = lib().infini_fwd_path(ctypes.byref(p))
    return r.decode() if r else ""
