"""GPU parity: the HIP library against the fp64 CPU oracle, element by element.

Tolerance: normwise max relative error ||x - ref||_inf / ||ref||_inf per output
tensor, 1e-4 for fp32 problems and 2e-2 for bf16 problems.
"""
import os

import numpy as np
import pytest

import oracle as O
from compressive_linear_memory_amd import inputs as I
from gpu_util import TOL, dev, guarded, host, log, rel

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from compressive_linear_memory_amd import binding
    binding.lib()


def B():
    from compressive_linear_memory_amd import binding
    return binding


def rnd(shape, seed, scale, dtype):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * np.float32(scale)
    return I.storage(x, dtype)


def make(Bn, Hq, Hkv, N, d, dtype, seed, scale=None, with_state=False):
    sc = (1.0 / np.sqrt(d)) if scale is None else scale
    Q = rnd((Bn, Hq, N, d), seed, sc, dtype)
    K = rnd((Bn, Hkv, N, d), seed + 1, sc, dtype)
    V = rnd((Bn, Hkv, N, d), seed + 2, sc, dtype)
    beta = np.random.default_rng(seed + 3).standard_normal(Hq).astype(np.float32)
    M0 = z0 = None
    if with_state:
        Kp = rnd((Bn, Hkv, 48, d), seed + 4, sc, dtype)
        Vp = rnd((Bn, Hkv, 48, d), seed + 5, sc, dtype)
        _, _, M0, z0 = O.state_sweep(Kp, Vp, 48)
        M0, z0 = M0.astype(np.float32), z0.astype(np.float32)
    return Q, K, V, beta, M0, z0


def run_fwd(Q, K, V, beta, L, M0, z0, dtype, want_lse=False, lens=None):
    """One forward call whose outputs sit inside canary guard bands; the
    bands are checked before the outputs are returned."""
    from gpu_util import torch_dtype
    Bn, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    td = torch_dtype(dtype)
    gs = [guarded(Q.shape, td), guarded((Bn, Hkv, d, d), torch.float32), guarded((Bn, Hkv, d), torch.float32)]
    if want_lse:
        gs.append(guarded((Bn, Hq, N), torch.float32))
    out = tuple(x.t for x in gs) + ((None,) if not want_lse else ())
    r = B().attn_fwd(dev(Q, dtype), dev(K, dtype), dev(V, dtype), dev(beta), L,
                     dev(M0), dev(z0), want_lse=want_lse, out=out, seq_lens=dev_lens(lens))
    torch.cuda.synchronize()
    for name, x in zip(("O", "M_S", "z_S", "lse"), gs):
        x.check(name)
    return r


def dev_lens(lens):
    return None if lens is None else torch.tensor(np.asarray(lens, dtype=np.int32), device="cuda")


def check_fwd(Q, K, V, beta, L, M0, z0, dtype, tag="", lens=None):
    log(f"fwd {tag} Q{Q.shape} K{K.shape} L={L} {dtype} state={M0 is not None} lens={lens}")
    o, M, z = run_fwd(Q, K, V, beta, L, M0, z0, dtype, lens=lens)
    ro, rM, rz = O.forward(Q, K, V, beta, L, M0, z0, lens=None if lens is None else np.clip(lens, 0, Q.shape[2]))
    eo, eM, ez = rel(host(o), ro), rel(host(M), rM), rel(host(z), rz)
    log(f"   err O {eo:.2e} M {eM:.2e} z {ez:.2e}")
    tol = TOL[dtype]
    assert eo < tol and eM < tol and ez < tol, (eo, eM, ez)
    return o, M, z


# ------------------------------------------------------------------ fp32 workload

def test_tiny_fp32_forward():
    w = I.WORKLOADS["tiny_fp32"]
    Q, K, V = I.qkv(w)
    check_fwd(Q, K, V, I.beta(w), w.seg_len, None, None, "fp32", "tiny_fp32")


def _check_bwd(Q, K, V, beta, L, M0, z0, dO, dMS, dzS, dtype, tag="", lse=None, lens=None, saved=None):
    """Backward through the C ABI against the oracle; `saved` = the forward's
    (M_S, z_S) on the device routes the call through infini_attn_bwd_saved.
    Returns the gradients (device tensors)."""
    log(f"bwd {tag} Q{Q.shape} K{K.shape} L={L} {dtype} state={M0 is not None} dstate={dMS is not None} "
        f"lse={lse is not None} saved={saved is not None}")
    from gpu_util import torch_dtype
    Bn, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    td = torch_dtype(dtype)
    gs = [guarded(Q.shape, td), guarded(K.shape, td), guarded(V.shape, td), guarded((Hq,), torch.float32),
          guarded((Bn, Hkv, d, d), torch.float32), guarded((Bn, Hkv, d), torch.float32)]
    g = B().attn_bwd(dev(Q, dtype), dev(K, dtype), dev(V, dtype), dev(beta), L, dev(dO, dtype),
                     dev(M0), dev(z0), dev(lse), dev(dMS), dev(dzS), want_state_grads=True,
                     out=tuple(x.t for x in gs), seq_lens=dev_lens(lens), state=saved)
    torch.cuda.synchronize()
    for name, x in zip(("dQ", "dK", "dV", "dbeta", "dM0", "dz0"), gs):
        x.check(name)
    ref = O.backward(Q, K, V, beta, L, dO, M0, z0, dMS, dzS, lens=lens)
    errs = {}
    for name, t in zip(("dQ", "dK", "dV", "dbeta", "dM0", "dz0"), g):
        errs[name] = rel(host(t), ref[name])
    log("   " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    tol = TOL[dtype]
    assert all(v < tol for v in errs.values()), errs
    return g


def test_tiny_fp32_backward():
    w = I.WORKLOADS["tiny_fp32"]
    Q, K, V = I.qkv(w)
    _check_bwd(Q, K, V, I.beta(w), w.seg_len, None, None, I.d_out(w), None, None, "fp32", "tiny_fp32")


def test_tiny_fp32_backward_with_state_and_upstream_state_grads():
    w = I.WORKLOADS["tiny_fp32"]
    Q, K, V = I.qkv(w)
    Kp, Vp = I.random_state(w, tokens=40)
    _, _, M0, z0 = O.state_sweep(Kp, Vp, 40)
    dMS, dzS = I.upstream_state_grads(w)
    _check_bwd(Q, K, V, I.beta(w), w.seg_len, M0.astype(np.float32), z0.astype(np.float32),
               I.d_out(w), dMS, dzS, "fp32", "tiny_fp32+state")


# ------------------------------------------------------------------ shape sweep

FWD_CASES = [
    # B, Hq, Hkv, N, d, L, dtype, state
    (1, 2, 2, 64, 32, 16, "fp32", True),
    (2, 4, 2, 96, 64, 32, "fp32", False),
    (1, 4, 1, 120, 128, 40, "fp32", True),     # ragged row and key tiles
    (2, 3, 3, 9, 32, 3, "fp32", True),         # tiny segments
    (1, 2, 2, 8, 64, 1, "fp32", False),        # one token per segment
    (1, 2, 2, 300, 64, 300, "fp32", True),     # one long segment, ragged tiles
    (2, 8, 2, 256, 128, 64, "bf16", True),
    (1, 6, 3, 390, 64, 130, "bf16", False),
    (1, 4, 4, 128, 32, 128, "bf16", True),
    # bf16 head_dim 64 / 128 take the matrix-core path: tails of query and key tiles
    (1, 2, 2, 8, 64, 1, "bf16", True),
    (2, 4, 2, 48, 128, 16, "bf16", False),
    (1, 4, 1, 200, 128, 100, "bf16", True),
    (1, 2, 2, 600, 64, 300, "bf16", True),
    (1, 8, 2, 1024, 128, 512, "bf16", True),
    (1, 4, 2, 1540, 128, 770, "bf16", True),   # 2-row last query tile
    (1, 2, 1, 1000, 64, 1000, "bf16", False),
    # sequence not a multiple of seg_len: the last segment is shorter
    (1, 2, 2, 70, 32, 16, "fp32", True),       # generic path, 6-token tail
    (1, 3, 3, 101, 64, 48, "fp32", False),
    (1, 4, 2, 1000, 128, 384, "bf16", True),   # long path, 232-token tail
    (1, 2, 2, 300, 64, 128, "bf16", False),    # long path, 44-token tail
    (1, 2, 1, 2049, 128, 1024, "bf16", True),  # long path, 1-token tail
    (2, 4, 2, 100, 64, 64, "bf16", True),      # fused short path, 36-token tail
    (1, 4, 4, 70, 128, 16, "bf16", True),      # fused short path, 6-token tail
    (1, 2, 2, 9, 64, 8, "bf16", False),        # fused short path, 1-token tail
    # wide query groups (query heads per K/V head)
    (1, 16, 2, 128, 128, 64, "bf16", True),    # fused short path, 8 heads per K/V head
    (1, 32, 2, 96, 64, 32, "bf16", True),      # fused short path, 16 heads per K/V head
    (1, 16, 1, 300, 128, 128, "bf16", True),   # long path, 16 heads per K/V head
]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "-".join(map(str, c)))
def test_forward_shapes(case):
    Bn, Hq, Hkv, N, d, L, dtype, st = case
    Q, K, V, beta, M0, z0 = make(Bn, Hq, Hkv, N, d, dtype, seed=N + d, with_state=st)
    check_fwd(Q, K, V, beta, L, M0, z0, dtype)


BWD_CASES = [
    (1, 2, 2, 64, 32, 16, "fp32", True),
    (1, 4, 2, 96, 64, 48, "fp32", True),
    (1, 2, 1, 80, 128, 40, "fp32", False),
    (2, 2, 2, 12, 32, 3, "fp32", True),
    (2, 4, 2, 256, 128, 64, "bf16", True),
    (1, 3, 3, 130, 64, 65, "bf16", False),
    # bf16 head_dim 64/128 with seg_len <= 64 take the fused matrix-core backward
    (1, 2, 2, 192, 64, 64, "bf16", True),
    (2, 8, 2, 96, 128, 48, "bf16", True),      # ragged segment tile, 4 heads per K/V head
    (1, 2, 1, 40, 128, 8, "bf16", False),
    (1, 2, 2, 5, 64, 1, "bf16", True),
    # sequence not a multiple of seg_len
    (1, 2, 2, 70, 32, 16, "fp32", True),       # generic backward, 6-token tail
    (1, 3, 3, 150, 64, 65, "bf16", True),      # generic backward (bf16, seg_len > 64), 20-token tail
    (2, 4, 2, 100, 64, 64, "bf16", True),      # fused short backward, 36-token tail
    (1, 4, 4, 70, 128, 16, "bf16", True),      # fused short backward, 6-token tail
    (1, 2, 1, 41, 128, 8, "bf16", False),      # fused short backward, 1-token tail
    # wide query groups: 16 heads per K/V head is the fused backward's limit,
    # 17 takes the generic backward
    (1, 16, 1, 128, 128, 64, "bf16", True),
    (1, 34, 2, 64, 64, 32, "bf16", False),
    # bf16 segments longer than 64: matrix-core query side
    (1, 4, 2, 520, 128, 256, "bf16", True),    # 3 segments, 8-token tail, 2 heads per K/V head
    (2, 2, 2, 384, 64, 128, "bf16", False),    # 3 full segments
    (1, 8, 2, 700, 128, 300, "bf16", True),    # seg_len not a multiple of 64, 100-token tail
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "-".join(map(str, c)))
def test_backward_shapes(case):
    Bn, Hq, Hkv, N, d, L, dtype, st = case
    Q, K, V, beta, M0, z0 = make(Bn, Hq, Hkv, N, d, dtype, seed=3 * N + d, with_state=st)
    dO = rnd(Q.shape, 99, 1.0, dtype)
    dMS = dzS = None
    if st:
        dMS = np.random.default_rng(7).standard_normal(M0.shape).astype(np.float32) * 1e-2
        dzS = np.random.default_rng(8).standard_normal(z0.shape).astype(np.float32) * 1e-2
    _check_bwd(Q, K, V, beta, L, M0, z0, dO, dMS, dzS, dtype)



@pytest.mark.parametrize("case", BWD_CASES[::2], ids=lambda c: "-".join(map(str, c)))
def test_backward_with_saved_lse(case):
    """The backward given the row log-sum-exp (here the oracle's, as float32)
    forms the probabilities from it directly; the gradients still match."""
    Bn, Hq, Hkv, N, d, L, dtype, st = case
    Q, K, V, beta, M0, z0 = make(Bn, Hq, Hkv, N, d, dtype, seed=3 * N + d, with_state=st)
    dO = rnd(Q.shape, 99, 1.0, dtype)
    lse = O.forward(Q, K, V, beta, L, M0, z0, want_lse=True)[3].astype(np.float32)
    _check_bwd(Q, K, V, beta, L, M0, z0, dO, None, None, dtype, "saved lse", lse=lse)


def test_saved_bytes_is_the_lse_size():
    p = B().Problem(2, 8, 2, 1000, 128, 384, 1)
    assert B().saved_bytes(p) == 2 * 8 * 1000 * 4


def _random_cases(n, seed):
    """Seeded shapes across every kernel path: head dims 32/64/128, fp32 and
    bf16, seg_len from 1 past the sequence length, ragged tails, GQA."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = int(rng.choice([32, 64, 128]))
        dtype = "fp32" if d == 32 or rng.random() < 0.25 else "bf16"
        Hkv = int(rng.integers(1, 4))
        Hq = Hkv * int(rng.choice([1, 2, 4, 8]))
        N = int(rng.integers(1, 400))
        L = int(rng.choice([1, 7, 16, 48, 64, 65, 128, 300, 512]))
        out.append((int(rng.integers(1, 3)), Hq, Hkv, N, d, L, dtype, bool(rng.random() < 0.5)))
    return out


@pytest.mark.parametrize("case", _random_cases(16, 2026), ids=lambda c: "-".join(map(str, c)))
def test_random_shapes_forward_and_backward(case):
    """Forward and backward of seeded random shapes against the oracle."""
    Bn, Hq, Hkv, N, d, L, dtype, st = case
    Q, K, V, beta, M0, z0 = make(Bn, Hq, Hkv, N, d, dtype, seed=N * 7 + d, with_state=st)
    check_fwd(Q, K, V, beta, L, M0, z0, dtype, "random")
    dO = rnd(Q.shape, N + 5, 1.0, dtype)
    dMS = dzS = None
    if st:
        dMS = np.random.default_rng(N).standard_normal(M0.shape).astype(np.float32) * 1e-2
        dzS = np.random.default_rng(N + 1).standard_normal(z0.shape).astype(np.float32) * 1e-2
    _check_bwd(Q, K, V, beta, L, M0, z0, dO, dMS, dzS, dtype, "random")


@pytest.mark.parametrize("case", [
    (1, 2, 2, 64, 32, 16, "fp32"),           # generic path
    (1, 4, 2, 600, 64, 256, "bf16"),         # long path, ragged tail
    (1, 16, 2, 512, 64, 256, "bf16"),        # long path, 8 query heads per K/V head
    (2, 4, 2, 100, 128, 64, "bf16"),         # fused short path, ragged tail
], ids=lambda c: "-".join(map(str, c)))
def test_forward_row_logsumexp(case):
    """The optional per-row log-sum-exp output (natural log of the causal
    softmax normaliser of the scaled scores) against the oracle's."""
    Bn, Hq, Hkv, N, d, L, dtype = case
    Q, K, V, beta, M0, z0 = make(Bn, Hq, Hkv, N, d, dtype, seed=5 * N + d, with_state=True)
    o, M, z, lse = run_fwd(Q, K, V, beta, L, M0, z0, dtype, want_lse=True)
    torch.cuda.synchronize()
    ro, rM, rz, rl = O.forward(Q, K, V, beta, L, M0, z0, want_lse=True)
    el = rel(host(lse), rl)
    log(f"   lse {case}: err {el:.2e} O {rel(host(o), ro):.2e}")
    assert el < TOL[dtype] and rel(host(o), ro) < TOL[dtype]

# ------------------------------------------------------------------ peaked softmax
#
# The workloads' inputs (Q, K ~ N(0,1)/sqrt(d)) give scaled scores with a
# standard deviation near 1/sqrt(d): the softmax is almost uniform and no key
# tile's maximum ever moves far past the first tile's.  These cases draw
# Q, K ~ N(0,1) * c (c = 1 or 4: score standard deviation c^2), and some let
# the key norms grow along the segment so that a later 64-key tile's maximum
# beats the first tile's by more than the attention kernel's lazy-rescale
# slack (2^8 in the base-2 domain); that the threshold is crossed is asserted
# on the CPU from the exact scores.  Softmax with the max subtracted and the
# online merge across key tiles and key chunks ([ASM] "방법론") are then
# exercised on every bf16 kernel.

RESCALE_SLACK_LOG2 = 8.0


def make_peaked(Bn, Hq, Hkv, N, d, L, dtype, seed, c, grow, with_state=False):
    """Q, K ~ N(0,1) c; V ~ N(0,1)/sqrt(d).  grow: key row j of every segment
    scaled by 1 + 3 (j mod L) / L before rounding to the storage type."""
    g = np.random.default_rng(seed)
    Q = I.storage(g.standard_normal((Bn, Hq, N, d)).astype(np.float32) * np.float32(c), dtype)
    K = g.standard_normal((Bn, Hkv, N, d)).astype(np.float32) * np.float32(c)
    if grow:
        pos = (np.arange(N) % L).astype(np.float32)
        K = K * (1.0 + 3.0 * pos / L)[None, None, :, None].astype(np.float32)
    K = I.storage(K, dtype)
    V = I.storage(g.standard_normal((Bn, Hkv, N, d)).astype(np.float32) / np.float32(np.sqrt(d)), dtype)
    beta = g.standard_normal(Hq).astype(np.float32)
    M0 = z0 = None
    if with_state:
        Kp = I.storage(g.standard_normal((Bn, Hkv, 48, d)).astype(np.float32) * np.float32(c), dtype)
        Vp = I.storage(g.standard_normal((Bn, Hkv, 48, d)).astype(np.float32) / np.float32(np.sqrt(d)), dtype)
        _, _, M0, z0 = O.state_sweep(Kp, Vp, 48)
        M0, z0 = M0.astype(np.float32), z0.astype(np.float32)
    return Q, K, V, beta, M0, z0


def rescale_events(Q, K, L, tile=64):
    """Rows (over every batch, query head, segment) at which a later key tile's
    maximum base-2 scaled score exceeds the running reference by more than the
    slack, replaying the attention kernel's lazy rule per row: the reference
    starts at the first tile's maximum and moves to a tile's maximum only when
    that exceeds it by more than the slack."""
    Bn, Hq, N, d = Q.shape
    G = Hq // K.shape[1]
    c = np.log2(np.e) / np.sqrt(d)
    events = 0
    for b in range(Bn):
        for h in range(Hq):
            for s0 in range(0, N, L):
                n = min(L, N - s0)
                S = (Q[b, h, s0:s0 + n].astype(np.float64) @ K[b, h // G, s0:s0 + n].astype(np.float64).T) * c
                S[np.triu_indices(n, 1)] = -np.inf
                for i in range(n):
                    m = S[i, :tile].max()
                    for t0 in range(tile, i + 1, tile):
                        mt = S[i, t0:t0 + tile].max()
                        if mt > m + RESCALE_SLACK_LOG2:
                            events += 1
                            m = mt
    return events


PEAKED_FWD = [
    # B, Hq, Hkv, N, d, L, dtype, c, grow, state, path
    (1, 4, 2, 600, 128, 256, "bf16", 1.0, True, True, "mfma_bf16"),      # GQA, 88-token tail
    (1, 4, 2, 600, 64, 300, "bf16", 1.0, True, False, "mfma_bf16"),
    (1, 2, 1, 520, 128, 520, "bf16", 4.0, False, True, "mfma_bf16"),     # c = 4, ragged key tile
    (1, 4, 4, 330, 64, 160, "bf16", 4.0, True, True, "mfma_bf16"),
    (2, 4, 2, 192, 128, 64, "bf16", 4.0, False, True, "mfma_bf16_short"),
    (1, 2, 2, 130, 64, 64, "bf16", 1.0, True, False, "mfma_bf16_short"),  # 2-token tail
    (1, 8, 2, 100, 128, 40, "bf16", 4.0, True, True, "mfma_bf16_short"),
    (1, 4, 2, 200, 64, 100, "fp32", 4.0, False, True, "generic_fp32"),
    (1, 2, 2, 300, 32, 150, "bf16", 1.0, True, True, "generic_fp32"),
    (1, 2, 1, 260, 128, 260, "fp32", 1.0, True, False, "generic_fp32"),
]


@pytest.mark.parametrize("case", PEAKED_FWD, ids=lambda c: "-".join(map(str, c)))
def test_forward_peaked_softmax(case):
    Bn, Hq, Hkv, N, d, L, dtype, c, grow, st, path = case
    Q, K, V, beta, M0, z0 = make_peaked(Bn, Hq, Hkv, N, d, L, dtype, 1000 + N + d, c, grow, st)
    q, k = dev(Q, dtype), dev(K, dtype)
    assert B().fwd_path(B().problem(q, k, L)) == path
    if L > 64:
        ev = rescale_events(Q, K, L)
        log(f"   rows with a lazy rescale after the first key tile: {ev}")
        assert ev > 0, "case does not cross the rescale threshold"
    check_fwd(Q, K, V, beta, L, M0, z0, dtype, f"peaked c={c} grow={grow}")


PEAKED_BWD = [
    # B, Hq, Hkv, N, d, L, dtype, c, grow, state
    (2, 4, 2, 192, 128, 64, "bf16", 4.0, False, True),     # fused short backward
    (1, 2, 2, 130, 64, 64, "bf16", 1.0, True, True),
    (1, 8, 2, 100, 128, 40, "bf16", 4.0, True, False),
    (1, 2, 2, 300, 64, 150, "bf16", 4.0, True, True),      # long-segment matrix-core backward
    (1, 4, 2, 520, 128, 256, "bf16", 4.0, True, True),     # long-segment, head_dim 128, 8-token tail
    (1, 4, 2, 200, 64, 100, "fp32", 4.0, False, True),
    (1, 2, 1, 200, 128, 200, "fp32", 1.0, True, False),
]


@pytest.mark.parametrize("case", PEAKED_BWD, ids=lambda c: "-".join(map(str, c)))
def test_backward_peaked_softmax(case):
    Bn, Hq, Hkv, N, d, L, dtype, c, grow, st = case
    Q, K, V, beta, M0, z0 = make_peaked(Bn, Hq, Hkv, N, d, L, dtype, 2000 + N + d, c, grow, st)
    dO = rnd(Q.shape, 5 + N, 1.0, dtype)
    dMS = dzS = None
    if st:
        dMS = np.random.default_rng(N).standard_normal(M0.shape).astype(np.float32) * 1e-2
        dzS = np.random.default_rng(N + 1).standard_normal(z0.shape).astype(np.float32) * 1e-2
    _check_bwd(Q, K, V, beta, L, M0, z0, dO, dMS, dzS, dtype, f"peaked c={c} grow={grow}")


# ------------------------------------------------------------------ variable-length batches

VARLEN_CASES = [
    # B, Hq, Hkv, N (capacity), d, L, dtype, state, lengths
    (3, 4, 2, 600, 128, 256, "bf16", True, [600, 0, 345]),       # long path, one empty sequence
    (2, 8, 2, 1000, 64, 384, "bf16", False, [1000, 130]),        # long path, ragged tails
    (4, 8, 2, 256, 128, 64, "bf16", True, [256, 100, 1, 0]),     # fused short path
    (1, 2, 2, 1024, 64, 64, "bf16", True, [700]),                # fused short, segments split over parts
    (2, 4, 4, 150, 64, 32, "bf16", False, [150, 77]),
    (3, 2, 2, 100, 32, 16, "fp32", True, [100, 37, 0]),          # generic path
    (2, 4, 2, 300, 64, 130, "bf16", True, [131, 300]),           # generic backward (bf16 seg_len > 64)
    (2, 4, 2, 90, 128, 40, "fp32", False, [90, 41]),
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: "-".join(map(str, c[:8])) + "-" + "_".join(map(str, c[8])))
def test_varlen_forward_and_backward(case):
    """infini_attn_fwd_varlen / infini_attn_bwd_varlen against the oracle's
    variable-length batch (each sequence processed as if alone; rows past its
    end zero), every output inside canary guard bands."""
    Bn, Hq, Hkv, N, d, L, dtype, st, lens = case
    Q, K, V, beta, M0, z0 = make(Bn, Hq, Hkv, N, d, dtype, seed=11 * N + d, with_state=st)
    check_fwd(Q, K, V, beta, L, M0, z0, dtype, "varlen", lens=lens)
    o, M, z, lse = run_fwd(Q, K, V, beta, L, M0, z0, dtype, want_lse=True, lens=lens)
    rl = O.forward(Q, K, V, beta, L, M0, z0, want_lse=True, lens=lens)[3]
    assert rel(host(lse), rl) < TOL[dtype]
    dO = rnd(Q.shape, 7 + N, 1.0, dtype)
    dMS = dzS = None
    if st:
        dMS = np.random.default_rng(N).standard_normal(M0.shape).astype(np.float32) * 1e-2
        dzS = np.random.default_rng(N + 1).standard_normal(z0.shape).astype(np.float32) * 1e-2
    _check_bwd(Q, K, V, beta, L, M0, z0, dO, dMS, dzS, dtype, "varlen", lens=lens)
    _check_bwd(Q, K, V, beta, L, M0, z0, dO, dMS, dzS, dtype, "varlen + saved lse", lens=lens,
               lse=host(lse).astype(np.float32))


def test_varlen_multi_chunk(monkeypatch):
    """More segments than one workspace chunk holds, with different lengths."""
    monkeypatch.setenv("INFINI_CHUNK_SEGMENTS", "3")
    Q, K, V, beta, M0, z0 = make(3, 4, 2, 20 * 16, 64, "fp32", seed=23, with_state=True)
    lens = [320, 150, 17]
    check_fwd(Q, K, V, beta, 16, M0, z0, "fp32", "varlen chunks", lens=lens)
    dO = rnd(Q.shape, 24, 1.0, "fp32")
    _check_bwd(Q, K, V, beta, 16, M0, z0, dO, None, None, "fp32", "varlen chunks", lens=lens)


def test_varlen_lengths_are_clamped():
    """Lengths below 0 or above the capacity act as 0 and the capacity."""
    Q, K, V, beta, M0, z0 = make(2, 4, 2, 128, 64, "bf16", seed=31, with_state=True)
    a = run_fwd(Q, K, V, beta, 64, M0, z0, "bf16", lens=[-5, 1000])
    b = run_fwd(Q, K, V, beta, 64, M0, z0, "bf16", lens=[0, 128])
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert np.array_equal(host(a[1])[0], M0[0])            # the empty sequence hands its state through


def test_varlen_full_lengths_equal_uniform_call():
    Q, K, V, beta, M0, z0 = make(2, 8, 2, 520, 128, "bf16", seed=37, with_state=True)
    a = run_fwd(Q, K, V, beta, 256, M0, z0, "bf16")
    b = run_fwd(Q, K, V, beta, 256, M0, z0, "bf16", lens=[520, 520])
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ------------------------------------------------------------------ Taylor feature map

TAYLOR_CASES = [
    # B, Hq, Hkv, N, d, L, dtype, state, lengths
    (1, 2, 2, 64, 32, 16, "fp32", True, None),
    (2, 4, 2, 150, 32, 48, "fp32", False, None),           # GQA, ragged tail
    (1, 2, 1, 96, 64, 40, "fp32", True, None),
    (2, 4, 2, 128, 64, 64, "bf16", True, None),
    (1, 2, 2, 70, 128, 32, "bf16", True, None),             # 16513 features
    (1, 2, 2, 40, 128, 40, "fp32", False, None),
    (3, 2, 2, 100, 32, 16, "fp32", True, [100, 0, 57]),     # variable lengths
]


def _taylor_fwd(Q, K, V, beta, L, M0, z0, dtype, lens, path):
    Bn, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    Bi = B()
    nf = Bi.feature_dim(d, "taylor2")
    td = torch.float32 if dtype == "fp32" else torch.bfloat16
    from gpu_util import guarded
    gs = [guarded(Q.shape, td), guarded((Bn, Hkv, nf, d), torch.float32), guarded((Bn, Hkv, nf), torch.float32),
          guarded((Bn, Hq, N), torch.float32)]
    q = dev(Q, dtype)
    assert Bi.fwd_path(Bi.problem(q, dev(K, dtype), L, "taylor2")) == path
    Bi.attn_fwd(q, dev(K, dtype), dev(V, dtype), dev(beta), L, dev(M0), dev(z0), want_lse=True,
                out=tuple(x.t for x in gs), seq_lens=dev_lens(lens), feature_map="taylor2")
    torch.cuda.synchronize()
    for name, x in zip(("O", "M_S", "z_S", "lse"), gs):
        x.check(name)
    ro, rM, rz, rl = O.forward(Q, K, V, beta, L, M0, z0, want_lse=True, lens=lens, fmap=O.Taylor2)
    errs = [rel(host(x.t), r) for x, r in zip(gs, (ro, rM, rz, rl))]
    log("   err O {:.2e} M {:.2e} z {:.2e} lse {:.2e}".format(*errs))
    assert all(e < TOL[dtype] for e in errs), errs


@pytest.mark.parametrize("case", TAYLOR_CASES, ids=lambda c: "-".join(map(str, c[:8])) + (
    "-" + "_".join(map(str, c[8])) if c[8] else ""))
def test_taylor_feature_map_forward(case):
    """The memory path with the second-order Taylor map (state of
    1 + d + d^2 rows) against the oracle with the same map."""
    Bn, Hq, Hkv, N, d, L, dtype, st, lens = case
    Q, K, V, beta, _, _ = make(Bn, Hq, Hkv, N, d, dtype, seed=13 * N + d)
    M0 = z0 = None
    if st:
        Kp = rnd((Bn, Hkv, 24, d), 5 + d, 1.0 / np.sqrt(d), dtype)
        Vp = rnd((Bn, Hkv, 24, d), 6 + d, 1.0 / np.sqrt(d), dtype)
        _, _, M0, z0 = O.state_sweep(Kp, Vp, 24, fmap=O.Taylor2)
        M0, z0 = M0.astype(np.float32), z0.astype(np.float32)
    log(f"taylor fwd Q{Q.shape} L={L} {dtype} state={st} lens={lens}")
    fast = dtype == "bf16" and d in (64, 128)
    _taylor_fwd(Q, K, V, beta, L, M0, z0, dtype, lens, "mfma_bf16_taylor2" if fast else "generic_fp32_taylor2")


# Matrix-core Taylor path (bf16, head_dim 64/128, no starting state): the
# scale sets q.k, so that at 0.4 and above the quadratic term of
# 1 + q.k + (q.k)^2 / 2 carries the weights (at 1/sqrt(d) it is ~1/(2 d^2)).
TAYLOR_FAST_CASES = [
    # B, Hq, Hkv, N, d, L, scale, lengths
    (2, 4, 2, 256, 64, 64, 0.125, None),
    (2, 4, 2, 300, 64, 64, 1.0, None),                      # ragged tail, peaked weights
    (1, 4, 1, 333, 64, 100, 0.4, None),                     # segments not on 64-key tiles, 2 query tiles
    (2, 2, 2, 260, 128, 48, 0.5, None),                     # seg_len < 64, tiles straddling segments
    (1, 2, 2, 520, 128, 200, 1.0, None),                    # 4 query tiles, online softmax over 4 key tiles
    (1, 2, 2, 400, 128, 200, 4.0, None),                    # very peaked scores and weights
    (3, 4, 2, 200, 64, 64, 0.5, [200, 0, 77]),              # variable lengths, one empty
    (1, 2, 1, 64, 64, 64, 1.0, None),                       # one segment: no earlier keys
    (1, 2, 2, 40, 128, 64, 1.0, None),                      # one short segment
    (2, 12, 12, 1024, 64, 64, 0.125, None),                 # the 200M-model shape at batch 2
]


@pytest.mark.parametrize("case", TAYLOR_FAST_CASES, ids=lambda c: "-".join(map(str, c[:7])) + (
    "-" + "_".join(map(str, c[7])) if c[7] else ""))
def test_taylor_matrix_core_forward(case):
    """bf16 Taylor forward on the matrix cores (polynomial-weighted attention
    over the earlier segments, state from K and V) against the oracle's
    segment-by-segment state path."""
    Bn, Hq, Hkv, N, d, L, sc, lens = case
    Q, K, V, beta, _, _ = make(Bn, Hq, Hkv, N, d, "bf16", seed=17 * N + d, scale=sc)
    log(f"taylor mfma fwd Q{Q.shape} L={L} scale={sc} lens={lens}")
    _taylor_fwd(Q, K, V, beta, L, None, None, "bf16", lens, "mfma_bf16_taylor2")


# The same path with a starting state M0, z0 (the Taylor state of earlier
# tokens, from the oracle): phi(q) M0 / phi(q) z0 join every query's retrieval
# and M0, z0 the final state.
TAYLOR_FAST_STATE_CASES = [
    # B, Hq, Hkv, N, d, L, scale, lengths
    (2, 4, 2, 200, 64, 64, 0.5, None),
    (1, 2, 2, 130, 128, 48, 1.0, None),
    (3, 4, 2, 150, 64, 100, 0.4, [150, 0, 61]),                 # variable lengths, one empty
    (1, 2, 1, 64, 64, 64, 1.0, None),                           # one segment: the state is all the memory
    (1, 4, 4, 300, 128, 256, 0.125, None),                      # 2 query-row tiles of the state kernel
]


@pytest.mark.parametrize("case", TAYLOR_FAST_STATE_CASES, ids=lambda c: "-".join(map(str, c[:7])) + (
    "-" + "_".join(map(str, c[7])) if c[7] else ""))
def test_taylor_matrix_core_forward_with_state(case):
    """bf16 Taylor forward on the matrix cores from a carried state against the
    oracle's state path."""
    Bn, Hq, Hkv, N, d, L, sc, lens = case
    Q, K, V, beta, _, _ = make(Bn, Hq, Hkv, N, d, "bf16", seed=19 * N + d, scale=sc)
    Kp = rnd((Bn, Hkv, 40, d), 7 + d, sc, "bf16")
    Vp = rnd((Bn, Hkv, 40, d), 8 + d, sc, "bf16")
    _, _, M0, z0 = O.state_sweep(Kp, Vp, 40, fmap=O.Taylor2)
    M0, z0 = M0.astype(np.float32), z0.astype(np.float32)
    log(f"taylor mfma fwd with state Q{Q.shape} L={L} scale={sc} lens={lens}")
    _taylor_fwd(Q, K, V, beta, L, M0, z0, "bf16", lens, "mfma_bf16_taylor2")


def _random_taylor_cases(n, seed):
    """Seeded shapes for the matrix-core Taylor path: head dims 64/128, GQA,
    seg_len from 1 past the sequence length, ragged tails, input scales from
    1/sqrt(d) to 2, and variable lengths (some empty)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.integers(1, 3))
        Hq = Hkv * int(rng.choice([1, 2, 4]))
        Bn = int(rng.integers(1, 4))
        N = int(rng.integers(1, 360))
        L = int(rng.choice([1, 5, 33, 64, 65, 100, 128, 300, 512]))
        sc = float(rng.choice([1.0 / np.sqrt(d), 0.5, 1.0, 2.0]))
        lens = [int(x) for x in rng.integers(0, N + 1, Bn)] if rng.random() < 0.4 else None
        out.append((Bn, Hq, Hkv, N, d, L, round(sc, 4), lens))
    return out


@pytest.mark.parametrize("case", _random_taylor_cases(10, 2027), ids=lambda c: "-".join(map(str, c[:7])) + (
    "-" + "_".join(map(str, c[7])) if c[7] else ""))
def test_taylor_matrix_core_random_shapes(case):
    """The matrix-core Taylor forward on seeded random shapes against the oracle."""
    Bn, Hq, Hkv, N, d, L, sc, lens = case
    Q, K, V, beta, _, _ = make(Bn, Hq, Hkv, N, d, "bf16", seed=31 * N + d, scale=sc)
    log(f"taylor mfma random Q{Q.shape} L={L} scale={sc} lens={lens}")
    _taylor_fwd(Q, K, V, beta, L, None, None, "bf16", lens, "mfma_bf16_taylor2")


def test_taylor_multi_chunk(monkeypatch):
    monkeypatch.setenv("INFINI_CHUNK_SEGMENTS", "3")
    Q, K, V, beta, _, _ = make(1, 2, 2, 8 * 8, 32, "fp32", seed=77)
    o, M, z = B().attn_fwd(dev(Q), dev(K), dev(V), dev(beta), 8, feature_map="taylor2")
    torch.cuda.synchronize()
    ro, rM, rz = O.forward(Q, K, V, beta, 8, fmap=O.Taylor2)
    assert rel(host(o), ro) < 1e-4 and rel(host(M), rM) < 1e-4 and rel(host(z), rz) < 1e-4


# ------------------------------------------------------------------ gate limits

def test_kernel_path_selection():
    from compressive_linear_memory_amd import binding as Bi
    assert Bi.fwd_path(Bi.Problem(1, 2, 2, 64, 128, 16, 1)) == "mfma_bf16_short"
    assert Bi.fwd_path(Bi.Problem(1, 2, 2, 64, 64, 64, 1)) == "mfma_bf16_short"
    assert Bi.fwd_path(Bi.Problem(1, 2, 2, 130, 64, 65, 1)) == "mfma_bf16"
    assert Bi.fwd_path(Bi.Problem(1, 2, 2, 256, 128, 128, 1)) == "mfma_bf16"
    assert Bi.fwd_path(Bi.Problem(1, 2, 2, 64, 32, 16, 1)) == "generic_fp32"
    assert Bi.fwd_path(Bi.Problem(1, 2, 2, 64, 128, 16, 0)) == "generic_fp32"


@pytest.mark.parametrize("bval", [-np.inf, np.inf])
def test_gate_limits_bf16_mfma(bval):
    Q, K, V, beta, M0, z0 = make(1, 4, 2, 256, 128, "bf16", seed=6)
    beta = np.full(4, bval, dtype=np.float32)
    o, _, _ = check_fwd(Q, K, V, beta, 64, None, None, "bf16", f"beta={bval}")
    oh = host(o)
    assert np.all(np.isfinite(oh))
    if bval > 0:
        assert np.all(oh[:, :, :64] == 0.0)


@pytest.mark.parametrize("bval", [-np.inf, np.inf])
def test_gate_limits(bval):
    Q, K, V, beta, M0, z0 = make(1, 4, 2, 64, 64, "fp32", seed=5)
    beta = np.full(4, bval, dtype=np.float32)
    o, _, _ = check_fwd(Q, K, V, beta, 16, None, None, "fp32", f"beta={bval}")
    oh = host(o)
    assert np.all(np.isfinite(oh))
    if bval > 0:
        assert np.all(oh[:, :, :16] == 0.0)      # empty memory retrieves exactly nothing


# ------------------------------------------------------------------ chaining, chunks, determinism

def test_chained_calls_equal_one_call():
    Q, K, V, beta, M0, z0 = make(2, 4, 2, 128, 64, "bf16", seed=17, with_state=True)
    L = 32
    o_all, M_all, z_all = run_fwd(Q, K, V, beta, L, M0, z0, "bf16")
    Ms, zs = dev(M0), dev(z0)
    outs = []
    for s in range(4):
        r = slice(s * L, (s + 1) * L)
        o, Ms, zs = B().attn_fwd(dev(Q[:, :, r], "bf16"), dev(K[:, :, r], "bf16"), dev(V[:, :, r], "bf16"),
                                 dev(beta), L, Ms, zs)
        outs.append(o)
    o_chain = torch.cat(outs, dim=2)
    assert rel(host(o_chain), host(o_all)) < 1e-6
    assert rel(host(Ms), host(M_all)) < 1e-6


def test_multi_chunk_matches_single_chunk(monkeypatch):
    Q, K, V, beta, M0, z0 = make(1, 4, 2, 20 * 16, 64, "fp32", seed=23, with_state=True)
    dO = rnd(Q.shape, 24, 1.0, "fp32")
    ref_f = run_fwd(Q, K, V, beta, 16, M0, z0, "fp32")
    ref_b = B().attn_bwd(dev(Q), dev(K), dev(V), dev(beta), 16, dev(dO), dev(M0), dev(z0),
                         want_state_grads=True)
    monkeypatch.setenv("INFINI_CHUNK_SEGMENTS", "3")
    got_f = run_fwd(Q, K, V, beta, 16, M0, z0, "fp32")
    got_b = B().attn_bwd(dev(Q), dev(K), dev(V), dev(beta), 16, dev(dO), dev(M0), dev(z0),
                         want_state_grads=True)
    for a, b in zip(ref_f, got_f):
        assert rel(host(a), host(b)) < 1e-5
    for a, b in zip(ref_b, got_b):
        assert rel(host(a), host(b)) < 1e-5
    ro, rM, rz = O.forward(Q, K, V, beta, 16, M0, z0)
    assert rel(host(got_f[0]), ro) < 1e-4


@pytest.mark.parametrize("L", [256, 64], ids=["long_path", "fused_short_path"])
def test_graph_replay_matches_eager(L):
    """Chained forward calls recorded once in a HIP graph: every replay equals
    the eager run bit for bit, with eager work and synchronisation between the
    replays (the library issues no memset or allocation inside the calls)."""
    Bi = B()
    Bn, Hq, Hkv, N, d = 1, 4, 2, 512, 64
    Q, K, V, beta, M0, z0 = make(Bn, Hq, Hkv, N, d, "bf16", seed=91, with_state=True)
    q, k, v, b, m0, s0 = dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), dev(beta), dev(M0), dev(z0)
    p = Bi.problem(q, k, L)
    ws = torch.empty(max(Bi.workspace_bytes(p), 1), dtype=torch.uint8, device="cuda")
    n = 3
    outs = [(torch.empty_like(q), torch.empty_like(m0), torch.empty_like(s0)) for _ in range(n)]

    def chain():
        m, z = m0, s0
        for i in range(n):
            Bi.attn_fwd(q, k, v, b, L, m, z, out=(outs[i][0], outs[i][1], outs[i][2], None), ws=ws)
            m, z = outs[i][1], outs[i][2]

    chain()
    torch.cuda.synchronize()
    eager = [tuple(t.clone() for t in o) for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain()
    torch.cuda.synchronize()
    for r in range(3):
        for o in outs:
            for t in o:
                t.fill_(float("nan"))
        Bi.attn_fwd(q, k, v, b, L, m0, s0, ws=ws)      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i in range(n):
            for a, e in zip(outs[i], eager[i]):
                assert torch.equal(a, e), (r, i)
    log(f"   graph L={L}: 3 replays of {n} chained calls equal the eager run")


def test_run_twice_bitwise_identical():
    Q, K, V, beta, M0, z0 = make(2, 8, 2, 256, 128, "bf16", seed=29, with_state=True)
    a = run_fwd(Q, K, V, beta, 64, M0, z0, "bf16")
    b = run_fwd(Q, K, V, beta, 64, M0, z0, "bf16")
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    dO = rnd(Q.shape, 30, 1.0, "bf16")
    args = (dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), dev(beta), 64, dev(dO, "bf16"), dev(M0), dev(z0))
    g1 = B().attn_bwd(*args)
    g2 = B().attn_bwd(*args)
    for x, y in zip(g1, g2):
        assert torch.equal(x, y)


def test_short_forward_needs_no_workspace():
    """The fused short-segment forward keeps its state on chip: with no
    workspace at all it gives the same bits as with one."""
    Q, K, V, beta, M0, z0 = make(2, 8, 2, 256, 128, "bf16", seed=29, with_state=True)
    q, k, v = dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16")
    assert B().fwd_path(B().problem(q, k, 64)) == "mfma_bf16_short"
    a = B().attn_fwd(q, k, v, dev(beta), 64, dev(M0), dev(z0))
    none = torch.empty(0, dtype=torch.uint8, device="cuda")
    b = B().attn_fwd(q, k, v, dev(beta), 64, dev(M0), dev(z0), ws=none)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_errors_raise_with_real_tensors():
    Q, K, V, beta, _, _ = make(1, 2, 2, 64, 32, "fp32", seed=31)
    q = dev(Q)
    Q3, K3, V3, beta3, _, _ = make(1, 3, 2, 64, 32, "fp32", seed=32)
    with pytest.raises(B().InfiniError) as e:
        B().attn_fwd(dev(Q3), dev(K3), dev(V3), dev(beta3), 16)   # 3 query heads over 2 K/V heads
    assert e.value.code == 2
    o = torch.empty_like(q)
    Ms = torch.empty((1, 2, 32, 32), device="cuda")
    zs = torch.empty((1, 2, 32), device="cuda")
    with pytest.raises(B().InfiniError) as e:
        B().attn_fwd(q, dev(K), dev(V), dev(beta), 16, out=(q, Ms, zs, None))   # O aliases Q
    assert e.value.code == 4
    del o


@pytest.mark.parametrize("dtype,d", [("fp32", 32), ("bf16", 128)])
def test_empty_sequence_passes_state_through(dtype, d):
    """seq_len = 0: no tokens, so the forward hands the state on unchanged
    (zeros for an empty memory) and the backward hands its gradient back
    (dbeta = 0); batch = 0 gives empty outputs."""
    log(f"empty sequence {dtype} d={d}")
    Q, K, V, beta, _, _ = make(2, 4, 2, 0, d, dtype, seed=41)
    M0, z0 = make(2, 4, 2, 48, d, dtype, seed=42, with_state=True)[4:]
    o, M, z = run_fwd(Q, K, V, beta, 16, M0, z0, dtype)
    assert o.shape == (2, 4, 0, d)
    assert np.array_equal(host(M), M0) and np.array_equal(host(z), z0)
    o, M, z = run_fwd(Q, K, V, beta, 16, None, None, dtype)
    assert not host(M).any() and not host(z).any()
    dMS = rnd((2, 2, d, d), 43, 1.0, "fp32")
    dzS = rnd((2, 2, d), 44, 1.0, "fp32")
    g = B().attn_bwd(dev(Q, dtype), dev(K, dtype), dev(V, dtype), dev(beta), 16, dev(Q, dtype),
                     dev(M0), dev(z0), dM_S=dev(dMS), dz_S=dev(dzS), want_state_grads=True)
    assert not host(g[3]).any()
    assert np.array_equal(host(g[4]), dMS) and np.array_equal(host(g[5]), dzS)
    g = B().attn_bwd(dev(Q, dtype), dev(K, dtype), dev(V, dtype), dev(beta), 16, dev(Q, dtype),
                     want_state_grads=True)
    assert not host(g[4]).any() and not host(g[5]).any()
    # the phased forward: the memory phase hands the state on, attend writes nothing
    q, k, v = dev(Q, dtype), dev(K, dtype), dev(V, dtype)
    p = B().problem(q, k, 16)
    ws = torch.empty(max(B().workspace_bytes(p), 1), dtype=torch.uint8, device="cuda")
    Ms = torch.full((2, 2, d, d), 7.0, device="cuda")
    zs = torch.full((2, 2, d), 7.0, device="cuda")
    B().fwd_memory(p, k, v, dev(M0), dev(z0), Ms, zs, ws)
    B().fwd_attend(p, q, k, v, dev(beta), torch.empty_like(q), None, ws)
    assert np.array_equal(host(Ms), M0) and np.array_equal(host(zs), z0)
    Q, K, V, beta, _, _ = make(0, 4, 2, 64, d, dtype, seed=45)
    o, M, z = run_fwd(Q, K, V, beta, 16, None, None, dtype)
    assert o.shape == (0, 4, 64, d) and M.numel() == 0 and z.numel() == 0
    torch.cuda.synchronize()


# ------------------------------------------------------------------ the five workloads at full size

def test_fwd_200m_full():
    w = I.WORKLOADS["fwd_200m"]
    Q, K, V = I.qkv(w)
    check_fwd(Q, K, V, I.beta(w), w.seg_len, None, None, "bf16", w.name)


def test_train_llama3_8b_full():
    w = I.WORKLOADS["train_llama3_8b"]
    Q, K, V = I.qkv(w)
    beta = I.beta(w)
    check_fwd(Q, K, V, beta, w.seg_len, None, None, "bf16", w.name)
    _check_bwd(Q, K, V, beta, w.seg_len, None, None, I.d_out(w), None, None, "bf16", w.name)


def test_train_llama3_8b_backward_from_gpu_forward_lse():
    """The training step as the benchmark runs it: the forward's lse output
    fed to the backward; every gradient matches the oracle."""
    w = I.WORKLOADS["train_llama3_8b"]
    Q, K, V = I.qkv(w)
    beta = I.beta(w)
    _, _, _, lse = run_fwd(Q, K, V, beta, w.seg_len, None, None, "bf16", want_lse=True)
    _check_bwd(Q, K, V, beta, w.seg_len, None, None, I.d_out(w), None, None, "bf16", w.name + " lse",
               lse=host(lse).astype(np.float32))


def test_train_llama3_8b_backward_from_saved_state():
    """The training step as the benchmark runs it: the forward's lse and final
    state fed to infini_attn_bwd_saved.  Every gradient matches the oracle, and
    the fused short-segment backward, which would rebuild that very state,
    gives the same gradients bit for bit."""
    w = I.WORKLOADS["train_llama3_8b"]
    Q, K, V = I.qkv(w)
    beta = I.beta(w)
    dO = I.d_out(w)
    _, M, z, lse = run_fwd(Q, K, V, beta, w.seg_len, None, None, "bf16", want_lse=True)
    lse_h = host(lse).astype(np.float32)
    a = _check_bwd(Q, K, V, beta, w.seg_len, None, None, dO, None, None, "bf16", w.name + " saved state",
                   lse=lse_h, saved=(M, z))
    b = _check_bwd(Q, K, V, beta, w.seg_len, None, None, dO, None, None, "bf16", w.name + " lse", lse=lse_h)
    for name, x, y in zip(("dQ", "dK", "dV", "dbeta", "dM0", "dz0"), a, b):
        assert torch.equal(x, y), name


SAVED_CASES = [
    # B, Hq, Hkv, N, d, L, dtype, lens, chunk segments (None = default)
    (2, 4, 2, 200, 64, 64, "bf16", [200, 130], None),     # fused short path, GQA, ragged, varlen
    (1, 2, 2, 190, 128, 40, "bf16", None, None),          # fused short path, head_dim 128, ragged
    (1, 4, 2, 520, 128, 256, "bf16", None, None),         # long-segment matrix-core path
    (2, 4, 2, 20 * 16, 64, 16, "fp32", [320, 150], "3"),  # generic path, several workspace chunks
]


@pytest.mark.parametrize("case", SAVED_CASES, ids=lambda c: "x".join(map(str, c[:6])) + c[6])
def test_backward_from_saved_state(case, monkeypatch):
    """infini_attn_bwd_saved with the forward's final state: every gradient
    matches the oracle, with a carried state and upstream state gradients."""
    Bn, Hq, Hkv, N, d, L, dtype, lens, chunks = case
    if chunks:
        monkeypatch.setenv("INFINI_CHUNK_SEGMENTS", chunks)
    Q, K, V, beta, M0, z0 = make(Bn, Hq, Hkv, N, d, dtype, seed=N + d, with_state=True)
    dO = rnd(Q.shape, N + 5, 1.0, dtype)
    g = np.random.default_rng(N + 9)
    dMS = (g.standard_normal(M0.shape) * 1e-2).astype(np.float32)
    dzS = (g.standard_normal(z0.shape) * 1e-2).astype(np.float32)
    _, M, z, lse = run_fwd(Q, K, V, beta, L, M0, z0, dtype, want_lse=True, lens=lens)
    _check_bwd(Q, K, V, beta, L, M0, z0, dO, dMS, dzS, dtype, "saved state", lens=lens,
               lse=host(lse).astype(np.float32), saved=(M, z))


def sampled_units(w, n_units, seed):
    """(b, h, s) units covering every segment index and K/V group, plus row picks."""
    g = np.random.default_rng(seed)
    units = []
    for u in range(n_units):
        s = u % w.segments
        h = (u * 7 + g.integers(0, w.q_heads)) % w.q_heads
        b = int(g.integers(0, w.batch))
        rows = np.unique(np.concatenate([[0, w.seg_len - 1], g.integers(0, w.seg_len, 30)]))
        units.append((b, int(h), s, rows))
    return units


def test_fwd_llama3_8b_full_sampled():
    w = I.WORKLOADS["fwd_llama3_8b"]
    log("generating fwd_llama3_8b inputs")
    Q, K, V = I.qkv(w)
    beta = I.beta(w)
    o, M, z = run_fwd(Q, K, V, beta, w.seg_len, None, None, "bf16")
    torch.cuda.synchronize()
    Msnap, zsnap, rM, rz = O.state_sweep(K, V, w.seg_len)
    eM, ez = rel(host(M), rM), rel(host(z), rz)
    G = w.q_heads // w.kv_heads
    L = w.seg_len
    got, ref = [], []
    for (b, h, s, rows) in sampled_units(w, 48, 3):
        r = slice(s * L, (s + 1) * L)
        ref.append(O.segment_unit(Q[b, h, r], K[b, h // G, r], V[b, h // G, r],
                                  Msnap[b, h // G, s], zsnap[b, h // G, s], beta[h], rows))
        got.append(host(o[b, h, s * L + rows]))
    eo = rel(np.concatenate(got), np.concatenate(ref))
    log(f"   fwd_llama3_8b err O(sampled) {eo:.2e} M {eM:.2e} z {ez:.2e}")
    assert eo < 2e-2 and eM < 2e-2 and ez < 2e-2


def test_stream_1m_launch_shape_chained():
    """Streaming workload's launch shape (one 2048-token segment per call),
    state carried across calls; the first launches of the 512-launch stream."""
    w = I.WORKLOADS["stream_1m"]
    beta = I.beta(w)
    n_launch = int(os.environ.get("INFINI_TEST_STREAM_LAUNCHES", "6"))
    Ms = zs = None
    rM = rz = None
    for t in range(n_launch):
        Q, K, V = I.qkv(w, launch=t)
        o, Ms, zs = B().attn_fwd(dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), dev(beta), w.seg_len, Ms, zs)
        Msnap, zsnap, rM1, rz1 = O.state_sweep(K, V, w.seg_len, rM, rz)
        ref = []
        got = []
        for h in range(0, w.q_heads, 5):
            rows = np.array([0, 1, 777, 2047])
            ref.append(O.segment_unit(Q[0, h], K[0, h], V[0, h], Msnap[0, h, 0], zsnap[0, h, 0], beta[h], rows))
            got.append(host(o[0, h, rows]))
        eo = rel(np.concatenate(got), np.concatenate(ref))
        rM, rz = rM1, rz1
        eM, ez = rel(host(Ms), rM), rel(host(zs), rz)
        log(f"   launch {t}: err O {eo:.2e} M {eM:.2e} z {ez:.2e}")
        assert eo < 2e-2 and eM < 2e-2 and ez < 2e-2


def test_stream_1m_all_512_launches_drift():
    """The streaming workload at its real length: 512 chained one-segment
    launches (1,048,576 tokens), issued through infini_fwd_stream in the
    benchmark's schedule (memory phases on one stream, groups of 4 launches'
    attention phases on 2 streams) with the benchmark's inputs (8 distinct
    launches cycled).  The state after every 32nd launch is compared with the
    oracle's memory sweep over all launches so far, and sampled output rows of
    every head at launches 0, 255 and 511 with the oracle's unit from the
    state before that launch.  The per-launch error is logged: it must stay
    bounded over the 512 compressions ([HF] "결론 및 기술적 시사점": quality
    degrades as compressions accumulate; here the question is only whether the
    fp32 state drifts from the exact sum)."""
    Bi = B()
    w = I.WORKLOADS["stream_1m"]
    nd, n_launch, per_call, npipe, group = 8, w.launches, 32, 2, 4
    L, H, d = w.seg_len, w.kv_heads, w.head_dim
    beta = I.beta(w)
    log("stream_1m: generating 8 distinct launch inputs")
    host_in = [I.qkv(w, launch=t) for t in range(nd)]
    dM, dz = [], []
    for (_, K, V) in host_in:                      # the oracle's update of one launch from an empty state
        _, _, m_, z_ = O.state_sweep(K, V, L)
        dM.append(m_)
        dz.append(z_)
    ins = [tuple(dev(x, "bf16") for x in t3) for t3 in host_in]
    b = dev(beta)
    p = Bi.problem(ins[0][0], ins[0][1], L)
    ws = torch.empty(Bi.stream_workspace_bytes(p, npipe, group), dtype=torch.uint8, device="cuda")
    pool = [torch.empty_like(ins[0][0]) for _ in range(npipe * group)]
    keep = {0: torch.empty_like(ins[0][0]), 255: torch.empty_like(ins[0][0]), 511: torch.empty_like(ins[0][0])}
    M = torch.zeros((1, H, d, d), device="cuda")
    z = torch.zeros((1, H, d), device="cuda")
    sm = torch.cuda.Stream()
    sa = [torch.cuda.Stream() for _ in range(npipe)]
    evs = [torch.cuda.Event() for _ in range(2 * npipe)]
    cur = torch.cuda.current_stream()
    rM = np.zeros((1, H, d, d))
    rz = np.zeros((1, H, d))
    before = {}                                    # oracle state before the launches whose rows are checked
    curve = []
    for c0 in range(0, n_launch, per_call):
        idx = list(range(c0, c0 + per_call))
        outs = [keep.get(i, pool[i % len(pool)]) for i in idx]
        torch.cuda.synchronize()
        Bi.fwd_stream(p, [ins[i % nd][0] for i in idx], [ins[i % nd][1] for i in idx],
                      [ins[i % nd][2] for i in idx], b, M, z, outs, ws, npipe, group, sm, sa, evs)
        cur.wait_stream(sm)
        for s_ in sa:
            cur.wait_stream(s_)
        torch.cuda.synchronize()
        for i in idx:
            if i in keep:
                before[i] = (rM.copy(), rz.copy())
            rM = rM + dM[i % nd]
            rz = rz + dz[i % nd]
        eM, ez = rel(host(M), rM), rel(host(z), rz)
        curve.append((idx[-1], eM, ez))
        log(f"   after launch {idx[-1]:3d}: err M {eM:.2e} z {ez:.2e}")
        assert eM < 2e-2 and ez < 2e-2, (idx[-1], eM, ez)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 1023, 1024, L - 1],
                                     np.random.default_rng(5).integers(0, L, 40)]))
    for i, o in keep.items():
        Q, K, V = host_in[i % nd]
        Mb, zb = before[i]
        got = host(o[0][:, rows])
        ref = np.stack([O.segment_unit(Q[0, h], K[0, h], V[0, h], Mb[0, h], zb[0, h], beta[h], rows)
                        for h in range(w.q_heads)])
        eo = rel(got, ref)
        log(f"   launch {i}: err O (every head, {len(rows)} rows) {eo:.2e}")
        assert eo < 2e-2, (i, eo)
    log("   drift curve (launch, err M, err z): " + ", ".join(f"({t}, {a:.1e}, {c:.1e})" for t, a, c in curve))


STREAM_CASES = [
    # B, Hq, Hkv, N per call, d, L, dtype, calls, n_pipe, group
    (1, 4, 4, 256, 64, 128, "bf16", 5, 3, 1),
    (1, 4, 4, 256, 64, 128, "bf16", 7, 2, 3),   # groups of 3, the last one short
    (2, 4, 2, 300, 128, 128, "bf16", 5, 2, 2),  # GQA, ragged last segment of each call
    (1, 2, 2, 48, 32, 16, "fp32", 5, 2, 2),     # generic fp32 path (attention per call)
    (1, 32, 32, 2048, 64, 2048, "bf16", 9, 2, 4),  # the streaming workload's call shape
]


@pytest.mark.parametrize("case", STREAM_CASES, ids=lambda c: "-".join(map(str, c)))
def test_fwd_stream_equals_chained_calls(case):
    """infini_fwd_stream (memory phases in order on one stream, each group
    of calls' memory phases as one run and its attention phases as one
    launch, overlapped on n_pipe other streams) gives the outputs and the
    final state
    of the same calls made one after another with infini_attn_fwd, bit for
    bit; the chained calls also match the oracle on the first call (small
    cases; the streaming-shape case relies on the chained test above)."""
    Bn, Hq, Hkv, N, d, L, dtype, n, npipe, group = case
    log(f"fwd_stream {case}")
    ins = [make(Bn, Hq, Hkv, N, d, dtype, 700 + 10 * t, with_state=(t == 0)) for t in range(n)]
    beta = dev(ins[0][3])
    qs = [dev(x[0], dtype) for x in ins]
    ks = [dev(x[1], dtype) for x in ins]
    vs = [dev(x[2], dtype) for x in ins]
    M0, z0 = ins[0][4], ins[0][5]
    # chained reference calls
    Mr, zr = dev(M0), dev(z0)
    refs = []
    for t in range(n):
        o, Mr, zr = B().attn_fwd(qs[t], ks[t], vs[t], beta, L, Mr, zr)
        refs.append(o)
    if Hq * N <= 4096:                    # the oracle in seconds
        ro, rM, rz = O.forward(ins[0][0], ins[0][1], ins[0][2], ins[0][3], L, M0, z0)
        assert rel(host(refs[0]), ro) < TOL[dtype]
    # one pipelined call
    p = B().problem(qs[0], ks[0], L)
    ws = torch.empty(B().stream_workspace_bytes(p, npipe, group), dtype=torch.uint8, device="cuda")
    outs = [torch.empty_like(q) for q in qs]
    M, z = dev(M0).clone(), dev(z0).clone()
    sm = torch.cuda.Stream()
    sa = [torch.cuda.Stream() for _ in range(npipe)]
    evs = [torch.cuda.Event() for _ in range(2 * npipe)]
    cur = torch.cuda.current_stream()
    torch.cuda.synchronize()
    B().fwd_stream(p, qs, ks, vs, beta, M, z, outs, ws, npipe, group, sm, sa, evs)
    cur.wait_stream(sm)
    for s_ in sa:
        cur.wait_stream(s_)
    torch.cuda.synchronize()
    for t in range(n):
        assert torch.equal(outs[t], refs[t]), t
    assert torch.equal(M, Mr) and torch.equal(z, zr)


def test_fwd_stream_refuses_graph_capture():
    """infini_fwd_stream cannot be recorded into a HIP graph: with its memory
    stream or an attention stream under capture it returns
    INFINI_ERR_UNSUPPORTED before issuing anything, and the capture ends
    empty.  The events are made real outside the capture."""
    Bi = B()
    Bn, Hq, Hkv, N, d, L, dtype = 1, 4, 4, 256, 64, 128, "bf16"
    ins = [make(Bn, Hq, Hkv, N, d, dtype, 900 + t) for t in range(2)]
    qs = [dev(x[0], dtype) for x in ins]
    ks = [dev(x[1], dtype) for x in ins]
    vs = [dev(x[2], dtype) for x in ins]
    beta = dev(ins[0][3])
    p = Bi.problem(qs[0], ks[0], L)
    ws = torch.empty(Bi.stream_workspace_bytes(p, 1, 1), dtype=torch.uint8, device="cuda")
    outs = [torch.empty_like(q) for q in qs]
    M = torch.zeros((Bn, Hkv, d, d), device="cuda")
    z = torch.zeros((Bn, Hkv, d), device="cuda")
    side = torch.cuda.Stream()
    evs = [torch.cuda.Event() for _ in range(2)]
    for e_ in evs:                # create the HIP events now, outside the capture
        e_.record()
    torch.cuda.synchronize()
    for which in ("memory", "attention"):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream()
            sm, sa = (cap, side) if which == "memory" else (side, cap)
            calls = Bi.StreamCalls(p, qs, ks, vs, beta, M, z, outs, ws, 1, 1, sm, [sa], evs)
            with pytest.raises(Bi.InfiniError) as e:
                calls()
            assert e.value.code == 3
        torch.cuda.synchronize()
    assert not M.any() and not z.any()      # nothing ran


# ------------------------------------------------------------------ streaming decode

DECODE_CASES = [
    # B, Hq, Hkv, N, d, L, dtype, state, pieces (tokens per call, cycled)
    (1, 4, 2, 40, 32, 16, "fp32", True, (1, 3, 1, 5)),
    (2, 2, 2, 150, 64, 64, "bf16", False, (1, 7, 2)),
    (1, 8, 2, 300, 128, 128, "bf16", True, (5, 1, 16)),
    (1, 2, 2, 2100, 64, 2048, "bf16", True, (1, 64, 1, 300)),   # rows past one 1024-key chunk
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "-".join(map(str, c[:8])))
def test_decode_in_pieces_equals_one_forward(case):
    """Feeding a sequence through infini_decode a few tokens at a time gives
    the oracle's forward over the whole sequence: every output row, and the
    state after every completed segment."""
    Bn, Hq, Hkv, N, d, L, dtype, st, pieces = case
    Q, K, V, beta, M0, z0 = make(Bn, Hq, Hkv, N, d, dtype, seed=N + 7 * d, with_state=st)
    _decode_in_pieces(Q, K, V, beta, L, M0, z0, dtype, pieces)


@pytest.mark.parametrize("case", [
    # B, Hq, Hkv, N, d, L, dtype, c, grow, pieces
    (1, 2, 2, 2100, 64, 2048, "bf16", 1.0, True, (1, 64, 1, 300)),    # rows past one 1024-key chunk
    (1, 4, 2, 1300, 128, 1300, "bf16", 4.0, False, (700, 1, 3, 50)),
    (1, 2, 1, 1100, 64, 1100, "fp32", 4.0, True, (1030, 1, 2)),
], ids=lambda c: "-".join(map(str, c[:9])))
def test_decode_peaked_softmax(case):
    """Decode with peaked scores (Q, K ~ N(0,1) c, key norms growing along the
    segment): the running softmax state of a row moves between 1024-key
    chunks and between key splits, so the merges rescale."""
    Bn, Hq, Hkv, N, d, L, dtype, c, grow, pieces = case
    Q, K, V, beta, M0, z0 = make_peaked(Bn, Hq, Hkv, N, d, L, dtype, 3000 + N, c, grow, True)
    S = Q[0, 0, :L].astype(np.float64) @ K[0, 0, :L].astype(np.float64).T / np.sqrt(d)
    last = min(L, N) - 1
    lead = S[last, 1024:last + 1].max() - S[last, :1024].max()
    log(f"   last row: later chunk's max leads the first chunk's by {lead:.1f} (natural log units)")
    _decode_in_pieces(Q, K, V, beta, L, M0, z0, dtype, pieces)


def _decode_in_pieces(Q, K, V, beta, L, M0, z0, dtype, pieces):
    Bn, Hq, N, d = Q.shape
    Hkv = K.shape[1]
    ro, rM, rz = O.forward(Q, K, V, beta, L, M0, z0)
    log(f"decode Q{Q.shape} L={L} {dtype} pieces={pieces}")
    Bi = B()
    td = torch.float32 if dtype == "fp32" else torch.bfloat16
    kc = torch.zeros((Bn, Hkv, L, d), dtype=td, device="cuda")
    vc = torch.zeros_like(kc)
    M, z = dev(M0), dev(z0)
    b = dev(beta)
    outs = []
    n, k, closed = 0, 0, 0
    while n < N:
        pos = n % L
        T = min(pieces[k % len(pieces)], L - pos, N - n)
        r = slice(n, n + T)
        res = Bi.decode(dev(Q[:, :, r], dtype), dev(K[:, :, r], dtype), dev(V[:, :, r], dtype), b, L, pos,
                        kc, vc, M, z)
        if pos + T == L:
            o, M, z = res
            closed += 1
        else:
            o = res
        outs.append(o)
        n += T
        k += 1
    torch.cuda.synchronize()
    got = torch.cat(outs, dim=2)
    eo = rel(host(got), ro)
    log(f"   {k} calls, {closed} completed segments: err O {eo:.2e}")
    assert eo < TOL[dtype]
    if N % L == 0:      # the state after the last completed segment is the forward's final state
        assert rel(host(M), rM) < TOL[dtype] and rel(host(z), rz) < TOL[dtype]
    else:
        _, _, sM, sz = O.state_sweep(K[:, :, : (N // L) * L], V[:, :, : (N // L) * L], L, M0, z0)
        if closed:
            assert rel(host(M), sM) < TOL[dtype] and rel(host(z), sz) < TOL[dtype]


def test_decode_argument_errors():
    """Rejected before any launch: a piece past the segment end, a negative
    position, an output overlapping the cache."""
    Bi = B()
    q = torch.zeros((1, 2, 3, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 2, 3, 64), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((1, 2, 16, 64), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    b = torch.zeros(2, device="cuda")
    for pos in (14, -1):
        with pytest.raises(Bi.InfiniError) as e:
            Bi.decode(q, k, k, b, 16, pos, kc, vc)
        assert e.value.code == 2
    with pytest.raises(Bi.InfiniError) as e:
        Bi.decode(q, k, k, b, 16, 0, kc, vc, out=kc[:, :, :3])
    assert e.value.code == 4
