"""CPU oracle for the Infini-attention segment kernel (test infrastructure).

This module is test infrastructure.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the library path never does.  It
shares no code with the HIP implementation.

Everything is evaluated in float64 with numpy, on the exact values the GPU
receives (bf16 or fp32 inputs are widened exactly before any arithmetic).
The functions follow the method's steps in the order the pages give them.

Sources (web pages; cited by title and section):
  [HF]  "Hugging Face Infini-Attention 재현 분석" (agentlenshq.com), section
        "Infini-Attention 메커니즘": the steps Segmentation, Local Attention,
        Memory Retrieval (ELU + 1 on the queries, memory M_{s-1}),
        Integration (learned scalar beta through a sigmoid balancing A_mem
        and A_dot), Memory Update (current segment's key-value states added
        to the buffer), State Transfer (only the updated memory is carried).
        Section "재현 도전 과제 및 수렴 문제": 16 rollouts of segment length 64.
  [LNCB] "[정보] KV선형 덧셈연산 인피니 어텐션에 대한 정보" (mir.rootios.com),
        the summary of "Leave No Context Behind": masked local attention and
        long-term *linear* attention in one block; memory reuses the standard
        attention's query/key/value states; minimal change to standard scaled
        dot-product attention; segment-level processing like Transformer-XL,
        but older KV states are compressed instead of discarded.
  [ASM] "Context Memorization for Efficient Long Context Generation"
        (gist.science), section "방법론": attention states (a, Z) over key
        sub-blocks merge exactly by the online-softmax identity.  The oracle
        does not use it (it forms full softmax rows); the GPU kernels do.

Readings where the pages leave a step open (each is stated where it is used):
  R1  Retrieval is linear attention over the compressed memory, normalised by
      the key-feature sum:  A_mem = sigma(Q) M_{s-1} / (sigma(Q) z_{s-1} + eps),
      with M_s = M_{s-1} + sigma(K_s)^T V_s and z_s = z_{s-1} + sum_rows sigma(K_s).
      [HF] names M, ELU+1 and the additive update; [LNCB] calls it linear
      attention, whose standard form carries the normaliser z.
  R2  eps = 1e-6 is added to the denominator (the pages are silent; with an
      empty memory, M0 = z0 = 0, it makes A_mem = 0 instead of 0/0).
  R3  Local attention scale is 1/sqrt(d) ([LNCB]: standard *scaled* dot product).
  R4  ELU has alpha = 1, so sigma(x) = x + 1 for x > 0 and exp(x) otherwise.
  R5  The gate is O = g A_mem + (1 - g) A_dot with g = sigmoid(beta_h), one
      beta per query head ([HF] Integration).
  R6  Retrieval in segment s reads M_{s-1}, the state before this segment's
      update ([HF]: retrieve from M_{s-1}, then update).
  R7  Grouped-query attention: query head h uses K/V head floor(h / G) with
      G = Hq / Hkv, and the memory (M, z) is per K/V head, since the update
      uses only K and V.
  R8  Q and K arrive with any positional encoding already applied.
  R9  The backward is the exact derivative of this forward (the pages only say
      the method is trainable end to end); dM_S, dz_S are optional upstream
      gradients of the carried state and dM0, dz0 the gradients of the state
      passed in, so backward chains across calls like the forward.
  R10 A sequence whose length is not a multiple of the segment length ends in
      one shorter segment ([HF] Segmentation fixes the segment length but not
      what happens to a remainder).  It is processed like every other segment:
      causal attention among its own tokens, retrieval from the state before
      it, and an update with its keys.  So segments are the slices
      [s L, min((s+1) L, N)) for s = 0 .. ceil(N / L) - 1.

  R14 Variable-length batches: each sequence b of a batch has its own length
      n_b <= N and is stored in the first n_b rows of its [N, d] slot; it is
      cut into segments and processed exactly as if it were alone (its own
      ragged last segment, R10), and its state M_S[b] is the state after its
      own last segment.  Rows past n_b belong to no segment: they are never
      read, and every per-row output there (O, lse, dQ, dK, dV) is zero.
      [HF] Segmentation cuts each input sequence; nothing couples the
      sequences of a batch.

  R15 Pluggable feature map.  The memory path's feature map is ELU + 1 (R4)
      by default; the alternative is the second-order Taylor map of the
      page "Based" (cartesia.ai), section "고정 크기 순환 상태를 사용하는
      방법도 중요합니다": phi is chosen so that phi(q) . phi(k) equals
      1 + q.k + (q.k)^2 / 2, the Taylor series of exp(q.k) to second order,
      with the key dimension growing from d to about d^2.  Written out:
      phi(x) = [1, x_1 .. x_d, x_a x_b / sqrt 2 for a, b = 1 .. d (a major)],
      D' = 1 + d + d^2 features.  It is applied to Q and K as they arrive
      (no 1/sqrt(d): the page states the approximation of exp(q k^T)
      itself), and everything else is unchanged: M is D' x d, z has D'
      entries, A_mem = phi(Q) M / (phi(Q) z + eps).  Since
      1 + x + x^2 / 2 >= 1/2 for every real x, the denominator stays
      positive.  The local attention keeps its exact softmax.

Parity pins: every public function is pinned by tests in tests/test_oracle_pins.py
against brute force, closed forms, invariants, a library attention routine
and finite differences.  No function here is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

EPS = 1e-6   # R2


# ------------------------------------------------------------------ helpers

def f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def sigma(x: np.ndarray) -> np.ndarray:
    """ELU + 1 with alpha = 1 ([HF] Memory Retrieval; reading R4)."""
    x = f64(x)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def sigma_grad(x: np.ndarray) -> np.ndarray:
    """Derivative of ELU + 1: 1 for x > 0, exp(x) otherwise (continuous at 0)."""
    x = f64(x)
    return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))


class Elu1:
    """The default feature map sigma = ELU + 1 (R4), D' = d features."""
    name = "elu1"

    @staticmethod
    def dim(d):
        return d

    @staticmethod
    def phi(x):
        return sigma(x)

    @staticmethod
    def vjp(x, g):
        """d<g, phi(x)>/dx for rows x (n, d) and g (n, D')."""
        return f64(g) * sigma_grad(x)

    @staticmethod
    def kernel(q, k):
        """phi(q) . phi(k) for single vectors."""
        return float(sigma(q) @ sigma(k))


class Taylor2:
    """Second-order Taylor feature map (R15; page "Based", section
    "고정 크기 순환 상태를 사용하는 방법도 중요합니다"):
    phi(x) = [1, x, x_a x_b / sqrt 2 (a major)], D' = 1 + d + d^2, so that
    phi(q) . phi(k) = 1 + q.k + (q.k)^2 / 2."""
    name = "taylor2"

    @staticmethod
    def dim(d):
        return 1 + d + d * d

    @staticmethod
    def phi(x):
        x = f64(x)
        n, d = x.shape
        quad = (x[:, :, None] * x[:, None, :]).reshape(n, d * d) / math.sqrt(2.0)
        return np.concatenate([np.ones((n, 1)), x, quad], axis=1)

    @staticmethod
    def vjp(x, g):
        x, g = f64(x), f64(g)
        n, d = x.shape
        G = g[:, 1 + d:].reshape(n, d, d)
        # d(x_a x_b)/dx_c = delta_ac x_b + x_a delta_bc
        quad = np.einsum("ncb,nb->nc", G, x) + np.einsum("nac,na->nc", G, x)
        return g[:, 1:1 + d] + quad / math.sqrt(2.0)

    @staticmethod
    def kernel(q, k):
        t = float(f64(q) @ f64(k))
        return 1.0 + t + 0.5 * t * t


FEATURE_MAPS = {"elu1": Elu1, "taylor2": Taylor2}


def gate(beta) -> np.ndarray:
    """g = sigmoid(beta) ([HF] Integration).  beta = -inf gives 0, +inf gives 1."""
    b = f64(beta)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-b))


def _dims(Q, K, seg_len):
    B, Hq, N, d = Q.shape
    Bk, Hkv, Nk, dk = K.shape
    assert (B, N, d) == (Bk, Nk, dk), "Q and K disagree in batch, length or head_dim"
    assert Hq % Hkv == 0, "query heads must be a multiple of K/V heads"
    return B, Hq, Hkv, N, d, Hq // Hkv, num_segments(N, seg_len)


def num_segments(N, seg_len):
    """Segments of a call: ceil(N / seg_len), the last one possibly shorter
    (R10); an empty call (N = 0) has none, so the state passes through (R13)."""
    assert N >= 0 and seg_len > 0
    return -(-N // seg_len)


def seg_rows(s, seg_len, N):
    """Token rows of segment s: [s L, min((s+1) L, N)) ([HF] Segmentation; R10)."""
    return slice(s * seg_len, min((s + 1) * seg_len, N))


def seq_lengths(lens, B, N):
    """Length of each sequence of the batch (R14); all N when lens is None."""
    if lens is None:
        return [N] * B
    out = [int(x) for x in np.asarray(lens).reshape(-1)]
    assert len(out) == B and all(0 <= x <= N for x in out), "lengths must lie in [0, N]"
    return out


def _state_or_zero(M0, z0, B, Hkv, d, fmap=Elu1):
    n = fmap.dim(d)
    M = np.zeros((B, Hkv, n, d)) if M0 is None else f64(M0).copy()
    z = np.zeros((B, Hkv, n)) if z0 is None else f64(z0).copy()
    return M, z


# ------------------------------------------------------------------ the steps

def local_attention(Qs, Ks, Vs, rows=None):
    """Causal softmax attention inside one segment ([HF] Local Attention).

    Qs: (L, d); Ks, Vs: (L, d).  Row i attends to keys j <= i of the same
    segment with scale 1/sqrt(d) (R3).  `rows` selects which query rows to
    return (all by default).  Returns (A_dot, P, lse) for those rows."""
    Qs, Ks, Vs = f64(Qs), f64(Ks), f64(Vs)
    L, d = Qs.shape
    rows = np.arange(L) if rows is None else np.asarray(rows)
    S = (Qs[rows] @ Ks.T) / math.sqrt(d)
    mask = np.arange(L)[None, :] > rows[:, None]
    S = np.where(mask, -np.inf, S)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    P = E / l
    return P @ Vs, P, (m + np.log(l))[:, 0]


def memory_retrieval(Qs, M, z, eps=EPS, fmap=Elu1):
    """A_mem = sigma(Q) M_{s-1} / (sigma(Q) z_{s-1} + eps) ([HF] Memory Retrieval; R1, R2),
    with fmap.phi in place of sigma (R15).

    Returns (A_mem, num, den, phi(Q))."""
    sQ = fmap.phi(Qs)
    num = sQ @ f64(M)
    den = sQ @ f64(z) + eps
    return num / den[:, None], num, den, sQ


def integrate(A_mem, A_dot, beta_h):
    """O = g A_mem + (1 - g) A_dot, g = sigmoid(beta_h) ([HF] Integration; R5)."""
    g = gate(beta_h)
    return g * A_mem + (1.0 - g) * A_dot


def memory_update(M, z, Ks, Vs, fmap=Elu1):
    """M_s = M_{s-1} + sigma(K)^T V and z_s = z_{s-1} + sum_rows sigma(K)
    ([HF] Memory Update; R1), with fmap.phi in place of sigma (R15).
    Returns new arrays."""
    sK = fmap.phi(Ks)
    return f64(M) + sK.T @ f64(Vs), f64(z) + sK.sum(axis=0)


# ------------------------------------------------------------------ forward

def state_sweep(K, V, seg_len, M0=None, z0=None, lens=None, fmap=Elu1):
    """Run only the memory path ([HF] Memory Update, State Transfer).

    Returns (Msnap, zsnap, M_S, z_S) where Msnap[b, k, s] is M_{s-1}, the state
    that segment s retrieves from (R6), and M_S the state after the last segment.
    With lens (R14) sequence b has ceil(lens[b] / seg_len) segments; its
    snapshots past them repeat its final state."""
    K, V = f64(K), f64(V)
    B, Hkv, N, d = K.shape
    S = num_segments(N, seg_len)
    nb = seq_lengths(lens, B, N)
    M, z = _state_or_zero(M0, z0, B, Hkv, d, fmap)
    Msnap = np.empty((B, Hkv, S) + M.shape[2:])
    zsnap = np.empty((B, Hkv, S) + z.shape[2:])
    for b in range(B):
        for k in range(Hkv):
            for s in range(S):
                Msnap[b, k, s] = M[b, k]
                zsnap[b, k, s] = z[b, k]
                if s >= num_segments(nb[b], seg_len):
                    continue
                r = seg_rows(s, seg_len, nb[b])
                M[b, k], z[b, k] = memory_update(M[b, k], z[b, k], K[b, k, r], V[b, k, r], fmap)
    return Msnap, zsnap, M, z


def segment_unit(Qs, Ks, Vs, Mprev, zprev, beta_h, rows=None, eps=EPS, fmap=Elu1):
    """Output rows of one (batch, query head, segment) unit given its M_{s-1}, z_{s-1}.

    Because the carried state is a prefix sum of per-segment terms, any unit
    is exact on its own once M_{s-1}, z_{s-1} are known; the benchmark and the
    full-size tests use this to check sampled rows."""
    Qs = f64(Qs)
    rows = np.arange(Qs.shape[0]) if rows is None else np.asarray(rows)
    A_dot, _, _ = local_attention(Qs, Ks, Vs, rows)
    A_mem, _, _, _ = memory_retrieval(Qs[rows], Mprev, zprev, eps, fmap)
    return integrate(A_mem, A_dot, beta_h)


def forward(Q, K, V, beta, seg_len, M0=None, z0=None, eps=EPS, want_lse=False, lens=None, fmap=Elu1):
    """Infini-attention forward over one call ([HF] all six steps, in order).

    Q: [B, Hq, N, d]; K, V: [B, Hkv, N, d]; beta: [Hq]; M0: [B, Hkv, d, d];
    z0: [B, Hkv, d] (None = empty memory).  Returns (O, M_S, z_S) and, with
    want_lse, the per-row log-sum-exp of the local attention scores.
    lens: optional per-sequence lengths (R14); rows past a sequence's length
    come out zero."""
    Q, K, V = f64(Q), f64(K), f64(V)
    B, Hq, Hkv, N, d, G, _ = _dims(Q, K, seg_len)
    nb = seq_lengths(lens, B, N)
    M, z = _state_or_zero(M0, z0, B, Hkv, d, fmap)
    O = np.zeros((B, Hq, N, d))
    lse = np.zeros((B, Hq, N))
    beta = f64(beta)
    for b in range(B):
        for k in range(Hkv):
            for s in range(num_segments(nb[b], seg_len)):       # Segmentation
                r = seg_rows(s, seg_len, nb[b])
                Ks, Vs = K[b, k, r], V[b, k, r]
                for h in range(k * G, (k + 1) * G):             # R7
                    Qs = Q[b, h, r]
                    A_dot, _, l = local_attention(Qs, Ks, Vs)   # Local Attention
                    A_mem, _, _, _ = memory_retrieval(Qs, M[b, k], z[b, k], eps, fmap)  # Retrieval
                    O[b, h, r] = integrate(A_mem, A_dot, beta[h])                        # Integration
                    lse[b, h, r] = l
                M[b, k], z[b, k] = memory_update(M[b, k], z[b, k], Ks, Vs, fmap)        # Update
                # State Transfer: nothing but (M, z) survives to the next segment.
    return (O, M, z, lse) if want_lse else (O, M, z)


def forward_per_token(Q, K, V, beta, seg_len, M0=None, z0=None, eps=EPS, fmap=Elu1):
    """Direct per-token evaluation, never forming M (linear-attention view, R1).

    For token i of segment s:
      A_dot_i = sum over keys j of segment s with j <= i of softmax_j(q_i.k_j / sqrt d) v_j
      A_mem_i = (phi(q_i) M0 + sum_{j before segment s} kappa(q_i, k_j) v_j)
                / (phi(q_i) z0 + sum_{j before segment s} kappa(q_i, k_j) + eps)
    where kappa(q, k) = phi(q).phi(k) is written out without any feature
    vector: sigma(q).sigma(k) with scalar loops for ELU + 1, and the closed
    form 1 + q.k + (q.k)^2 / 2 for the Taylor map (R15).  Explicit loops over
    tokens; for tiny inputs only."""
    Q, K, V = f64(Q), f64(K), f64(V)
    B, Hq, Hkv, N, d, G, S = _dims(Q, K, seg_len)
    n = fmap.dim(d)
    M0 = np.zeros((B, Hkv, n, d)) if M0 is None else f64(M0)
    z0 = np.zeros((B, Hkv, n)) if z0 is None else f64(z0)
    O = np.zeros((B, Hq, N, d))
    inv = 1.0 / math.sqrt(d)
    elu = lambda v: np.array([x + 1.0 if x > 0 else math.exp(x) for x in v])

    def kappa(q, k):
        if fmap is Taylor2:
            t = sum(q[c] * k[c] for c in range(d))
            return 1.0 + t + 0.5 * t * t
        return float(elu(q) @ elu(k))

    for b in range(B):
        for h in range(Hq):
            k = h // G
            g = 1.0 / (1.0 + math.exp(-float(beta[h]))) if np.isfinite(beta[h]) else float(beta[h] > 0)
            for i in range(N):
                s = i // seg_len
                start = s * seg_len
                q = Q[b, h, i]
                # local causal softmax, scalar loop over keys
                scores = [float(np.dot(q, K[b, k, j])) * inv for j in range(start, i + 1)]
                mx = max(scores)
                w = [math.exp(t - mx) for t in scores]
                tot = sum(w)
                a_dot = np.zeros(d)
                for t, j in enumerate(range(start, i + 1)):
                    a_dot += (w[t] / tot) * V[b, k, j]
                # memory as a sum over all earlier segments' tokens
                pq = elu(q) if fmap is Elu1 else fmap.phi(q[None, :])[0]
                num = pq @ M0[b, k]
                den = float(pq @ z0[b, k]) + eps
                for j in range(0, start):
                    a = kappa(q, K[b, k, j])
                    num = num + a * V[b, k, j]
                    den += a
                O[b, h, i] = g * (num / den) + (1.0 - g) * a_dot
    return O


# ------------------------------------------------------------------ backward

def backward(Q, K, V, beta, seg_len, dO, M0=None, z0=None, dM_S=None, dz_S=None, eps=EPS, lens=None,
             fmap=Elu1):
    """Exact gradient of `forward` (R9) for loss = <dO, O> + <dM_S, M_S> + <dz_S, z_S>.

    Returns dict with dQ, dK, dV, dbeta, dM0, dz0.  Steps, per (batch, K/V head),
    walking segments from last to first with dM = dLoss/dM_s carried:
      update:    dV_s += sigma(K_s) dM;  dsigma(K_s) = V_s dM^T + 1 dz^T
      gate:      dA_mem = g dO, dA_dot = (1-g) dO, dbeta += g(1-g) sum dO*(A_mem - A_dot)
      retrieval: dnum = dA_mem / den, dden = -rowsum(dA_mem * A_mem) / den,
                 dsigma(Q) = dnum M_{s-1}^T + dden z_{s-1}^T,
                 and dM += sigma(Q)^T dnum, dz += sigma(Q)^T dden  (giving dLoss/dM_{s-1})
      local:     dV += P^T dA_dot, dP = dA_dot V^T, dS = P * (dP - rowsum(P*dP)),
                 dQ += dS K / sqrt d, dK += dS^T Q / sqrt d."""
    Q, K, V, dO = f64(Q), f64(K), f64(V), f64(dO)
    B, Hq, Hkv, N, d, G, _ = _dims(Q, K, seg_len)
    nb = seq_lengths(lens, B, N)
    Msnap, zsnap, _, _ = state_sweep(K, V, seg_len, M0, z0, lens, fmap)
    n = fmap.dim(d)
    dM = np.zeros((B, Hkv, n, d)) if dM_S is None else f64(dM_S).copy()
    dz = np.zeros((B, Hkv, n)) if dz_S is None else f64(dz_S).copy()
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    dbeta = np.zeros(Hq)
    g_all = gate(beta)
    inv = 1.0 / math.sqrt(d)
    for b in range(B):
        for k in range(Hkv):
            for s in reversed(range(num_segments(nb[b], seg_len))):
                r = seg_rows(s, seg_len, nb[b])
                Ks, Vs = K[b, k, r], V[b, k, r]
                sK = fmap.phi(Ks)
                # memory update of segment s: M_s = M_{s-1} + sK^T V_s
                dsK = Vs @ dM[b, k].T + dz[b, k][None, :]
                dK[b, k, r] += fmap.vjp(Ks, dsK)
                dV[b, k, r] += sK @ dM[b, k]
                Mprev, zprev = Msnap[b, k, s], zsnap[b, k, s]
                addM = np.zeros((n, d))
                addz = np.zeros(n)
                for h in range(k * G, (k + 1) * G):
                    g = g_all[h]
                    Qs, dOs = Q[b, h, r], dO[b, h, r]
                    A_dot, P, _ = local_attention(Qs, Ks, Vs)
                    A_mem, num, den, sQ = memory_retrieval(Qs, Mprev, zprev, eps, fmap)
                    dA_mem = g * dOs
                    dA_dot = (1.0 - g) * dOs
                    dbeta[h] += g * (1.0 - g) * np.sum(dOs * (A_mem - A_dot))
                    # retrieval
                    dnum = dA_mem / den[:, None]
                    dden = -np.sum(dA_mem * A_mem, axis=1) / den
                    dsQ = dnum @ Mprev.T + dden[:, None] * zprev[None, :]
                    dQ[b, h, r] += fmap.vjp(Qs, dsQ)
                    addM += sQ.T @ dnum
                    addz += sQ.T @ dden
                    # local causal attention
                    dV[b, k, r] += P.T @ dA_dot
                    dP = dA_dot @ Vs.T
                    dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
                    dQ[b, h, r] += inv * (dS @ Ks)
                    dK[b, k, r] += inv * (dS.T @ Qs)
                dM[b, k] += addM
                dz[b, k] += addz
    return dict(dQ=dQ, dK=dK, dV=dV, dbeta=dbeta, dM0=dM, dz0=dz)


# ------------------------------------------------------------------ metrics

def state_bytes(batch, kv_heads, head_dim, seq_len, fmap=Elu1):
    """Bytes of the carried fp32 state (M, z) for a call of any length ([HF]
    State Transfer: only the fixed-size memory crosses segments).  The
    sequence length does not enter; the feature map sets the key dimension."""
    del seq_len
    n = fmap.dim(head_dim)
    return batch * kv_heads * (n * head_dim + n) * 4
