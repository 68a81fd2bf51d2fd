#!/usr/bin/env python3
"""Infini-attention forward throughput on one MI355X.

Workload (default): the Llama-3-8B head shape — B=4, 32 query heads sharing
8 K/V heads, head_dim 128, segments of 2048 tokens, 16 segments (32768
tokens), bf16 Q/K/V ~ N(0,1)/sqrt(128), beta ~ N(0,1), fp32 memory state;
seeded synthetic inputs (no dataset or trained weights exist for it here).

One step is one whole forward call over the batch: the memory phase
(infini_fwd_memory: sigma(K)^T V and sum sigma(K) per segment, exclusive
prefix over segments) followed by the attention phase (infini_fwd_attend:
causal softmax attention inside each segment, retrieval from the memory,
sigmoid gate).  Inputs are resident in HBM before the timed region.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from compressive_linear_memory_amd import inputs as I  # noqa: E402

PEAK_BF16_MFMA_TFLOPS = 2500.0
PEAK_FP32_VECTOR_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
METRIC = "Infini-attention fwd tokens/s at Llama-3-8B head shape; % bf16 MFMA peak"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(w: I.Workload):
    """Algorithmic work of one forward call (the method's own arithmetic and a
    single pass over every tensor; no masked-out upper triangle, no recompute)."""
    B, Hq, Hkv, L, S, d = w.batch, w.q_heads, w.kv_heads, w.seg_len, w.segments, w.head_dim
    eb = 4 if w.dtype == "fp32" else 2
    uq, ukv = B * Hq * S, B * Hkv * S
    local = 2 * 2 * d * L * (L + 1) / 2            # QK^T and PV over the causal lower triangle
    retrieval = 2 * L * d * d + 2 * L * d           # sigma(Q) M and sigma(Q) z
    update = 2 * L * d * d + L * d                  # sigma(K)^T V and sum sigma(K)
    n_q = B * Hq * w.seq_len * d
    n_kv = B * Hkv * w.seq_len * d
    state = B * Hkv * (d * d + d) * 4
    snaps = ukv * (d * d + d) * 4                   # per-segment state handed from phase 1 to phase 2
    return dict(
        attend_flop=uq * (local + retrieval),
        attend_bytes=eb * (2 * n_q + 2 * n_kv) + snaps,
        memory_flop=ukv * update,
        memory_bytes=eb * 2 * n_kv + snaps + state,
        step_flop=uq * (local + retrieval) + ukv * update,
        step_bytes=eb * (2 * n_q + 2 * n_kv) + 2 * state,
    )


def algorithmic_bwd_flop(w: I.Workload):
    """Matrix work of one backward call: the local backward's five causal
    products (recomputed scores, dP, dS K, dS^T Q, P^T dA_dot), the retrieval
    backward's three (A_mem, dnum M^T, sigma(Q)^T dnum) and the update
    backward's two (sigma(K) dM, V dM^T)."""
    B, Hq, Hkv, L, S, d = w.batch, w.q_heads, w.kv_heads, w.seg_len, w.segments, w.head_dim
    local = 5 * 2 * d * L * (L + 1) / 2
    return B * Hq * S * (local + 3 * 2 * L * d * d) + B * Hkv * S * 2 * 2 * L * d * d


def recorded_traffic(w, path):
    """HBM bytes per launch of the attention kernel from the committed counter
    summary, or None if there is none for this workload or the kernel source
    changed since the counters were taken."""
    import hashlib
    if w.name != "fwd_llama3_8b" or path != "mfma_bf16":
        return None
    prof = os.path.join(ROOT, "profiles", "fwd_llama3_8b_traffic.md")
    src = os.path.join(ROOT, "compressive_linear_memory_amd", "csrc", "fwd_mfma.hip")
    try:
        text = open(prof).read()
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except OSError:
        return None
    vals = dict(line.split(": ", 1) for line in text.splitlines()
                if line.startswith(("traffic_bytes_per_launch:", "kernel_source_sha256:")))
    if vals.get("kernel_source_sha256", "").strip() != sha:
        return None
    return float(vals["traffic_bytes_per_launch"])


def cpu_baseline(w, Q, K, V, beta, o_gpu_host_rows, budget_s=12.0):
    """Time the fp64 oracle on a bounded sample of the same workload, with
    numpy's BLAS given every core this process may run on."""
    import oracle as O
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threadpool_limits(limits=cores, user_api="blas")
        threads = max([t.get("num_threads", 1) for t in threadpool_info() if t.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    L = w.seg_len
    G = w.q_heads // w.kv_heads
    t0 = time.perf_counter()
    Msnap, zsnap, _, _ = O.state_sweep(K, V, L)
    t_sweep = time.perf_counter() - t0
    rng = np.random.default_rng(1234)
    units, t_units = 0, 0.0
    errs = []
    while t_units < budget_s and units < 1024:
        b = int(rng.integers(0, w.batch)); h = int(rng.integers(0, w.q_heads)); s = units % w.segments
        r = slice(s * L, (s + 1) * L)
        t1 = time.perf_counter()
        ref = O.segment_unit(Q[b, h, r], K[b, h // G, r], V[b, h // G, r], Msnap[b, h // G, s],
                             zsnap[b, h // G, s], beta[h])
        t_units += time.perf_counter() - t1
        units += 1
        got = o_gpu_host_rows(b, h, s)
        errs.append((np.max(np.abs(got - ref)), np.max(np.abs(ref))))
    per_unit = t_units / units
    total_units = w.batch * w.q_heads * w.segments
    est = t_sweep + per_unit * total_units
    tok = w.batch * w.seq_len
    err = max(e for e, _ in errs) / max(m for _, m in errs)
    return dict(value=tok / est, unit="tokens/s", cores=int(cores), blas_threads=int(threads), kind="oracle",
                sample=(f"full fp64 state sweep ({t_sweep:.2f} s) + {units} of {total_units} "
                        f"(batch, head, segment) units in full ({t_units:.2f} s); "
                        f"whole-workload time extrapolated as sweep + per-unit x units = {est:.1f} s")), err


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10,
                    help="untimed steps; the first few launches run slower while the GPU clocks ramp up")
    ap.add_argument("--workload", default="fwd_llama3_8b", choices=sorted(I.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", default="fwd", choices=["fwd", "train", "stream", "decode", "copy", "taylor"],
                    help="fwd: forward throughput (default, the headline line); train: forward + "
                         "backward step; stream: chained single-segment launches carrying the state; "
                         "decode: token-by-token streaming decode through one segment; "
                         "copy: a plain device copy of known size (calibrates HBM byte counters); "
                         "taylor: forward with the second-order Taylor feature map (200M-model shape)")
    ap.add_argument("--launches", type=int, default=512, help="stream mode: chained launches per step")
    ap.add_argument("--long-segments", action="store_true",
                    help="train mode: the --workload's own shape (default: 64-token training segments)")
    ap.add_argument("--graph", action="store_true",
                    help="stream mode: capture the chained launches of one step in a HIP graph and replay it; "
                         "fwd mode: also time the step replayed from a HIP graph (no per-call host work), "
                         "reported beside the eager step")
    ap.add_argument("--decode-tokens", type=int, default=0,
                    help="decode mode: decode only the last N tokens of the segment (the cache prefilled "
                         "with the rest); 0 = the whole segment")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the sequence-parallel "
              "multi-GPU path is a design note, not built", file=sys.stderr)
        sys.exit(2)
    if args.mode == "train":
        return bench_train(args)
    if args.mode == "stream":
        return bench_stream(args)
    if args.mode == "copy":
        return bench_copy(args)
    if args.mode == "decode":
        return bench_decode(args)
    if args.mode == "taylor":
        return bench_taylor(args)

    import torch
    from compressive_linear_memory_amd import binding as Bi
    Bi.lib()                                    # fail loudly if the HIP library is missing
    w = I.WORKLOADS[args.workload]
    if w.launches != 1:
        w = w.with_(launches=1)
    if w.segments > 16:
        raise SystemExit("bench times single-chunk workloads")
    say(f"[bench] generating {w.name} inputs")
    Q, K, V = I.qkv(w)
    beta = I.beta(w)
    tdt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    dev = torch.device("cuda:0")
    q = torch.from_numpy(Q).to(dev).to(tdt)
    k = torch.from_numpy(K).to(dev).to(tdt)
    v = torch.from_numpy(V).to(dev).to(tdt)
    b = torch.from_numpy(beta).to(dev)
    p = Bi.problem(q, k, w.seg_len)
    path = Bi.fwd_path(p)
    ws = torch.empty(Bi.workspace_bytes(p), dtype=torch.uint8, device=dev)
    O_ = torch.empty_like(q)
    B_, Hkv, d = w.batch, w.kv_heads, w.head_dim
    M_S = torch.empty((B_, Hkv, d, d), dtype=torch.float32, device=dev)
    z_S = torch.empty((B_, Hkv, d), dtype=torch.float32, device=dev)

    fused = path == "mfma_bf16_short"      # short segments: one fused kernel, no phases

    def step():
        if fused:
            Bi.attn_fwd(q, k, v, b, w.seg_len, out=(O_, M_S, z_S, None), ws=ws)
            return
        Bi.fwd_memory(p, k, v, None, None, M_S, z_S, ws)
        Bi.fwd_attend(p, q, k, v, b, O_, None, ws)

    say(f"[bench] path {path}; warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        if not fused:
            Bi.fwd_memory(p, k, v, None, None, M_S, z_S, ws)
        ev[i][1].record()
        if fused:
            Bi.attn_fwd(q, k, v, b, w.seg_len, out=(O_, M_S, z_S, None), ws=ws)
        else:
            Bi.fwd_attend(p, q, k, v, b, O_, None, ws)
        ev[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = ev[0][0].elapsed_time(ev[-1][2])
    mem_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    att_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    ms_step = total_ms / args.steps
    tokens = w.batch * w.seq_len
    value = tokens * args.steps / (total_ms / 1e3)
    say(f"[bench] {ms_step:.3f} ms/step (memory {mem_ms:.3f} ms, attend {att_ms:.3f} ms); wall {wall:.2f} s")

    graph_ms = None
    if args.graph:
        # the same step's launches recorded once and replayed: the GPU time of
        # the step without the binding's per-call host work
        import torch
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        g0, g1 = _events(2)
        g0.record()
        for _ in range(args.steps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.steps
        say(f"[bench] graph-replayed step {graph_ms:.4f} ms")

    alg = algorithmic(w)
    if fused:   # the one kernel does the whole step
        alg["attend_flop"] = alg["step_flop"]
    if path.startswith("mfma_bf16"):
        roof = dict(bound="mfma", peak=PEAK_BF16_MFMA_TFLOPS, unit="TFLOP/s")
        dtype = "bf16"
    else:
        roof = dict(bound="alu", peak=PEAK_FP32_VECTOR_TFLOPS, unit="TFLOP/s")
        dtype = "fp32"
    achieved = alg["attend_flop"] / (att_ms / 1e3) / 1e12
    if fused:   # short segments stream every tensor once at low arithmetic intensity
        roof = dict(bound="hbm", peak=PEAK_HBM_GBS, unit="GB/s")
        achieved = alg["step_bytes"] / (att_ms / 1e3) / 1e9
    roof.update(achieved=round(achieved, 3), frac=round(achieved / roof["peak"], 5),
                traffic=recorded_traffic(w, path), traffic_unit="HBM bytes per launch",
                kernel="infini_attn_fwd (fused)" if fused else "infini_fwd_attend",
                flop_per_launch=alg["attend_flop"], launch_ms=round(att_ms, 4))
    step_tflops = alg["step_flop"] / (ms_step / 1e3) / 1e12
    out = {
        "metric": METRIC if w.name == "fwd_llama3_8b" else f"Infini-attention fwd tokens/s ({w.name})",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
                   "head_dim": w.head_dim, "seg_len": w.seg_len, "segments": w.segments,
                   "seq_len": w.seq_len, "io_dtype": w.dtype, "kernel_path": path},
        "pct_bf16_mfma_peak": round(100 * step_tflops / PEAK_BF16_MFMA_TFLOPS, 3),
        "step_tflops": round(step_tflops, 3),
        "phases_ms": {"memory": round(mem_ms, 4), "attend": round(att_ms, 4)},
        "ms_per_step_graph": None if graph_ms is None else round(graph_ms, 4),
        "memory_phase_gbs": round(alg["memory_bytes"] / (mem_ms / 1e3) / 1e9, 1),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        say("[bench] timing the CPU oracle on a bounded sample")
        o_cpu = None

        def rows(bb, hh, ss):
            nonlocal o_cpu
            L = w.seg_len
            return O_[bb, hh, ss * L:(ss + 1) * L].float().cpu().numpy().astype(np.float64)

        cb, err = cpu_baseline(w, Q, K, V, beta, rows)
        out["cpu_baseline"] = cb
        out["parity_sampled_max_rel_err"] = float(err)
    print(json.dumps(out), flush=True)


def _events(n):
    import torch
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def bench_train(args):
    """Forward (with row log-sum-exp saved) + backward per step on the training workload.  The
    backward gets the forward's lse and final state (infini_attn_bwd_saved), as a training step
    that keeps them would pass them."""
    import torch
    from compressive_linear_memory_amd import binding as Bi
    Bi.lib()
    if args.long_segments:            # the forward workload's shape (2048-token segments)
        w = I.WORKLOADS[args.workload]
    else:
        w = I.WORKLOADS["train_llama3_8b"] if args.workload == "fwd_llama3_8b" else I.WORKLOADS[args.workload]
    say(f"[bench] generating {w.name} inputs")
    Q, K, V = I.qkv(w)
    dO = I.d_out(w)
    tdt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    dev = torch.device("cuda:0")
    t = lambda x: torch.from_numpy(x).to(dev).to(tdt)
    q, k, v, do = t(Q), t(K), t(V), t(dO)
    b = torch.from_numpy(I.beta(w)).to(dev)
    p = Bi.problem(q, k, w.seg_len)
    wsf = torch.empty(Bi.workspace_bytes(p), dtype=torch.uint8, device=dev)
    wsb = torch.empty(Bi.workspace_bytes(p, backward=True), dtype=torch.uint8, device=dev)
    B_, Hq, Hkv, N, d = w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim
    out = (torch.empty_like(q), torch.empty((B_, Hkv, d, d), device=dev), torch.empty((B_, Hkv, d), device=dev),
           torch.empty((B_, Hq, N), device=dev))

    def step(evs=None):
        if evs: evs[0].record()
        Bi.attn_fwd(q, k, v, b, w.seg_len, want_lse=True, out=out, ws=wsf)
        if evs: evs[1].record()
        Bi.attn_bwd(q, k, v, b, w.seg_len, do, lse=out[3], ws=wsb, state=(out[1], out[2]))
        if evs: evs[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [_events(3) for _ in range(args.steps)]
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    total = ev[0][0].elapsed_time(ev[-1][2])
    fwd = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    bwd = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    tok = w.batch * w.seq_len
    # Short training segments stream every tensor a few times at low arithmetic
    # intensity: the HBM roofline binds.  Algorithmic bytes: the forward's
    # (Q, K, V in, O out, state) plus the backward's (Q, K, V, dO, row LSE in;
    # dQ, dK, dV out; state).
    alg = algorithmic(w)
    eb = 4 if w.dtype == "fp32" else 2
    n_q, n_kv = B_ * Hq * N * d, B_ * Hkv * N * d
    bwd_bytes = eb * (2 * n_q + 2 * n_kv) + 4 * B_ * Hq * N + eb * (n_q + 2 * n_kv) + 2 * B_ * Hkv * (d * d + d) * 4
    step_bytes = alg["step_bytes"] + 4 * B_ * Hq * N + bwd_bytes
    if args.long_segments:
        # long segments: the causal products dominate and the matrix cores bind
        flop = alg["step_flop"] + algorithmic_bwd_flop(w)
        ach = flop / (total / args.steps / 1e3) / 1e12
        roof = dict(bound="mfma", peak=PEAK_BF16_MFMA_TFLOPS, unit="TFLOP/s", achieved=round(ach, 3),
                    frac=round(ach / PEAK_BF16_MFMA_TFLOPS, 5), traffic=None,
                    kernel="infini_attn_fwd + infini_attn_bwd_saved", flop_per_step=flop)
        name = w.name + "_train"
    else:
        ach = step_bytes / (total / args.steps / 1e3) / 1e9
        roof = dict(bound="hbm", peak=PEAK_HBM_GBS, unit="GB/s", achieved=round(ach, 1), frac=round(ach / PEAK_HBM_GBS, 5),
                    traffic=None, kernel="infini_attn_fwd + infini_attn_bwd_saved", bytes_per_step=step_bytes)
        name = w.name
    print(json.dumps({"metric": f"Infini-attention fwd+bwd tokens/s ({name})", "value": round(tok * args.steps / (total / 1e3), 1),
                      "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "ms_per_step": round(total / args.steps, 4), "higher_is_better": True, "scaling": "weak",
                      "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
                      "config": {"workload": name, "mode": "train", "kernel_path": Bi.fwd_path(p)},
                      "phases_ms": {"fwd": round(fwd, 4), "bwd": round(bwd, 4)}, "roofline": roof}), flush=True)


def bench_stream(args):
    """Chained single-segment launches carrying (M, z) between two state buffers.
    Inputs for 8 distinct launches are generated and cycled (same shapes and
    traffic as distinct inputs; the state still chains through every launch).

    Two schedules are timed.  Serial: one infini_attn_fwd per launch on one
    stream.  Pipelined (the reported value): one infini_fwd_stream call per
    step; the memory phase of every launch runs in order on one stream (it
    carries the state), and the attention phase of launch i, which needs only
    the state launch i retrieves from, runs on one of NPIPE streams as soon
    as its memory phase is done, so one launch's attention fills the compute
    units the previous launch's longest query tiles leave idle."""
    import torch
    from compressive_linear_memory_amd import binding as Bi
    Bi.lib()
    w = I.WORKLOADS["stream_1m"]
    dev = torch.device("cuda:0")
    say("[bench] generating stream_1m launch inputs (8 distinct launches, cycled)")
    nd = 8
    ins = []
    for t_ in range(nd):
        Q, K, V = I.qkv(w, launch=t_)
        ins.append(tuple(torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (Q, K, V)))
    b = torch.from_numpy(I.beta(w)).to(dev)
    p = Bi.problem(ins[0][0], ins[0][1], w.seg_len)
    ws = torch.empty(Bi.workspace_bytes(p), dtype=torch.uint8, device=dev)
    d, H = w.head_dim, w.kv_heads
    st = [(torch.zeros((1, H, d, d), device=dev), torch.zeros((1, H, d), device=dev)) for _ in range(2)]
    O_ = torch.empty_like(ins[0][0])
    nl = args.launches

    def run():
        for i in range(nl):
            q, k, v = ins[i % nd]
            src, dst = st[i & 1], st[(i + 1) & 1]
            Bi.attn_fwd(q, k, v, b, w.seg_len, M0=src[0], z0=src[1], out=(O_, dst[0], dst[1], None), ws=ws)

    NPIPE = 2                                   # groups in flight / attention streams (with the
                                                # memory stream and the current one, within the 4
                                                # hardware queues a process gets)
    GROUP = 4                                   # calls per attention launch
    # Pipelined: one infini_fwd_stream call per step issues all nl calls (the
    # memory phases of each group of GROUP calls as one run on sm, their
    # attention phases as one launch on sa[group % NPIPE]).
    wsp = torch.empty(max(Bi.stream_workspace_bytes(p, NPIPE, GROUP), NPIPE * Bi.workspace_bytes(p)),
                      dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(ins[0][0]) for _ in range(NPIPE * GROUP)]
    Mp, zp = torch.zeros_like(st[0][0]), torch.zeros_like(st[0][1])
    sm = torch.cuda.Stream()
    sa = [torch.cuda.Stream() for _ in range(NPIPE)]
    evs = [torch.cuda.Event() for _ in range(2 * NPIPE)]
    calls = Bi.StreamCalls(p, [ins[i % nd][0] for i in range(nl)], [ins[i % nd][1] for i in range(nl)],
                           [ins[i % nd][2] for i in range(nl)], b, Mp, zp,
                           [outs[i % (NPIPE * GROUP)] for i in range(nl)], wsp, NPIPE, GROUP, sm, sa, evs)

    def run_pipelined():
        cur = torch.cuda.current_stream()
        sm.wait_stream(cur)
        for s_ in sa:
            s_.wait_stream(cur)
        calls()
        cur.wait_stream(sm)
        for s_ in sa:
            cur.wait_stream(s_)

    # The same schedule issued call by call from Python through the phased
    # entry points (infini_fwd_memory / infini_fwd_attend) with torch events;
    # arguments marshalled once.
    L_ = Bi.lib()
    fm, fa = L_.infini_fwd_memory, L_.infini_fwd_attend
    P_ = lambda t: ctypes.c_void_p(t.data_ptr())
    pp = ctypes.byref(p)
    hm = ctypes.c_void_p(sm.cuda_stream)
    ha = [ctypes.c_void_p(x.cuda_stream) for x in sa]
    wsz = Bi.workspace_bytes(p)
    wsl = [wsp[r * wsz:(r + 1) * wsz] for r in range(NPIPE)]
    nws = ctypes.c_size_t(wsz)
    ev_mem, ev_att = evs[:NPIPE], evs[NPIPE:]
    percall = []
    for i in range(nl):
        r = i % NPIPE
        q, k, v = ins[i % nd]
        percall.append((r, (pp, P_(k), P_(v), P_(Mp), P_(zp), P_(st[1][0]), P_(st[1][1]), P_(wsl[r]), nws, hm),
                        (pp, P_(q), P_(k), P_(v), P_(b), P_(outs[r]), None, P_(wsl[r]), nws, ha[r]),
                        (pp, P_(k), P_(v), P_(st[1][0]), P_(st[1][1]), P_(Mp), P_(zp), P_(wsl[r]), nws, hm)))

    def run_pipelined_calls():
        cur = torch.cuda.current_stream()
        sm.wait_stream(cur)
        for s_ in sa:
            s_.wait_stream(cur)
        for i, (r, m_even, aargs, m_odd) in enumerate(percall):
            if i >= NPIPE:                      # slot r is reused once attention i - NPIPE is done
                sm.wait_event(ev_att[r])
            rc = fm(*(m_even if i % 2 == 0 else m_odd))   # state alternates between two buffers
            if rc:
                raise Bi.InfiniError(rc, "infini_fwd_memory")
            ev_mem[r].record(sm)
            sa[r].wait_event(ev_mem[r])
            rc = fa(*aargs)
            if rc:
                raise Bi.InfiniError(rc, "infini_fwd_attend")
            ev_att[r].record(sa[r])
        cur.wait_stream(sm)
        for s_ in sa:
            cur.wait_stream(s_)

    def timed(fn):
        e0, e1 = _events(2)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    for _ in range(max(1, args.warmup // 3)):
        run()
        run_pipelined()
        run_pipelined_calls()
    torch.cuda.synchronize()
    ms_serial = timed(run)

    def host_issue_us(fn):
        # host time to issue one step (no synchronisation inside)
        torch.cuda.synchronize()
        th0 = time.perf_counter()
        fn()
        us = (time.perf_counter() - th0) * 1e6 / nl
        torch.cuda.synchronize()
        return us

    host_lib, host_calls = host_issue_us(run_pipelined), host_issue_us(run_pipelined_calls)
    ms_lib, ms_calls = timed(run_pipelined), timed(run_pipelined_calls)
    if args.graph:
        # One step's launches recorded once and replayed: the host issues one
        # graph launch per step instead of two kernel launches per segment.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ms, schedule = timed(graph.replay), "serial, graph-replayed"
    elif ms_lib <= ms_calls:
        ms, schedule = ms_lib, "pipelined, one infini_fwd_stream call per step"
    else:
        ms, schedule = ms_calls, "pipelined, issued per call (infini_fwd_memory / infini_fwd_attend)"
    say(f"[bench] stream: {1e3 * ms_serial / nl:.2f} us/launch serial, {1e3 * ms_lib / nl:.2f} pipelined by "
        f"infini_fwd_stream (host {host_lib:.1f}), {1e3 * ms_calls / nl:.2f} pipelined per call (host "
        f"{host_calls:.1f}); reported: {schedule}")
    tok = w.seq_len * nl
    # Each launch is one 2048-token segment per head: matrix-core bound in
    # principle (arithmetic intensity ~545 flop/byte).
    alg = algorithmic(w.with_(launches=1))
    ach = alg["step_flop"] / (ms / nl / 1e3) / 1e12
    roof = dict(bound="mfma", peak=PEAK_BF16_MFMA_TFLOPS, unit="TFLOP/s", achieved=round(ach, 3),
                frac=round(ach / PEAK_BF16_MFMA_TFLOPS, 5), traffic=None,
                kernel="infini_attn_fwd (memory + attention) per launch", flop_per_launch=alg["step_flop"])
    print(json.dumps({"metric": "Infini-attention streaming fwd tokens/s (stream_1m)", "value": round(tok / (ms / 1e3), 1),
                      "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "ms_per_step": round(ms, 4), "us_per_launch": round(1e3 * ms / nl, 2),
                      "us_per_launch_serial": round(1e3 * ms_serial / nl, 2),
                      "us_per_launch_pipelined_stream_call": round(1e3 * ms_lib / nl, 2),
                      "us_per_launch_pipelined_per_call": round(1e3 * ms_calls / nl, 2),
                      "host_issue_us_per_launch": {"stream_call": round(host_lib, 2), "per_call": round(host_calls, 2)},
                      "higher_is_better": True,
                      "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": "stream_1m", "mode": "stream", "launches": nl,
                                 "schedule": schedule, "graph": bool(args.graph), "kernel_path": Bi.fwd_path(p)},
                      "roofline": roof}), flush=True)


def bench_decode(args):
    """Token-by-token decode through one whole segment of the streaming
    workload's shape (B=1, 32 heads, d=64, seg_len 2048), starting from a
    carried state; the last token completes the segment and folds it into the
    memory.  One step = the 2048 single-token calls, recorded once in a HIP
    graph and replayed (the eager per-token time is reported beside it)."""
    import torch
    from compressive_linear_memory_amd import binding as Bi
    Bi.lib()
    w = I.WORKLOADS["stream_1m"]
    dev = torch.device("cuda:0")
    say("[bench] generating decode inputs (one 2048-token segment of stream_1m)")
    Q, K, V = I.qkv(w, launch=1)
    Kp, Vp = I.qkv(w, launch=0)[1:]
    t = lambda x: torch.from_numpy(x).to(dev).to(torch.bfloat16)
    q, k, v = t(Q), t(K), t(V)
    b = torch.from_numpy(I.beta(w)).to(dev)
    B_, H, L, d = w.batch, w.kv_heads, w.seg_len, w.head_dim
    # the state after the previous segment, from the library itself
    M = torch.empty((B_, H, d, d), device=dev)
    z = torch.empty((B_, H, d), device=dev)
    Bi.attn_fwd(t(Kp), t(Kp), t(Vp), b, L, out=(torch.empty_like(q), M, z, None))
    kc = torch.zeros((B_, H, L, d), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    O_ = torch.empty((L, B_, w.q_heads, 1, d), dtype=torch.bfloat16, device=dev)   # one contiguous row block per token
    Mn = torch.empty_like(M)
    zn = torch.empty_like(z)
    p1 = Bi.problem(q[:, :, :1], k[:, :, :1], L)
    ws = torch.empty(max(Bi.lib().infini_decode_workspace_bytes(ctypes.byref(p1)), 1), dtype=torch.uint8,
                     device=dev)
    rows = [(q[:, :, i:i + 1].contiguous(), k[:, :, i:i + 1].contiguous(), v[:, :, i:i + 1].contiguous(),
             O_[i]) for i in range(L)]
    first = L - args.decode_tokens if 0 < args.decode_tokens < L else 0
    if first:   # the cache holds the segment's earlier rows already
        kc[:, :, :first] = k[:, :, :first]
        vc[:, :, :first] = v[:, :, :first]

    def run():
        for i in range(first, L):
            qi, ki, vi, oi = rows[i]
            Bi.decode(qi, ki, vi, b, L, i, kc, vc, M, z, out=oi, state_out=(Mn, zn), ws=ws)

    for _ in range(max(1, args.warmup // 5)):
        run()
    torch.cuda.synchronize()

    def timed(fn):
        e0, e1 = _events(2)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_eager = timed(run)
    # The same 2048 calls recorded once in a HIP graph: the GPU time of the
    # decode loop without the host's per-call cost.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    ms = timed(graph.replay)
    T = L - first                                   # tokens per step
    say(f"[bench] decode: {1e3 * ms_eager / T:.2f} us/token eager, {1e3 * ms / T:.2f} us/token graph-replayed")
    # Algorithmic bytes of the step's tokens decoded one by one: for token i the
    # cached rows 0..i of K and V, its own Q/K/V/O rows and the state read once;
    # the closing update reads the cache once and writes the state.
    eb = 2
    kv_rows = B_ * H * (L * (L + 1) // 2 - first * (first + 1) // 2)
    step_bytes = (eb * 2 * d * kv_rows + T * (eb * d * (2 * w.q_heads + 2 * H) + B_ * H * (d * d + d) * 4)
                  + eb * 2 * B_ * H * L * d + 2 * B_ * H * (d * d + d) * 4)
    ach = step_bytes / (ms / 1e3) / 1e9
    roof = dict(bound="hbm", peak=PEAK_HBM_GBS, unit="GB/s", achieved=round(ach, 1), frac=round(ach / PEAK_HBM_GBS, 5),
                traffic=None, kernel="infini_decode, one token per call", bytes_per_step=step_bytes)
    print(json.dumps({"metric": "Infini-attention streaming decode tokens/s (stream_1m shape, one token per call)",
                      "value": round(T / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
                      "warmup": args.warmup, "ms_per_step": round(ms, 4), "us_per_token": round(1e3 * ms / T, 2),
                      "us_per_token_eager": round(1e3 * ms_eager / T, 2), "graph": True, "tokens_per_step": T,
                      "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                      "data": "synthetic", "config": {"workload": "stream_1m", "mode": "decode", "seg_len": L, "tokens": T},
                      "roofline": roof}), flush=True)


def bench_taylor(args):
    """Forward with the second-order Taylor feature map on the 200M-model
    shape (B=8, H=12, d=64, seg_len 64, 16 segments, bf16).  The memory path
    carries 1 + d + d^2 = 4161 features per key.  With no starting state the
    matrix-core path forms the retrieval as polynomial-weighted attention over
    the earlier segments' keys and the final state from K and V; otherwise the
    fp32 vector kernels sweep the per-segment states."""
    import torch
    from compressive_linear_memory_amd import binding as Bi
    Bi.lib()
    w = I.WORKLOADS["fwd_200m"] if args.workload == "fwd_llama3_8b" else I.WORKLOADS[args.workload]
    say(f"[bench] generating {w.name} inputs (Taylor feature map)")
    Q, K, V = I.qkv(w)
    tdt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    dev = torch.device("cuda:0")
    t = lambda x: torch.from_numpy(x).to(dev).to(tdt)
    q, k, v = t(Q), t(K), t(V)
    b = torch.from_numpy(I.beta(w)).to(dev)
    p = Bi.problem(q, k, w.seg_len, "taylor2")
    ws = torch.empty(Bi.workspace_bytes(p), dtype=torch.uint8, device=dev)
    B_, Hq, Hkv, N, d, L, S = w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim, w.seg_len, w.segments
    nf = Bi.feature_dim(d, "taylor2")
    out = (torch.empty_like(q), torch.empty((B_, Hkv, nf, d), device=dev), torch.empty((B_, Hkv, nf), device=dev),
           None)

    def step():
        Bi.attn_fwd(q, k, v, b, L, out=out, ws=ws, feature_map="taylor2")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = _events(2)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    path = Bi.fwd_path(p)
    local = 2 * 2 * d * L * (L + 1) / 2
    if path == "mfma_bf16_taylor2":
        # algorithmic work of the kernel form: per (b, query head) the local
        # causal attention of every segment and the products with the earlier
        # segments' keys (segment s: s L keys for each of its L queries, score
        # and value products, 2 * 2 d per pair); per (b, K/V head) the state,
        # 2 N D' d for M and 2 N D' for z.  All on bf16 matrix cores.
        poly = 2 * 2 * d * L * L * S * (S - 1) / 2
        flop = B_ * Hq * (S * local + poly) + B_ * Hkv * (2 * N * nf * d + 2 * N * nf)
        bound, peak, kern = "mfma", PEAK_BF16_MFMA_TFLOPS, "infini_attn_fwd (Taylor map: state + polynomial attention)"
    else:
        # state form: local attention as for ELU + 1, retrieval 2 L D' d + 2 L D'
        # per (b, query head, segment), update 2 L D' d + L D' per (b, K/V head, segment)
        flop = B_ * Hq * S * (local + 2 * L * nf * d + 2 * L * nf) + B_ * Hkv * S * (2 * L * nf * d + L * nf)
        bound, peak, kern = "alu", PEAK_FP32_VECTOR_TFLOPS, "infini_attn_fwd (Taylor map: sweep + retrieval + attention)"
    ach = flop / (ms / 1e3) / 1e12
    roof = dict(bound=bound, peak=peak, unit="TFLOP/s", achieved=round(ach, 3), frac=round(ach / peak, 5),
                traffic=None, kernel=kern, flop_per_step=flop)
    print(json.dumps({"metric": f"Infini-attention fwd tokens/s, Taylor feature map ({w.name})",
                      "value": round(B_ * N / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
                      "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
                      "scaling": "weak", "vs_baseline": None,
                      "dtype": "bf16" if path == "mfma_bf16_taylor2" else "f32", "data": "synthetic",
                      "config": {"workload": w.name, "mode": "taylor", "feature_dim": nf, "io_dtype": w.dtype,
                                 "kernel_path": path},
                      "roofline": roof}), flush=True)


def bench_copy(args):
    """A plain 1 GiB device-to-device copy per step: the reference for scaling
    the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = 1 << 28                      # float32 elements = 1 GiB
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = _events(2)
    e0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    print(json.dumps({"metric": "device copy GB/s", "value": round(2 * n * 4 / (ms / 1e3) / 1e9, 1), "unit": "GB/s",
                      "bytes_read_per_step": n * 4, "bytes_written_per_step": n * 4, "ms_per_step": round(ms, 4),
                      "steps": args.steps, "warmup": args.warmup}), flush=True)


if __name__ == "__main__":
    main()
