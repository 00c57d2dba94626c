#!/usr/bin/env python
"""Throughput of the PaTH attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

A step is one full forward pass (path_attn_fwd_prepare: per-chunk UT
transform; path_attn_fwd_scan: right-to-left scan) over one batch of
synthetic inputs already resident in HBM.  Default workload: PaTH-FoX,
B=8, H=24, L=4096, d=64, bf16.  Other forward workloads: bf16_L1k,
fox_L16k, d128_L8k_prefill (B=2, H=32, L=8192, d=128).  With --workload
d128_L8k_decode the step is one decode step (in-place key-cache update +
one-token attention) and the 256 steps after that prefill are timed.  With
--workload transition_L4k the step is one path_transition_prep launch (w and
beta of every token from the layer input; B=8, L=4096, width 1536, rank 64,
H=24, d=64).  With --workload d128_L8k_kcache the step is one prefill ->
decode key-cache hand-off (path_kcache_from_prefill) after that prefill.
With --workload fox_L4k_bwd (or <forward workload>_bwd) the step is one
backward pass (path_attn_bwd) of that workload.

Prints one JSON line: effective TFLOP/s (2*B*H*L^2*d per forward), tokens/s,
the roofline of the dominant kernel (HIP events on its launch stream) and the
CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
MFMA_BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0                # MI355X HBM3E


def flop_model(B, H, L, d, C=64):
    """Algorithmic FLOPs of one forward with chunk C, as the library computes it:
      eff   2 L^2 d per head: QK^T and PV over the causal triangle, the count
            behind "effective TFLOP/s" (independent of the carry form)
      carry the query carried through every full chunk strictly between its
            own chunk and the key chunk: 2 d^2 C per (query chunk, chunk) pair
            with the d x d product (the rank-C form Q - (Q W^T) U would take
            4 C^2 d: twice as much at d = 64, the same at d = 128)
      diag  the own-chunk extras: Q W^T, the carry to the chunk start and the
            lower(Q W^T) Y correction
      prep  the per-chunk UT work (G, R, T^{-1}, U, Y, K~, and M = W^T U for
            the d x d carry), which the survey's count of the prepare stage
            also takes to cover the own-chunk extras
    "scan" is what the scan kernel computes: the prepare stage takes the
    own-chunk step (its extras and the own-chunk Q K^T, C^2 d per chunk).
    "alg" is the whole forward: eff + carry + prep."""
    N = (L + C - 1) // C
    pairs = (N - 1) * (N - 2) / 2.0
    f_eff = 2.0 * L * L * d
    f_carry = pairs * 2.0 * d * d * C
    f_prep = N * (12.0 * C * C * d + 4.0 * C ** 3 + 2.0 * C * d * d)
    BH = B * H
    f_scan = f_eff + f_carry - N * C * C * d
    return {"eff": BH * f_eff, "scan": BH * f_scan, "alg": BH * (f_eff + f_carry + f_prep)}


def _kernel_sha(name):
    with open(os.path.join(ROOT, "softmax_attention_ut_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(profile_md, kernel_src):
    """HBM bytes per launch from a committed rocprofv3 counter summary, only if
    it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", profile_md)
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    if not m or not h or h.group(1) != _kernel_sha(kernel_src):
        return None
    return float(m.group(1))


def host_cpu():
    """The host's CPU model, logical CPU count and the CPUs this process may
    run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0))}


def default_cpu_threads():
    """All the host cores this process is given: OMP_NUM_THREADS when the
    environment sets it (the share of a shared host), else the affinity set."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    return len(os.sched_getaffinity(0))


def cpu_baseline(inp, cfg, threads, heads):
    """The fp64 oracle (recurrent form), unmodified, on the first `heads`
    heads of the same inputs with `threads` OpenMP threads, then extrapolated
    to the whole job by the head count (heads are independent and equal in
    cost, so the job time is linear in them)."""
    import oracle
    BH = cfg.B * cfg.H
    n = max(1, min(heads, BH))
    sl = lambda t: None if t is None else t.reshape(-1, *t.shape[2:])[:n]
    t0 = time.perf_counter()
    _, _, _, used = oracle.recurrent(sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.w), sl(inp.beta),
                                     sl(inp.log_f), cfg.scale, nthreads=threads)
    dt = time.perf_counter() - t0
    t_full = dt * BH / n
    f = flop_model(cfg.B, cfg.H, cfg.L, cfg.d)
    res = {"value": f["eff"] / t_full / 1e12, "unit": "TFLOP/s (effective)",
           "cores": used, "kind": "oracle",
           "tokens_per_s": cfg.B * cfg.L / t_full,
           "extrapolated": n < BH, "extrapolation_factor": BH / n,
           "sample": f"{n} of {BH} heads, all {cfg.L} rows, fp64 recurrent oracle on {used} "
                     f"threads, {dt:.2f} s wall" + (f"; whole-job time extrapolated x{BH / n:.1f} "
                                                    f"by head count" if n < BH else "")}
    res.update(host_cpu())
    return res


def bench_fwd(args, cfg, torch, pa, inputs):
    inp = inputs.generate_config(cfg)
    B, H, L, d = cfg.B, cfg.H, cfg.L, cfg.d
    if inp.q.shape[2] != L:    # a prefill + decode workload: time its prefill
        inp = type(inp)(**{k: (None if t is None else t[:, :, :L].contiguous())
                           for k, t in vars(inp).items()})
    g = {k: (None if t is None else t.cuda()) for k, t in vars(inp).items()}
    nbytes = pa.path_attn_fwd_workspace_bytes(B, H, L, d, pa.PATH_BF16, 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(g["q"])
    lse = torch.empty(B, H, L, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        pa.path_attn_fwd_prepare(g["q"], g["k"], g["v"], g["w"], g["beta"], g["log_f"], cfg.scale,
                                 0, ws, stream)
        if ev:
            ev[1].record(stream)
        pa.path_attn_fwd_scan(g["q"], g["k"], g["v"], g["w"], g["log_f"], out, lse, cfg.scale,
                              0, ws, stream)
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / args.steps
    prep_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    scan_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    step_ev = sorted(e[0].elapsed_time(e[2]) for e in evs)
    f = flop_model(B, H, L, d)
    achieved = f["scan"] / (scan_ms * 1e-3) / 1e12
    # the committed counter summary covers the 4k FoX workload only
    traffic = _traffic("path_fwd_bf16_fox_L4k.md", "path_fwd_bf16.hip") if cfg.name == "fox_L4k" else None
    res = {
        "metric": f"PaTH fwd effective TFLOP/s + tokens/s (bf16, L={L}, d={d}) and % MFMA peak",
        "value": f["eff"] / (ms * 1e-3) / 1e12,
        "unit": "TFLOP/s (effective: 2*B*H*L^2*d per forward)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: PaTH-FoX forward B={B} H={H} L={L} d={d} "
                               f"bf16, chunk 64" if cfg.gate else
                               f"{cfg.name}: PaTH forward B={B} H={H} L={L} d={d} bf16",
                   "global_batch": B, "seq_len": L, "heads": H, "head_dim": d,
                   "forget_gate": cfg.gate, "parallelism": "single GPU"},
        "tokens_per_s": B * L / (ms * 1e-3),
        "tflops_algorithmic": f["alg"] / (ms * 1e-3) / 1e12,
        "mfma_peak_frac_algorithmic": f["alg"] / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "stage_ms": {"prepare(path_ut)": prep_ms, "scan(path_fwd)": scan_ms},
        # per-step HIP-event times (prepare + scan), inputs resident, L2 not flushed
        "step_ms_events": {"median": step_ev[len(step_ev) // 2], "min": step_ev[0],
                           "mean": sum(step_ev) / len(step_ev)},
        "l2_flushed": False,
        "roofline": {"kernel": (f"path_fwd_bf16_d64pp_kernel<{'true' if cfg.gate else 'false'}>" if d == 64
                                else f"path_fwd_bf16_d128pp_kernel<{'true' if cfg.gate else 'false'}>"),
                     "bound": "mfma",
                     "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": traffic,
                     "algorithmic_flops_per_launch": f["scan"]},
    }
    return res, inp


def bench_decode(args, cfg, torch, pa, inputs):
    inp = inputs.generate_config(cfg)
    g = {k: (None if t is None else t.cuda()) for k, t in vars(inp).items()}
    B, H, L, T, d = cfg.B, cfg.H, cfg.L, cfg.L_total, cfg.d
    pre = lambda t: t[:, :, :L].contiguous()
    page = args.page
    if page:
        # a pool of pages of `page` slots in a shuffled order (plus spares),
        # one block table row per sequence
        max_blocks = (T + page - 1) // page
        num_blocks = B * max_blocks + 8
        perm = torch.randperm(num_blocks, generator=torch.Generator().manual_seed(0))
        table = perm[:B * max_blocks].reshape(B, max_blocks).to(torch.int32).cuda()
        kc = torch.zeros(num_blocks, H, page, d, dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        kws = torch.empty(pa.path_kcache_workspace_bytes(B, H, L, d, pa.PATH_BF16),
                          dtype=torch.uint8, device="cuda")
        pa.path_kcache_from_prefill_paged(pre(g["k"]), pre(g["v"]), pre(g["w"]), pre(g["beta"]),
                                          kc, vc, table, kws)
    else:
        kc, vc = pa.kcache_from_prefill(pre(g["k"]), pre(g["v"]), pre(g["w"]), pre(g["beta"]), T)
    Tcap = max_blocks * page if page else T       # slots the cache holds
    fc = pa.fcache_from_prefill(pre(g["log_f"]), Tcap) if cfg.gate else None
    names = ("q", "k", "v", "w", "beta") + (("log_f",) if cfg.gate else ())
    steps_in = [{k: g[k][:, :, t].contiguous() for k in names} for t in range(L, T)]

    def step(s, t):
        if page:
            pa.path_decode_step_paged(kc, vc, table, s["q"], s["k"], s["v"], s["w"], s["beta"], o,
                                      ls, t, cfg.scale, f_cache=fc,
                                      log_f_t=s["log_f"] if cfg.gate else None, workspace=ws,
                                      stream=stream)
        elif cfg.gate:
            pa.path_decode_step_gated(kc, vc, fc, s["q"], s["k"], s["v"], s["w"], s["beta"],
                                      s["log_f"], o, ls, t, cfg.scale, ws, stream)
        else:
            pa.path_decode_step(kc, vc, s["q"], s["k"], s["v"], s["w"], s["beta"], o, ls, t,
                                cfg.scale, ws, stream)
    ws = pa.decode_workspace(B, H, Tcap, d, pa.PATH_BF16, kc.device)
    o = torch.empty(B, H, d, dtype=torch.bfloat16, device="cuda")
    ls = torch.empty(B, H, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    kc0, vc0 = kc.clone(), vc.clone()
    fc0 = fc.clone() if cfg.gate else None
    n = min(args.steps, T - L) if args.steps else T - L
    n = T - L if n <= 0 else n
    # warmup on a copy of the cache, then restore
    for i in range(min(args.warmup, n)):
        step(steps_in[i], L + i)
    kc.copy_(kc0)
    vc.copy_(vc0)
    if cfg.gate:
        fc.copy_(fc0)
    torch.cuda.synchronize()
    if args.graph:
        # the n steps captured once in a HIP graph, then replayed from the
        # restored caches: one launch for the whole run
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        outer = stream
        stream = side
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                for i in range(n):
                    step(steps_in[i], L + i)
        stream = outer
        kc.copy_(kc0)
        vc.copy_(vc0)
        if cfg.gate:
            fc.copy_(fc0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = wall * 1e3 / n
        step_ms = [e0.elapsed_time(e1) / n] * n
    else:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        t0 = time.perf_counter()
        ev[0].record(stream)
        for i in range(n):
            step(steps_in[i], L + i)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = wall * 1e3 / n
        step_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]
    # per key: read k, write k, read v (bf16), and with the gate read F_j (fp32)
    per_key = d * 2 * 3 + (4 if cfg.gate else 0)
    bytes_total = sum(B * H * ((L + i) * per_key + 4 * d * 2) for i in range(n))
    gbs = bytes_total / (sum(step_ms) * 1e-3) / 1e9
    res = {
        "metric": (f"PaTH{'-FoX' if cfg.gate else ''} decode tokens/s and HBM GB/s "
                   f"(bf16, d={d}, in-place key update)"),
        "value": B * n / (wall), "unit": "tokens/s",
        "n_gpus": 1, "steps": n, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {n} PaTH{'-FoX' if cfg.gate else ''} decode steps after a prefill of "
                               f"L={L}, B={B} H={H} d={d}, bf16 K/V cache"
                               + (f" in pages of {page} slots (shuffled block table)" if page else "")
                               + (", replayed from one HIP graph" if args.graph else ""),
                   "global_batch": B, "seq_len": L, "parallelism": "single GPU"},
        "roofline": {"kernel": f"path_decode_split_kernel<{d}, {'true' if cfg.gate else 'false'}, "
                               f"{'true' if page else 'false'}> + combine",
                     "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS,
                     "traffic": (_traffic("path_decode_d128_L8k.md", "path_decode.hip")
                                 if cfg.name == "d128_L8k_decode" and not page else None)},
    }
    return res, None


def bwd_flop_model(B, H, L, d, C=64):
    """FLOPs of one backward (d = C = 64, chunk C), per the algorithm the
    library runs:
      eff   5 L^2 d per head: the five products of attention's backward (S,
            dP = dO V^T, dV, dK, dQ) over the causal triangle, the count behind
            "effective TFLOP/s" (2.5 times the forward's 2 L^2 d)
      pairs per pair of chunks b < a: those five (5 * 2 C^2 d) and, for b >= 1,
            the query's transport Q P_b, the adjoint's G P_b^T and dM_b (3 * 2 C d^2)
      own   per chunk: the fourteen C x C x d products of the own-chunk step
            and of the carry to the chunk start, read backwards
      prep  the forward's UT work per chunk (recomputed): as in flop_model
      utb   per chunk: the UT transform's backward, seventeen C^3 products and
            the triangular substitution (C^3 / 3)
    "alg" = pairs + own + prep + utb."""
    N = (L + C - 1) // C
    pairs = N * (N - 1) / 2.0
    f_eff = 5.0 * L * L * d
    f_pairs = pairs * 10.0 * C * C * d + (pairs - (N - 1)) * 6.0 * C * d * d
    f_own = N * 14 * 2.0 * C * C * d
    f_prep = N * (12.0 * C * C * d + 4.0 * C ** 3 + 2.0 * C * d * d)
    f_utb = N * (17 * 2.0 * C ** 3 + C ** 3 / 3.0)
    BH = B * H
    return {"eff": BH * f_eff, "alg": BH * (f_pairs + f_own + f_prep + f_utb)}


def bwd_bytes_model(B, H, L, d, gate, C=64):
    """HBM bytes of one backward as the library runs it: the inputs q, k, v,
    w, out, d_out (bf16) and beta, lse (and log f) read once; the gradients
    dq, dk, dv, dw (fp32) and dbeta (and dlog f) written once; and the
    per-pair states of the blockwise algorithm, the query carried to key
    chunk b (N(N-1)/2 pairs) and the query's adjoint (pairs with b >= 1),
    64 x 64 bf16 each, written once, the queries read twice (the adjoint's
    pass and the key pass), the adjoints once.  The per-chunk tiles (about
    0.1 % of this at L = 4096) are left out."""
    N = (L + C - 1) // C
    BH = B * H
    io = BH * L * (6 * d * 2 + (3 if gate else 2) * 4) + BH * L * (4 * d * 4 + (2 if gate else 1) * 4)
    tile = C * d * 2
    pq, pg = N * (N - 1) // 2, (N - 1) * (N - 2) // 2
    states = BH * (3 * pq + 2 * pg) * tile
    return io + states


def bench_bwd(args, cfg, torch, pa, inputs):
    """One backward pass (path_attn_bwd: the per-chunk prepare, the query- and
    key-stationary kernels, the gate's suffix sums) after one forward of the
    same inputs, with d_out drawn once; everything resident in HBM."""
    import numpy as np
    inp = inputs.generate_config(cfg)
    B, H, L, d = cfg.B, cfg.H, cfg.L, cfg.d
    g = {k: (None if t is None else t.cuda()) for k, t in vars(inp).items()}
    rng = np.random.default_rng(cfg.seed + 1000)
    d_out = torch.from_numpy(rng.standard_normal((B, H, L, d)).astype(np.float32)).to(
        torch.bfloat16).cuda()
    out, lse = pa.attention(g["q"], g["k"], g["v"], g["w"], g["beta"], g["log_f"], scale=cfg.scale)
    ws = torch.empty(pa.path_attn_bwd_workspace_bytes(B, H, L, d, pa.PATH_BF16), dtype=torch.uint8,
                     device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    dq, dk, dv, dw = (torch.empty(B, H, L, d, **f32) for _ in range(4))
    dbeta = torch.empty(B, H, L, **f32)
    dlog_f = torch.empty(B, H, L, **f32) if cfg.gate else None
    stream = torch.cuda.current_stream()

    def step():
        pa.path_attn_bwd(g["q"], g["k"], g["v"], g["w"], g["beta"], g["log_f"], out, lse, d_out,
                         dq, dk, dv, dw, dbeta, dlog_f, cfg.scale, ws, stream)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in evs:
        e[0].record(stream)
        step()
        e[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / args.steps
    ev_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    f = bwd_flop_model(B, H, L, d)
    nbytes = bwd_bytes_model(B, H, L, d, cfg.gate)
    tflops = f["alg"] / (ev_ms * 1e-3) / 1e12
    gbs = nbytes / (ev_ms * 1e-3) / 1e9
    # the committed counter summary covers the 4k FoX workload only
    traffic = _traffic("path_bwd_fox_L4k.md", "path_bwd.hip") if cfg.name == "fox_L4k" else None
    res = {
        "metric": f"PaTH bwd effective TFLOP/s + tokens/s (bf16, L={L}, d={d}) and % MFMA peak",
        "value": f["eff"] / (ms * 1e-3) / 1e12,
        "unit": "TFLOP/s (effective: 5*B*H*L^2*d per backward)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}_bwd: PaTH{'-FoX' if cfg.gate else ''} backward "
                               f"B={B} H={H} L={L} d={d} bf16, chunk 64",
                   "global_batch": B, "seq_len": L, "heads": H, "head_dim": d,
                   "forget_gate": cfg.gate, "parallelism": "single GPU"},
        "tokens_per_s": B * L / (ms * 1e-3),
        "step_ms_events": ev_ms,
        "tflops_algorithmic": tflops,
        "mfma_peak_frac_algorithmic": tflops / MFMA_BF16_PEAK_TFLOPS,
        # the pair states make the design HBM-bound: its bytes at 8 TB/s take
        # longer than its flops at 2.5 PFLOP/s
        "roofline": {"kernel": "path_attn_bwd (path_ut_bf16_kernel<64,false,false> + "
                               "path_bwd_layout/own/chain/own_end/key/ut"
                               + ("/gate" if cfg.gate else "") + " kernels; HIP events around the call)",
                     "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": nbytes,
                     "algorithmic_flops_per_launch": f["alg"]},
    }
    return res, inp


def bwd_cpu_baseline(inp, cfg, L_sample, heads):
    """The fp64 oracle's backward (reverse-mode differentiation of the
    recurrent form, torch CPU ops), unmodified, on the first L_sample tokens
    of the first `heads` heads; its cost is quadratic in the length and linear
    in the heads, so the whole job's time is extrapolated by
    (L / L_sample)^2 * BH / heads."""
    import numpy as np
    import torch
    import oracle
    BH = cfg.B * cfg.H
    rng = np.random.default_rng(cfg.seed + 2000)
    flat = lambda t: None if t is None else t.reshape(-1, *t.shape[2:])
    q, k, v, w, beta, lf = (flat(t) for t in (inp.q, inp.k, inp.v, inp.w, inp.beta, inp.log_f))
    t0 = time.perf_counter()
    for h in range(heads):
        d_out = rng.standard_normal((L_sample, cfg.d))
        oracle.backward(q[h, :L_sample], k[h, :L_sample], v[h, :L_sample], w[h, :L_sample],
                        beta[h, :L_sample], None if lf is None else lf[h, :L_sample], cfg.scale,
                        d_out)
    dt = time.perf_counter() - t0
    factor = (cfg.L / L_sample) ** 2 * BH / heads
    t_full = dt * factor
    res = {"value": bwd_flop_model(cfg.B, cfg.H, cfg.L, cfg.d)["eff"] / t_full / 1e12,
           "unit": "TFLOP/s (effective)", "cores": torch.get_num_threads(), "kind": "oracle",
           "tokens_per_s": cfg.B * cfg.L / t_full, "extrapolated": True,
           "extrapolation_factor": factor,
           "sample": f"{heads} of {BH} heads, first {L_sample} of {cfg.L} tokens, fp64 autograd "
                     f"of the recurrent oracle, {dt:.2f} s wall; whole-job time extrapolated "
                     f"x{factor:.0f} (quadratic in length, linear in heads)"}
    res.update(host_cpu())
    return res


def kcache_bytes_flops(B, H, L, d, C=64, G=8):
    """Algorithmic HBM bytes and FLOPs of one prefill -> decode key-cache
    hand-off: read k, w, v (bf16) and beta, write the key and value caches'
    L slots; the UT work of every chunk (G, T^{-1}, Z, R, Y, K~: about
    N (8 C^2 d + 4 C^3)), the carry of every key to its group's end and of
    the d identity rows through the group (4 C^2 d per chunk passed), the
    suffix products of the group products (2 d^3 per group) and the product
    of every key with its group's suffix (2 d^2 per key), per head."""
    N = (L + C - 1) // C
    NG = (N + G - 1) // G
    nbytes = B * H * (5 * L * d * 2 + L * 4)
    carries = NG * (G * (G - 1) / 2 + G * d / C)     # chunk passes of 64 rows
    flops = B * H * (N * (8.0 * C * C * d + 4.0 * C ** 3) + carries * 4.0 * C * C * d
                     + (NG - 1) * 2.0 * d ** 3 + L * 2.0 * d * d)
    return nbytes, flops


def bench_kcache(args, cfg, torch, pa, inputs):
    """The prefill -> decode hand-off of a prefill + decode workload: the key
    cache H_{L-1} ... H_{j+1} k_j and the value cache after a prefill of L
    tokens, one path_kcache_from_prefill per step (the line's value), and the
    same caches by path_kcache_from_forward from the prefill forward's
    workspace (reported beside it)."""
    inp = inputs.generate_config(cfg)
    B, H, L, d, T = cfg.B, cfg.H, cfg.L, cfg.d, cfg.L_total
    g = {k: (None if t is None else t[:, :, :L].contiguous().cuda()) for k, t in vars(inp).items()}
    ws = torch.empty(pa.path_kcache_workspace_bytes(B, H, L, d, pa.PATH_BF16), dtype=torch.uint8,
                     device="cuda")
    kc = torch.zeros(B, H, T, d, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    stream = torch.cuda.current_stream()

    def step():
        pa.path_kcache_from_prefill(g["k"], g["v"], g["w"], g["beta"], kc, vc, ws, stream)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in evs:
        e[0].record(stream)
        step()
        e[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / args.steps
    ev_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    nbytes, flops = kcache_bytes_flops(B, H, L, d)
    gbs = nbytes / (ev_ms * 1e-3) / 1e9

    # the same caches from the workspace of the prefill's forward pass (its K~
    # and per-chunk -M^T): one forward fills the workspace, then the timed
    # calls read it
    fws = torch.empty(pa.path_attn_fwd_workspace_bytes(B, H, L, d, pa.PATH_BF16, 0),
                      dtype=torch.uint8, device="cuda")
    out = torch.empty_like(g["q"])
    lse = torch.empty(B, H, L, dtype=torch.float32, device="cuda")
    pa.path_attn_fwd(g["q"], g["k"], g["v"], g["w"], g["beta"], g["log_f"], out, lse, cfg.scale,
                     0, fws, stream)
    del out, lse

    def step_fwd():
        pa.path_kcache_from_forward(fws, g["v"], kc, vc, ws, stream)
    for _ in range(args.warmup):
        step_fwd()
    torch.cuda.synchronize()
    evf = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for e in evf:
        e[0].record(stream)
        step_fwd()
        e[1].record(stream)
    torch.cuda.synchronize()
    ff_ms = sum(a.elapsed_time(b) for a, b in evf) / args.steps
    # algorithmic bytes: K~ and -M^T read from the workspace, v read, both caches' L slots written
    N = (L + 63) // 64
    ff_bytes = B * H * (L * d * 2 * 4 + N * d * d * 2)
    res = {
        "metric": "PaTH prefill -> decode key-cache hand-off: ms and HBM GB/s",
        "value": ev_ms, "unit": "ms per hand-off (HIP events)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}_kcache: key and value caches after a prefill of "
                               f"L={L}, B={B} H={H} d={d}, bf16",
                   "global_batch": B, "seq_len": L, "parallelism": "single GPU"},
        "tflops": flops / (ev_ms * 1e-3) / 1e12,
        "roofline": {"kernel": f"path_kcache_from_prefill: path_ut_bf16_kernel<{d}, true, false> "
                               f"+ path_kcache_group/suffix/apply_kernel<{d}>",
                     "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS,
                     "traffic": (_traffic("path_kcache_d128_L8k.md", "path_kcache.hip")
                                 if cfg.name == "d128_L8k_decode" else None),
                     "algorithmic_bytes_per_launch": nbytes,
                     "algorithmic_flops_per_launch": flops},
        "from_forward": {"entry": "path_kcache_from_forward (after path_attn_fwd on the same inputs)",
                         "ms": ff_ms, "achieved_GBps": ff_bytes / (ff_ms * 1e-3) / 1e9,
                         "frac_of_hbm_peak": ff_bytes / (ff_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "algorithmic_bytes_per_launch": ff_bytes},
    }
    return res, None


def transition_bytes_flops(cfg):
    """Algorithmic HBM bytes and FLOPs of one path_transition_prep launch:
    read x (bf16) once and the weights once, write w (bf16) and beta (fp32);
    the low-rank map and the beta projection 2 (r + H) Dm per token, the up
    projection 2 H d r, the convolution and the norm 8 H d per token."""
    B, L, Dm, r, H, d = cfg.B, cfg.L, cfg.Dm, cfg.r, cfg.H, cfg.d
    weights = (r + H) * Dm * 2 + H * d * r * 2 + H * d * 3 * 4 + H * 4
    nbytes = B * L * Dm * 2 + B * H * L * d * 2 + B * H * L * 4 + weights
    flops = B * L * (2.0 * (r + H) * Dm + 2.0 * H * d * r + 8.0 * H * d)
    return nbytes, flops


def bench_transition(args, cfg, torch, pa, inputs):
    inp = inputs.generate_transition(cfg.B, cfg.L, cfg.Dm, cfg.r, cfg.H, cfg.d, seed=cfg.seed)
    g = {k: t.cuda() for k, t in vars(inp).items()}
    w = torch.empty(cfg.B, cfg.H, cfg.L, cfg.d, dtype=torch.bfloat16, device="cuda")
    beta = torch.empty(cfg.B, cfg.H, cfg.L, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        pa.path_transition_prep(g["x"], g["w_down"], g["w_up"], g["conv"], g["u"], g["b"], w,
                                beta, stream)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # one event pair around each launch, on the stream it is launched on
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in evs:
        e[0].record(stream)
        step()
        e[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / args.steps
    kern_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    nbytes, flops = transition_bytes_flops(cfg)
    gbs = nbytes / (kern_ms * 1e-3) / 1e9
    res = {
        "metric": "PaTH transition parameters (w, beta) from the layer input: tokens/s and HBM GB/s",
        "value": cfg.B * cfg.L / (ms * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: B={cfg.B} L={cfg.L} width={cfg.Dm} rank={cfg.r} "
                               f"H={cfg.H} d={cfg.d}, bf16 in, bf16 w + fp32 beta out",
                   "global_batch": cfg.B, "seq_len": cfg.L, "parallelism": "single GPU"},
        "tflops": flops / (kern_ms * 1e-3) / 1e12,
        "roofline": {"kernel": f"path_transition_kernel<{cfg.d}, {cfg.r}>", "bound": "hbm",
                     "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS,
                     "traffic": _traffic("path_transition_L4k.md", "path_transition.hip"),
                     "algorithmic_bytes_per_launch": nbytes},
    }
    return res, inp


def transition_cpu_baseline(inp, cfg, threads):
    """The fp64 oracle (numpy), unmodified, on the whole workload (well under
    a second of CPU time) with `threads` BLAS threads."""
    from threadpoolctl import threadpool_limits
    import oracle
    with threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        oracle.transition_prep(inp.x.double().numpy(), inp.w_down.double().numpy(),
                               inp.w_up.double().numpy(), inp.conv.double().numpy(),
                               inp.u.double().numpy(), inp.b.double().numpy(), cfg.d)
        dt = time.perf_counter() - t0
    return {"value": cfg.B * cfg.L / dt, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the whole workload ({cfg.B} x {cfg.L} tokens), fp64 numpy oracle, "
                      f"{dt:.2f} s wall"}


def copy_calibration(mib, torch):
    """A plain device-to-device copy of a known size: its FETCH_SIZE /
    WRITE_SIZE counters calibrate the HBM-traffic figures of the kernels."""
    n = mib * 2 ** 20
    x = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    y = torch.empty_like(x)
    for _ in range(2):
        y.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": ms,
                      "GB_per_s": 2 * n / (ms * 1e-3) / 1e9}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="fox_L4k")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="oracle baseline threads (default: all host cores given to this process)")
    ap.add_argument("--graph", action="store_true",
                    help="decode workloads: capture the timed steps in one HIP graph and replay it")
    ap.add_argument("--page", type=int, default=0,
                    help="decode workloads: use a paged K/V cache with pages of this many slots")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="heads the oracle baseline runs, the sample it extrapolates from "
                         "(default: two per thread, about 10-30 s of CPU work at the 4k workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (traffic-counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the PaTH hot path is data-parallel over "
              "independent (batch, head) pairs and this build runs on a single MI355X; "
              "run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import softmax_attention_ut_amd as pa
    from softmax_attention_ut_amd import inputs
    pa.load_library()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, torch)
        return
    if args.workload == "d128_L8k_prefill":    # the forward pass of the prefill + decode workload
        cfg = inputs.CONFIGS["d128_L8k_decode"]
        res, inp = bench_fwd(args, cfg, torch, pa, inputs)
        res["config"]["workload"] = (f"d128_L8k_prefill: PaTH forward B={cfg.B} H={cfg.H} "
                                     f"L={cfg.L} d={cfg.d} bf16 (the prefill of d128_L8k_decode)")
        print(json.dumps(res), flush=True)
        return
    if args.workload in inputs.TRANSITION_CONFIGS:
        cfg = inputs.TRANSITION_CONFIGS[args.workload]
        res, inp = bench_transition(args, cfg, torch, pa, inputs)
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = transition_cpu_baseline(inp, cfg, args.cpu_threads or default_cpu_threads())
        print(json.dumps(res), flush=True)
        return
    if args.workload.endswith("_bwd"):
        cfg = inputs.CONFIGS[args.workload[:-len("_bwd")]]
        res, inp = bench_bwd(args, cfg, torch, pa, inputs)
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = bwd_cpu_baseline(inp, cfg, 1024, 6)
        print(json.dumps(res), flush=True)
        return
    if args.workload.endswith("_kcache"):
        cfg = inputs.CONFIGS[args.workload[:-len("_kcache")] + "_decode"]
        res, _ = bench_kcache(args, cfg, torch, pa, inputs)
        print(json.dumps(res), flush=True)
        return
    cfg = inputs.CONFIGS[args.workload]
    if args.workload.endswith("_decode"):
        res, inp = bench_decode(args, cfg, torch, pa, inputs)
    else:
        res, inp = bench_fwd(args, cfg, torch, pa, inputs)
    if inp is not None and not args.no_cpu_baseline:
        threads = args.cpu_threads or default_cpu_threads()
        res["cpu_baseline"] = cpu_baseline(inp, cfg, threads, args.cpu_heads or 2 * threads)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
