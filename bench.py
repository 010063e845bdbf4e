#!/usr/bin/env python3
"""Benchmark of the log-linear attention (Mamba-2 form) hot path on one MI355X.

One step = one loglinear_fwd over the 16K-token workload (B=1, H=16, T=16384,
dk=128, dv=64, bf16 q/k/v, fp32 decay and lambda, chunk 64) followed, in a
second timed region, by one loglinear_decode_step over the batched decode
workload (64 sequences x 16 heads at positions drawn from U{1..32768}, fp32
Fenwick stacks of 17 slots).  Prints ONE JSON line on stdout.

  value        forward tokens/s (B*T / forward time), inputs resident in HBM
  roofline     of the dominant kernel (ll_chunk_walk): algorithmic HBM bytes
               per launch / its mean launch time against 8 TB/s.  The launch
               times come from HIP events that the library records as part of
               each kernel's dispatch on the launch stream (timing-only, no
               system fence), over a second pass of the same K steps; the
               first pass, with no events between launches, gives `value`
  decode       decode GB/s (algorithmic bytes / step time), tokens/s and its
               own roofline
  prefill      the forward that also writes the decode stack of the last
               position (loglinear_prefill, 17 slots): step time and the
               stack kernel's roofline
  backward     loglinear_bwd on the same workload (K/4 steps): step time,
               per-kernel times and the whole call's share of HBM peak for
               its mandatory bytes
  cpu_baseline the fp64 oracle on a bounded row sample of the same workload

Three input sets (3 x 218 MB) rotate through the forward steps and two
decode stacks (2 x 570 MB) through the decode steps, so no step finds its
inputs in the 256 MB MALL left there by the previous one.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
FP32_PEAK_TFLOPS = 157.3    # MI355X fp32 vector, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_ll_chunk_walk_fwd_bf16_T16K.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "log_linear_attention_amd", "csrc", f)
                  for f in ("ll_fwd.hip", "ll_device.h")]
FUSED_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_ll_fused_fwd_bf16_T16K.txt")
FUSED_SOURCES = [os.path.join(ROOT, "log_linear_attention_amd", "csrc", f)
                 for f in ("ll_fused.hip", "ll_device.h")]
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_ll_decode_bf16_S64.txt")
BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_ll_bwd_chunk_fwd_bf16_T16K.txt")
BWD_SOURCES = [os.path.join(ROOT, "log_linear_attention_amd", "csrc", f)
               for f in ("ll_bwd.hip", "ll_fwd.hip", "ll_device.h", "ll_internal.h")]
DECODE_SOURCES = [os.path.join(ROOT, "log_linear_attention_amd", "csrc", f)
                  for f in ("ll_decode.hip", "ll_device.h", "ll_internal.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(sources=None) -> str:
    """Hash of the kernel sources' code (comments and layout ignored)."""
    import re
    h = hashlib.sha256()
    for p in KERNEL_SOURCES if sources is None else sources:
        with open(p, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def fwd_algorithmic(cfg):
    """Mandatory HBM bytes and algorithmic flops of one forward.

    Bytes per (b, h): T*(2*dk + dv)*e (q, k, v) + 4T (a) + 4T*L (lambda) +
    T*dv*e (out).  Flops per (b, h): intra-chunk causal N*C(C+1)/2*2(dk+dv),
    chunk states N*2C*dk*dv, inter-chunk reads (sum over chunks c of
    popcount(c)) * 2C*dk*dv."""
    e = 2 if cfg.dtype == "bf16" else 4
    T, C, dk, dv, L = cfg.T, cfg.chunk, cfg.dk, cfg.dv, cfg.L
    BH = cfg.B * cfg.H
    per_bh_bytes = T * (2 * dk + dv) * e + 4 * T + 4 * T * L + T * dv * e
    N = (T + C - 1) // C
    pop = sum(bin(c).count("1") for c in range(N))
    per_bh_flops = N * C * (C + 1) // 2 * 2 * (dk + dv) + N * 2 * C * dk * dv + pop * 2 * C * dk * dv
    return BH * per_bh_bytes, BH * per_bh_flops


def decode_algorithmic(cfg, positions):
    """Algorithmic bytes of one decode step: every occupied incoming slot read
    once, the merged slot and the new token's slot written, plus the token,
    a, lambda, logscale (read + write) and the output."""
    e = 2 if cfg.dtype == "bf16" else 4
    slot = cfg.dk * cfg.dv * 4
    total = 0
    for t in positions:
        occ = 1 + bin(int(t) - 1).count("1") if t >= 1 else 0
        per_head = slot * (occ + (2 if t >= 1 else 1)) + (2 * cfg.dk + cfg.dv) * e + 4 * (1 + cfg.Lcap) \
            + 8 * cfg.Lcap + cfg.dv * e
        total += cfg.H * per_head
    return total


def auto_group_log2(cfg) -> int:
    """The forward's automatic group size: the largest g <= 3 whose groups of
    2^g chunks still give at least 512 workgroups of two groups each."""
    N = (cfg.T + cfg.chunk - 1) // cfg.chunk
    g = 0
    while g < 3 and (2 << g) <= N and cfg.B * cfg.H * ((N + (2 << g) - 1) // (2 << g)) >= 512:
        g += 1
    return g


def one_launch(cfg, group_log2: int) -> bool:
    """Whether the library runs this forward (and prefill) as its one-launch
    kernel: bf16, dk 128, dv 64, more than one 128-token group, automatic
    groups."""
    return group_log2 < 0 and cfg.dtype == "bf16" and cfg.dk == 128 and cfg.dv == 64 and cfg.T > 128


def stack_algorithmic(cfg, g: int, Lcap: int, fused: bool = False):
    """Algorithmic bytes of the prefill's stack export for the prompt's last
    position p = T-1: one stored block state (input dtype) per occupied
    bucket of whole groups, the group decay totals between those buckets and
    the last group (after the one-launch forward, whose groups are 128
    tokens: one Fenwick node total per such bucket), k, v and a of the keys
    of the last group (the finer buckets and the decays inside it), and the
    occupied slots and their log-scales written in fp32."""
    e = 2 if cfg.dtype == "bf16" else 4
    p = cfg.T - 1
    lgc = 7 if fused else (cfg.chunk << g).bit_length() - 1
    t0 = (p >> lgc) << lgc
    whole = bin(p >> lgc).count("1")
    n_groups = whole if fused else t0 >> lgc
    occ = 1 + bin(p).count("1")
    per_head = whole * cfg.dk * cfg.dv * e + 4 * n_groups + (p + 1 - t0) * ((cfg.dk + cfg.dv) * e + 4) \
        + occ * (cfg.dk * cfg.dv * 4 + 4)
    return cfg.B * cfg.H * per_head


def bwd_algorithmic(cfg):
    """Mandatory HBM bytes of one backward: q, k, v, do, a, lambda in and
    dq, dk, dv, da, dlambda out, once each."""
    e = 2 if cfg.dtype == "bf16" else 4
    T, dk, dv, L = cfg.T, cfg.dk, cfg.dv, cfg.L
    per_bh = T * (2 * dk + 2 * dv) * e + 4 * T + 4 * T * L + T * (2 * dk + dv) * e + 4 * T + 4 * T * L
    return cfg.B * cfg.H * per_bh


def bwd_chunk_algorithmic(cfg):
    """Mandatory HBM bytes of one ll_bwd_chunk launch: q, k, v, do, a and
    lambda of every token in, dk, dv, dlambda and the in-chunk part of da out
    (the level states it reads are intermediate, not counted)."""
    e = 2 if cfg.dtype == "bf16" else 4
    T, dk, dv, L = cfg.T, cfg.dk, cfg.dv, cfg.L
    per_bh = T * (2 * dk + 2 * dv) * e + 4 * T + 4 * T * L + T * (dk + dv) * e + 4 * T * L + 4 * T
    return cfg.B * cfg.H * per_bh


def read_traffic(path=TRAFFIC_FILE, sources=None):
    """Counter-measured HBM bytes per launch of a kernel (ll_chunk_walk by
    default) from its committed profile summary, or None if absent or taken
    on different kernel sources."""
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha") != source_hash(sources):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, cfg, n_rows: int, seed: int):
    import numpy as np

    import oracle

    rng = np.random.Generator(np.random.PCG64(seed))
    rows = np.stack([rng.integers(0, cfg.B * cfg.H, n_rows), rng.integers(0, cfg.T, n_rows)], axis=1)
    q, k, v, a, lam = (oracle._f64(inp[x]) for x in ("q", "k", "v", "a", "lam"))
    t0 = time.perf_counter()
    oracle.fwd_rows(q, k, v, a, lam, rows)
    dt = time.perf_counter() - t0
    # A token of the forward's `value` is one position of one sequence over
    # all H heads, i.e. H (head, position) rows.
    return {
        "value": round(n_rows / cfg.H / dt, 2),
        "unit": "tokens/s",
        "head_rows_per_s": round(n_rows / dt, 1),
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{n_rows} uniformly drawn (head, position) rows of the fwd_bf16_T16K workload "
                  f"(fp64 O(T^2) row sums, mean cost equal to a full-workload row) = {n_rows / cfg.H:.0f} "
                  f"tokens of {cfg.H} heads; {dt:.1f} s",
    }


def step_stats(torch, step, n):
    """Per-step device times of n calls of step(i), from one timing event
    recorded between consecutive steps on the current stream (a separate pass
    from the bracketed one that gives the mean): median, p10 and p90 in ms."""
    import numpy as np

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(n):
        step(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    d = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(n)])
    return {"median_ms": round(float(np.median(d)), 5), "p10_ms": round(float(np.percentile(d, 10)), 5),
            "p90_ms": round(float(np.percentile(d, 90)), 5), "n": n}


def measure_backward(ll, torch, dev, cfg, dsets, args, e0, e1):
    """loglinear_bwd on the forward's workload: K/2 timed steps after up to
    three warm-up steps, then the same steps with per-kernel events."""
    bws = torch.empty(ll.bwd_workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.chunk), dtype=torch.uint8,
                      device=dev)
    dout = torch.randn((cfg.B, cfg.H, cfg.T, cfg.dv), device=dev, generator=torch.Generator(device=dev).manual_seed(5)
                       ).to(cfg.torch_dtype)

    def bstep(i):
        d = dsets[i % 3]
        ll.bwd(d["q"], d["k"], d["v"], d["a"], d["lam"], dout, chunk=cfg.chunk, workspace=bws)

    bsteps = max(2, args.steps // 2)
    for i in range(min(args.warmup, 3)):
        bstep(i)
    torch.cuda.synchronize()
    e0.record()
    for i in range(bsteps):
        bstep(i)
    e1.record()
    torch.cuda.synchronize()
    bwd_ms = e0.elapsed_time(e1) / bsteps
    bwd_stats = step_stats(torch, bstep, bsteps)
    ll.profile_begin(16 * bsteps + 16)
    torch.cuda.synchronize()
    for i in range(bsteps):
        bstep(i)
    torch.cuda.synchronize()
    bk = {k: v[1] / v[0] for k, v in ll.profile_end().items()}
    bbytes = bwd_algorithmic(cfg)
    log(f"backward: {bwd_ms:.4f} ms/step; kernels: { {k: round(v * 1e3, 1) for k, v in bk.items()} }")
    dom = max(bk, key=bk.get)
    # roofline of the chunk kernel (the dominant one): its mandatory bytes
    # per launch over its mean launch time
    cbytes, cms = bwd_chunk_algorithmic(cfg), bk["ll_bwd_chunk"]
    return {
        "workload": "fwd_bf16_T16K gradients", "ms_per_step": round(bwd_ms, 5), "timing": bwd_stats,
        "tokens_per_s": round(cfg.B * cfg.T / (bwd_ms * 1e-3), 1),
        "algorithmic_bytes": bbytes,
        "kernels_ms": {k: round(v, 5) for k, v in bk.items()},
        "hbm_frac_whole_call": round(bbytes / (bwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "dominant_kernel": dom,
        "roofline": {"bound": "hbm", "achieved": round(cbytes / (cms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(cbytes / (cms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic(BWD_TRAFFIC_FILE, BWD_SOURCES),
                     "kernel": "ll_bwd_chunk", "kernel_avg_ms": round(cms, 5), "algorithmic_bytes": cbytes},
    }


def gdn_algorithmic(cfg, es: int = 4):
    """Algorithmic flops per kernel of the Log-Linear Gated DeltaNet forward
    and its mandatory bytes.  Per chunk of C (dk, dv): Q K^T and K K^T
    (lower half), the W solve, the carried queries, the in-chunk solve
    (C^3/3), the in-chunk output and pseudo-value solve, the transition
    W^T K and the chunk state; per tree merge dk x (dk + dv) x dk; per
    chunk-level bucket used by a chunk C x dk x dv plus, for each but the
    coarsest, C x dk x dk to carry the queries on."""
    T, C, dk, dv, L = cfg.T, cfg.chunk, cfg.dk, cfg.dv, cfg.L
    BH = cfg.B * cfg.H
    N = (T + C - 1) // C
    chunk = 2 * C * C * dk + C * C * dk + C * C * dk + C * C * dk + C ** 3 // 3 + C * C * dv + C * C * dv \
        + 2 * C * dk * dk + 2 * C * dk * dv
    P = (N - 1).bit_length() - 1 if N > 1 else 0
    merges = sum(N >> p for p in range(1, P + 1))
    tree = merges * 2 * dk * (dk + dv) * dk
    walk = 0
    for c in range(1, N):
        pc = bin(c).count("1")
        walk += pc * 2 * C * dk * dv + (pc - 1) * 2 * C * dk * dk
    flops = {"ll_gdn_chunk": BH * N * chunk, "ll_gdn_tree": BH * tree, "ll_gdn_walk": BH * walk}
    nbytes = BH * T * ((2 * dk + 2 * dv) * es + (2 + L) * 4)   # q, k, v, out in the input dtype
    return flops, nbytes


def measure_gdn(ll, torch, dev, args, e0, e1, bf16=False):
    """The Log-Linear Gated DeltaNet forward at the 16K shape: float32
    inputs, or the same inputs rounded to bf16 (float32 arithmetic)."""
    import synth

    cfg = synth.WORKLOADS["gdn_f32_T16K"]
    d = {k: v.to(dev) for k, v in synth.make_gdn_inputs(cfg).items()}
    if bf16:
        for n in ("q", "k", "v"):
            d[n] = d[n].to(torch.bfloat16)
    out = torch.empty((cfg.B, cfg.H, cfg.T, cfg.dv), dtype=d["q"].dtype, device=dev)
    ws = torch.empty(ll.gdn_fwd_workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.chunk), dtype=torch.uint8,
                     device=dev)

    def step():
        ll.gdn_fwd(d["q"], d["k"], d["v"], d["a"], d["beta"], d["lam"], chunk=cfg.chunk, out=out, workspace=ws)

    n = max(2, args.steps // 2)
    for _ in range(min(args.warmup, 3)):
        step()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    gstats = step_stats(torch, lambda i: step(), n)
    ll.profile_begin(16 * n + 16)
    torch.cuda.synchronize()
    for _ in range(n):
        step()
    torch.cuda.synchronize()
    stats = ll.profile_end()
    ks = {k: v[1] / n for k, v in stats.items()}   # per step (the tree kernel runs once per level)
    flops, nbytes = gdn_algorithmic(cfg, 2 if bf16 else 4)
    dom = max(ks, key=ks.get)
    launches = stats[dom][0] / n
    achieved = flops[dom] / (ks[dom] * 1e-3) / 1e12
    log(f"gdn ({'bf16' if bf16 else 'f32'} inputs): {ms:.4f} ms/step; kernels (ms per step): "
        f"{ {k: round(v, 4) for k, v in ks.items()} }")
    return {
        "workload": cfg.name, "dtype": "f32", "inputs": "bf16" if bf16 else "f32", "ms_per_step": round(ms, 5),
        "timing": gstats,
        "tokens_per_s": round(cfg.B * cfg.T / (ms * 1e-3), 1),
        "kernels_ms_per_step": {k: round(v, 5) for k, v in ks.items()},
        "algorithmic_flops": flops, "mandatory_bytes": nbytes,
        "roofline": {"bound": "alu", "achieved": round(achieved, 2), "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / FP32_PEAK_TFLOPS, 4), "traffic": None, "kernel": dom,
                     "kernel_avg_ms": round(ks[dom] / launches, 5)},
    }


def measure_grouped(ll, torch, cfg, dsets, args, e0, e1, Hqk):
    """The forward of the same workload with q and k shared by groups of
    H/Hqk heads (the first Hqk q/k heads of each input set): K timed steps,
    then per-kernel times.  Mandatory bytes drop by the q/k heads not read."""
    gsets = [dict(d, q=d["q"][:, :Hqk].contiguous(), k=d["k"][:, :Hqk].contiguous()) for d in dsets]
    out = torch.empty((cfg.B, cfg.H, cfg.T, cfg.dv), dtype=cfg.torch_dtype, device=dsets[0]["q"].device)
    ws = ll.alloc_workspace(cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.chunk, args.group_log2)

    def step(i):
        d = gsets[i % 3]
        ll.fwd(d["q"], d["k"], d["v"], d["a"], d["lam"], chunk=cfg.chunk, out=out, workspace=ws,
               group_log2=args.group_log2)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    qstats = step_stats(torch, step, args.steps)
    ll.profile_begin(8 * args.steps + 8)
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ks = {k: v[1] / v[0] for k, v in ll.profile_end().items()}
    e = 2 if cfg.dtype == "bf16" else 4
    fbytes, _ = fwd_algorithmic(cfg)
    gbytes = fbytes - cfg.B * (cfg.H - Hqk) * cfg.T * 2 * cfg.dk * e
    dom = max(ks, key=ks.get)
    walk_gbs = gbytes / (ks[dom] * 1e-3) / 1e9
    log(f"grouped forward Hqk={Hqk}: {ms:.4f} ms/step; {dom} {ks[dom] * 1e3:.1f} us, {walk_gbs:.1f} GB/s")
    return {
        "workload": f"fwd_bf16_T16K with {Hqk} q/k heads for {cfg.H} heads", "Hqk": Hqk,
        "ms_per_step": round(ms, 5), "timing": qstats, "tokens_per_s": round(cfg.B * cfg.T / (ms * 1e-3), 1),
        "algorithmic_bytes": gbytes, "kernels_ms": {k: round(v, 5) for k, v in ks.items()},
        "dominant_kernel": dom, "dominant_hbm_frac": round(walk_gbs / HBM_PEAK_GBS, 4),
    }


def measure_fwd_workload(ll, torch, dev, name, args, e0, e1, wall=False):
    """The forward on another workload (the 2K batch or the 64K long
    context): K timed steps over rotating input sets whose combined size
    exceeds 512 MB (so no step finds its inputs in the 256 MB MALL), the
    per-step distribution, per-kernel times, and for small workloads the host
    wall-clock of one call followed by a stream synchronisation."""
    import synth

    cfg = synth.WORKLOADS[name]
    base = {k: v.to(dev) for k, v in synth.make_fwd_inputs(cfg).items()}
    set_bytes = sum(t.numel() * t.element_size() for t in base.values())
    nsets = max(3, -(-(512 << 20) // set_bytes) + 1)
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(nsets - 1)]
    out = torch.empty((cfg.B, cfg.H, cfg.T, cfg.dv), dtype=cfg.torch_dtype, device=dev)
    ws = ll.alloc_workspace(cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.chunk)

    def step(i):
        d = sets[i % nsets]
        ll.fwd(d["q"], d["k"], d["v"], d["a"], d["lam"], chunk=cfg.chunk, out=out, workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    stats = step_stats(torch, step, args.steps)
    ll.profile_begin(8 * args.steps + 8)
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ks = {k: v[1] / v[0] for k, v in ll.profile_end().items()}
    fbytes, fflops = fwd_algorithmic(cfg)
    dom = max(ks, key=ks.get)
    dom_gbs = fbytes / (ks[dom] * 1e-3) / 1e9
    res = {
        "workload": name, "B": cfg.B, "H": cfg.H, "T": cfg.T, "a_scale": cfg.a_scale,
        "ms_per_step": round(ms, 5), "timing": stats, "tokens_per_s": round(cfg.B * cfg.T / (ms * 1e-3), 1),
        "input_sets": nsets, "algorithmic_bytes": fbytes, "algorithmic_flops": fflops,
        "hbm_frac_whole_call": round(fbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "mfma_frac_whole_call": round(fflops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "kernels_ms": {k: round(v, 5) for k, v in ks.items()},
        "roofline": {"bound": "hbm", "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": dom,
                     "kernel_avg_ms": round(ks[dom], 5)},
    }
    if wall:
        import numpy as np

        w = []
        for i in range(args.steps):
            t0 = time.perf_counter()
            step(i)
            torch.cuda.synchronize()
            w.append((time.perf_counter() - t0) * 1e3)
        res["host_wall_ms_per_call"] = {"median": round(float(np.median(w)), 4),
                                        "p10": round(float(np.percentile(w, 10)), 4),
                                        "p90": round(float(np.percentile(w, 90)), 4)}
    log(f"{name}: {ms:.4f} ms/step, {res['tokens_per_s'] / 1e6:.1f} M tokens/s; kernels {res['kernels_ms']}")
    del sets, base
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-rows", type=int, default=98304, help="oracle rows timed for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 1 GiB device copy first (reference kernel for counter scaling)")
    ap.add_argument("--group-log2", type=int, default=-1)
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward measurement")
    ap.add_argument("--no-gdn", action="store_true", help="skip the Gated DeltaNet measurement")
    ap.add_argument("--no-grouped", action="store_true", help="skip the shared q/k measurement")
    ap.add_argument("--no-other-workloads", action="store_true", help="skip the 2K and 64K forward workloads")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import log_linear_attention_amd as ll
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.WORKLOADS["fwd_bf16_T16K"]
    dcfg = synth.WORKLOADS["decode_bf16_S64"]

    if args.calib_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    log("generating inputs ...")
    host_sets = [synth.make_fwd_inputs(cfg, seed=cfg.seed + i) for i in range(3)]
    dsets = [{k: v.to(dev) for k, v in s.items()} for s in host_sets]
    out = torch.empty((cfg.B, cfg.H, cfg.T, cfg.dv), dtype=cfg.torch_dtype, device=dev)
    ws = ll.alloc_workspace(cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.chunk, args.group_log2)

    def fwd(i):
        d = dsets[i % 3]
        ll.fwd(d["q"], d["k"], d["v"], d["a"], d["lam"], chunk=cfg.chunk, out=out, workspace=ws,
               group_log2=args.group_log2)

    for i in range(args.warmup):
        fwd(i)
    torch.cuda.synchronize()

    # Timed region: K forward steps with nothing between the library's own
    # launches.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        fwd(i)
    e1.record()
    torch.cuda.synchronize()
    w1 = time.perf_counter()
    fwd_ms = e0.elapsed_time(e1) / args.steps
    fwd_stats = step_stats(torch, fwd, args.steps)
    # Per-kernel durations: the same K steps again, with HIP events recorded
    # around each launch on the launch stream by the library's profiler.
    ll.profile_begin(8 * args.steps + 8)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        fwd(i)
    e1.record()
    torch.cuda.synchronize()
    kstats = ll.profile_end()
    log(f"forward: {fwd_ms:.4f} ms/step (with per-kernel events {e0.elapsed_time(e1) / args.steps:.4f}; "
        f"wall {(w1 - w0) * 1e3 / args.steps:.4f}); kernels: {kstats}")

    fbytes, fflops = fwd_algorithmic(cfg)
    # the dominant kernel: the one with the most device time per step
    dom = max(kstats, key=lambda n: kstats[n][1])
    dom_launches, dom_ms = kstats[dom]
    dom_avg_ms = dom_ms / dom_launches
    achieved = fbytes / (dom_avg_ms * 1e-3) / 1e9
    traffic = read_traffic() if dom == "ll_chunk_walk" else read_traffic(FUSED_TRAFFIC_FILE, FUSED_SOURCES)
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
        "kernel": dom, "kernel_avg_ms": round(dom_avg_ms, 5),
    }
    whole_gbs = fbytes / (fwd_ms * 1e-3) / 1e9
    mfma_tflops = fflops / (fwd_ms * 1e-3) / 1e12

    # ---- decode ---------------------------------------------------------
    log("generating decode stacks ...")
    dec_host = [synth.make_decode_inputs(dcfg, seed=dcfg.seed + i) for i in range(2)]
    pos0 = dec_host[0]["pos"].numpy()
    for s in dec_host[1:]:
        s["pos"] = dec_host[0]["pos"].clone()  # same positions: same work per step
    dec = [{k: v.to(dev) for k, v in s.items()} for s in dec_host]
    del dec_host
    dout = torch.empty((dcfg.S, dcfg.H, dcfg.dv), dtype=dcfg.torch_dtype, device=dev)

    def dstep(i):
        d = dec[i % 2]
        ll.decode_step(d["q"], d["k"], d["v"], d["a"], d["lam"], d["state"], d["logscale"], d["pos"], out=dout)

    for i in range(args.warmup):
        dstep(i)
    torch.cuda.synchronize()
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        dstep(i)
    e1.record()
    torch.cuda.synchronize()
    dec_ms = e0.elapsed_time(e1) / args.steps
    dec_stats = step_stats(torch, dstep, args.steps)
    ll.profile_begin(4 * args.steps + 4)
    torch.cuda.synchronize()
    for i in range(args.steps):
        dstep(i)
    torch.cuda.synchronize()
    dstats = ll.profile_end()
    dbytes = decode_algorithmic(dcfg, pos0)
    dl, dms = dstats["ll_decode"]
    dec_kernel_ms = dms / dl
    dec_gbs = dbytes / (dec_kernel_ms * 1e-3) / 1e9
    log(f"decode: {dec_ms:.4f} ms/step, kernel {dec_kernel_ms:.4f} ms, {dec_gbs:.1f} GB/s")

    # ---- prefill: the forward plus the decode stack of the last position ----
    Lcap = 17
    g_used = args.group_log2 if args.group_log2 >= 0 else auto_group_log2(cfg)
    pstate = torch.empty((cfg.B, cfg.H, Lcap, cfg.dk, cfg.dv), dtype=torch.float32, device=dev)
    plog = torch.empty((cfg.B, cfg.H, Lcap), dtype=torch.float32, device=dev)

    def pstep(i):
        d = dsets[i % 3]
        ll.prefill(d["q"], d["k"], d["v"], d["a"], d["lam"], pstate, plog, chunk=cfg.chunk, out=out,
                   workspace=ws, group_log2=args.group_log2)

    for i in range(args.warmup):
        pstep(i)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        pstep(i)
    e1.record()
    torch.cuda.synchronize()
    pre_ms = e0.elapsed_time(e1) / args.steps
    pre_stats = step_stats(torch, pstep, args.steps)
    ll.profile_begin(8 * args.steps + 8)
    torch.cuda.synchronize()
    for i in range(args.steps):
        pstep(i)
    torch.cuda.synchronize()
    pstats = ll.profile_end()
    sl, sms = pstats["ll_prefill_stack"]
    stack_ms = sms / sl
    sbytes = stack_algorithmic(cfg, g_used, Lcap, fused=one_launch(cfg, args.group_log2))
    stack_gbs = sbytes / (stack_ms * 1e-3) / 1e9
    log(f"prefill: {pre_ms:.4f} ms/step (forward alone {fwd_ms:.4f}); stack kernel {stack_ms:.4f} ms, "
        f"{stack_gbs:.1f} GB/s")

    # ---- the other forward workloads: the 2K batch and the 64K long context ----
    others = None
    if not args.no_other_workloads:
        others = {"fwd_bf16_T2K": measure_fwd_workload(ll, torch, dev, "fwd_bf16_T2K", args, e0, e1, wall=True),
                  "fwd_bf16_T64K": measure_fwd_workload(ll, torch, dev, "fwd_bf16_T64K", args, e0, e1)}

    # ---- q/k shared across heads: the same forward with fewer q/k heads ----
    grouped = None if args.no_grouped else [measure_grouped(ll, torch, cfg, dsets, args, e0, e1, hq)
                                            for hq in (4, 1)]

    # ---- Log-Linear Gated DeltaNet forward ----
    gdn_res = None if args.no_gdn else [measure_gdn(ll, torch, dev, args, e0, e1, bf16=b) for b in (False, True)]

    # ---- backward: gradients of the forward on the same workload ----
    backward = None if args.no_bwd else measure_backward(ll, torch, dev, cfg, dsets, args, e0, e1)

    result = {
        "metric": "tokens/s, log-linear Mamba-2 fwd at T=16K (% MFMA peak); decode GB/s",
        "value": round(cfg.B * cfg.T / (fwd_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(fwd_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "fwd_bf16_T16K", "B": cfg.B, "H": cfg.H, "T": cfg.T, "dk": cfg.dk, "dv": cfg.dv,
            "chunk": cfg.chunk, "levels": cfg.L, "group_log2": args.group_log2,
            "inputs": "q,k,v bf16; a,lambda fp32; out bf16",
        },
        "roofline": roofline,
        "timing": fwd_stats,
        "forward": {
            "kernels_ms": {k: round(v[1] / v[0], 5) for k, v in kstats.items()},
            "algorithmic_bytes": fbytes, "algorithmic_flops": fflops,
            "hbm_frac_whole_call": round(whole_gbs / HBM_PEAK_GBS, 4),
            "mfma_frac_whole_call": round(mfma_tflops / BF16_PEAK_TFLOPS, 4),
        },
        "decode": {
            "workload": "decode_bf16_S64", "metric": "decode GB/s", "value": round(dec_gbs, 1), "unit": "GB/s",
            "ms_per_step": round(dec_ms, 5), "timing": dec_stats,
            "tokens_per_s": round(dcfg.S / (dec_ms * 1e-3), 1),
            "algorithmic_bytes": dbytes,
            "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                         "traffic": read_traffic(DECODE_TRAFFIC_FILE, DECODE_SOURCES),
                         "kernel": "ll_decode", "kernel_avg_ms": round(dec_kernel_ms, 5)},
        },
        "prefill": {
            "workload": "fwd_bf16_T16K + stack (Lcap 17)", "ms_per_step": round(pre_ms, 5), "timing": pre_stats,
            "tokens_per_s": round(cfg.B * cfg.T / (pre_ms * 1e-3), 1),
            "stack_algorithmic_bytes": sbytes,
            "roofline": {"bound": "hbm", "achieved": round(stack_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(stack_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                         "kernel": "ll_prefill_stack", "kernel_avg_ms": round(stack_ms, 5)},
        },
        "other_workloads": others,
        "grouped_qk": grouped,
        "gated_deltanet": gdn_res,
        "backward": backward,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host ...")
        result["cpu_baseline"] = cpu_baseline(host_sets[0], cfg, args.cpu_rows, seed=123)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
