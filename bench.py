#!/usr/bin/env python3
"""Decode throughput of the SeKV path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one decode token through every layer of the workload: per layer,
routing with the budget cap (sekv_route) then attention over anchors,
pseudo-tokens and the factored spans (sekv_decode_attend), launched layer by
layer as a model's decode loop would.  Inputs (cache, index, queries, thresholds) are resident in
HBM before the timed region.  Prints one JSON line on stdout.

value       = decode query-tokens/s = B * K / (timed wall time of K steps)
step_ms     = p10 / median / p90 of the K per-step durations, from a pass of
              the same steps with an event after each (the timed region
              holds the K steps alone)
roofline    = the attention kernel's algorithmic bytes per launch (resident
              K/V rows, the factor blobs of the routed union at their stored
              ranks, queries, masks) over its mean launch time, against
              MI355X's 8 TB/s HBM peak.  The launch time comes from HIP events
              recorded in each attention launch's own dispatch packet, in an
              instrumented pass over the same steps on the same stream (the
              timed region itself carries no events); `traffic` is the
              committed rocprofv3 FETCH_SIZE + WRITE_SIZE reading for the same
              kernel source, or null
cpu_baseline= the fp64 CPU oracle (BLAS on the process's cores; a one-thread
              run beside it), on a bounded sample of the
              same workload (one layer x one KV head), scaled to a full step
pcie        = the same decode with span factors in pinned host memory and the
              routed union gathered into an HBM ring slot (PCIe bytes and time
              per step; query-tokens/s including PCIe for per-layer calls and
              for one call over all layers; reported beside the value, never
              as it)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "decode query-tokens/s at 128K ctx; achieved HBM GB/s vs peak (1 MI355X)"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attend_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def span_alg_bytes(rk, rv, d, n):
    """Bytes of one span's factors with rk key and rv value components stored:
    U (n x r), V^T (r x d) in bf16 and sigma * m in fp32, per K and V."""
    return 2 * (rk + rv) * (n + d) + 4 * (rk + rv)


def kernel_source_hash():
    p = os.path.join(ROOT, "compressed_kv_cache_sekv_amd", "csrc", "attend.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def traffic_from_profile(bytes_per_launch_alg):
    """HBM traffic per attention launch from the committed rocprofv3 PMC
    summary, or None when absent or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def union_alg_bytes(masks, n_spans, span_len, G, ranks, d):
    """Algorithmic factor bytes of one attention launch: for every (b, g), the
    blobs of the union over the G heads' routed spans.  masks: uint64 [B, Hq,
    Wd]; ranks[b]: the layer's stored ranks, int [Hkv, N_S(b), 2] (K, V)."""
    B, Hq, Wd = masks.shape
    bits = np.unpackbits(masks.astype(">u8").view(np.uint8).reshape(B, Hq, Wd, 8), axis=3)[..., ::-1]
    bits = bits.reshape(B, Hq, Wd * 64).astype(bool)
    tot, nun = 0, 0
    off = 0
    for b in range(B):
        ns = int(n_spans[b])
        lens = span_len[off:off + ns].astype(np.int64)
        for g in range(Hq // G):
            blob = span_alg_bytes(ranks[b][g, :, 0].astype(np.int64), ranks[b][g, :, 1].astype(np.int64), d, lens)
            u = bits[b, g * G:(g + 1) * G, :ns].any(0)
            tot += int(blob[u].sum())
            nun += int(u.sum())
        off += ns
    return tot, nun


def cpu_baseline(w, H, K, V, W, gates, tau, cap, q_steps, budget_s=8.0):
    """Time the oracle on one (layer 0, KV head 0) unit of the workload: build
    that unit's index (untimed), then route + attend for the G query heads for
    as many decode steps as fit in ~budget_s, scaled to the L Hkv B units of a
    step.  Run with BLAS on the process's cores (the oracle as it stands; the
    reported baseline) and again on one thread (`one_thread`)."""
    from threadpoolctl import threadpool_limits
    from oracle import sekv_oracle as O
    G = w.G
    cores = len(os.sched_getaffinity(0))
    t0 = time.time()
    gb = None if gates is None else gates[0][0:1, 0:1].double().numpy()
    idx = O.build_index_b(H[0].numpy(), K[0][0:1, 0:1].double().numpy(),
                          V[0][0:1, 0:1].double().numpy(), W[0:1, 0:G].double().numpy(), gb,
                          R=w.R, alpha_sp=w.alpha_sp, l_min=w.l_min, Hq=G)
    log(f"[cpu] oracle index of one (layer, kv head) unit built in {time.time() - t0:.1f} s")
    Wn = W[0, 0:G].double().numpy()
    units = w.L * w.Hkv * w.B

    def run(threads):
        with threadpool_limits(threads):
            done, t0 = 0, time.time()
            while True:
                q = q_steps[done % len(q_steps)][0, 0, 0:G].double().numpy()   # [G, d]
                for h in range(G):
                    _, z = O.route_head(Wn[h], q[h], idx.s[0, h], float(tau[0, h]), cap)
                    O.decode_head(q[h], idx, 0, 0, z)
                done += 1
                el = time.time() - t0
                if el > budget_s or done >= 200:
                    break
        per_unit = el / done
        return done, per_unit, w.B / (per_unit * units)

    done, per_unit, value = run(cores)
    done1, per_unit1, value1 = run(1)
    return {"value": value, "unit": "query-tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"{done} decode steps of one (layer 0, KV head 0) unit (route + attend for its {G} "
                       f"query heads over the oracle-built index of that unit at T={w.T}), "
                       f"{per_unit * 1e3:.1f} ms per unit with BLAS on {cores} threads, scaled by {units} "
                       f"units per step"),
            "one_thread": {"value": value1, "cores": 1, "ms_per_unit": round(per_unit1 * 1e3, 2),
                           "steps": done1}}


def prefill(args) -> int:
    """Prefill leg: index build of the 128K single-layer workload, then the
    randomized SVD (sekv_rsvd_batched) of every span's K and V of that layer,
    timed with HIP events on the library's stream.  GEMM work per matrix
    (n x d, sketch width l = min(R + p, n, d)): A Omega, q power steps of two
    products each, and the final projection, 2 n d l flops apiece."""
    import torch
    from compressed_kv_cache_sekv_amd import synth
    from compressed_kv_cache_sekv_amd import lib as sl
    w = synth.WORKLOADS["prefill_8b_128k"]
    dev = "cuda"
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    H, K, V = synth.kv_cache(w, device=dev)
    W = torch.stack([synth.routing_w(w, l, dev) for l in range(w.L)])
    ctx = sl.Context(0, stream=stream)
    reps = 3
    build_ms = []
    for r in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        idx = ctx.build_index(sl.build_params(w), K, V, H, W, None)
        e1.record(stream)
        torch.cuda.synchronize()
        if r:
            build_ms.append(e0.elapsed_time(e1))
        start, length, _ = idx.spans()
        idx.free()
    # every span's K and V rows of the layer, for each KV head, as one batch
    st = torch.from_numpy(start.astype(np.int64)).to(dev)
    ln = torch.from_numpy(length.astype(np.int64)).to(dev)
    tok = torch.repeat_interleave(st, ln) + (torch.arange(int(ln.sum()), device=dev)
                                             - torch.repeat_interleave(torch.cumsum(ln, 0) - ln, ln))
    mats = [X[0, 0, g].index_select(0, tok) for g in range(w.Hkv) for X in (K, V)]
    A = torch.cat(mats).contiguous()
    nspan = len(length)
    rows = torch.from_numpy(np.tile(length.astype(np.int32), 2 * w.Hkv)).to(dev)
    row_off = (torch.cumsum(rows.long(), 0) - rows.long()) * w.d
    cnt, mr = int(rows.numel()), int(length.max())
    U = torch.empty(cnt, mr, w.R, device=dev)
    S = torch.empty(cnt, w.R, device=dev)
    Vt = torch.empty(cnt, w.R, w.d, device=dev)
    rsvd_ms = []
    for r in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        ctx.rsvd_batched(A, row_off, rows, mr, w.d, w.R, w.oversample, w.power_iters, w.seed, U, S, Vt)
        e1.record(stream)
        torch.cuda.synchronize()
        if r:
            rsvd_ms.append(e0.elapsed_time(e1))
    n = np.tile(length.astype(np.int64), 2 * w.Hkv)
    lw = np.minimum(np.minimum(w.R + w.oversample, n), w.d)
    flops = float(np.sum(2 * n * w.d * lw * (2 + 2 * w.power_iters)))
    t = float(np.median(rsvd_ms))
    tflops = flops / (t * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle's exact truncated SVD (LAPACK, fp64) of the first span
        # matrices of the same batch, one thread, ~10 s, scaled to all of them
        from threadpoolctl import threadpool_limits
        from oracle import sekv_oracle as O
        Ah = A.cpu()
        offs = row_off.cpu().numpy() // w.d
        done, t0 = 0, time.time()
        with threadpool_limits(1):
            while done < cnt and time.time() - t0 < 10.0:
                O.truncated_svd(Ah[offs[done]:offs[done] + int(n[done])].double().numpy(), w.R)
                done += 1
        el = time.time() - t0
        cpu = {"value": round(el / done * cnt * 1e3, 1), "unit": "ms", "cores": 1, "kind": "oracle",
               "sample": f"exact truncated SVD (numpy LAPACK, fp64) of the first {done} of the {cnt} span "
                         f"matrices in {el:.1f} s, scaled to all {cnt}"}
        log(f"[cpu] oracle SVD of {done} matrices in {el:.1f} s: {cpu['value']:.0f} ms for the layer")
    print(json.dumps({
        "metric": "prefill: randomized SVD of every span K/V of one 128K layer (R=32, oversampling 8, "
                  "2 power iterations)",
        "value": round(t, 3), "unit": "ms", "higher_is_better": False, "dtype": "bf16 MFMA / fp32, fp64",
        "data": "synthetic", "matrices": cnt, "spans": nspan,
        "build_index_ms": round(float(np.median(build_ms)), 3),
        "gemm_gflop": round(flops / 1e9, 2),
        "mfma": {"achieved": round(tflops, 3), "peak": 2500.0, "unit": "TFLOP/s",
                 "frac": round(tflops / 2500.0, 5)},
        "cpu_baseline": cpu,
        "config": {"workload": w.name, "kv_heads": w.Hkv, "head_dim": w.d, "context": w.T, "R": w.R}}),
        flush=True)
    ctx.close()
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_l32_128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-pinned", action="store_true")
    ap.add_argument("--graph", action="store_true", help="time a HIP graph replay of the step instead of eager launches")
    ap.add_argument("--pooled", action="store_true",
                    help="replace the per-(layer, head) cap with one budget per layer pooled over its heads "
                         "(sekv_route_pooled, budget = cap x query heads); workloads with a cap only")
    ap.add_argument("--prefill", action="store_true",
                    help="time the prefill side instead: the index build of one 128K layer (R = 32) and the "
                         "randomized SVD of all its span matrices alone; prints one JSON line")
    ap.add_argument("--gate-eps", type=float, default=0.0,
                    help="build with this gate_eps: components whose gate is below it are not stored "
                         "(variable effective rank; 0 keeps every component)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 4 plain device copies of MIB MiB each (a known-size kernel that scales "
                         "rocprofv3's FETCH_SIZE / WRITE_SIZE readings) and exit")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the SeKV decode path here has no multi-GPU mode "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        return 2

    import torch
    from compressed_kv_cache_sekv_amd import synth
    from compressed_kv_cache_sekv_amd import lib as sl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_probe:
        n = args.copy_probe << 18   # fp32 elements
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_each_way": n * 4, "launches": 4}), flush=True)
        return 0
    if args.prefill:
        return prefill(args)
    w = synth.WORKLOADS[args.workload]
    dev = "cuda"
    torch.cuda.set_device(0)
    # one default-priority stream for everything: the library context, the
    # timed region and the graph capture
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    t0 = time.time()
    H, K, V = synth.kv_cache(w, device=dev)
    W = torch.stack([synth.routing_w(w, l, dev) for l in range(w.L)])
    S_max = synth.max_spans(w.T, w.l_min)
    gl = [[synth.gates(w, b, l, S_max, dev) for l in range(w.L)] for b in range(w.B)]
    gates = None if gl[0][0] is None else torch.stack([torch.stack(x) for x in gl])
    torch.cuda.synchronize()
    log(f"[bench] inputs for {w.name} generated on the GPU in {time.time() - t0:.1f} s")

    ctx = sl.Context(0, stream=stream)
    t0 = time.time()
    idx = ctx.build_index(sl.build_params(w, tier=sl.TIER_HBM, gate_eps=args.gate_eps), K, V, H, W, gates)
    build_s = time.time() - t0
    info = idx.info
    log(f"[bench] index built in {build_s:.2f} s: spans {list(idx.n_spans)[:4]} raw {list(idx.n_raw)[:4]} "
        f"resident {info.resident_bytes / 1e9:.2f} GB factors {info.factor_bytes / 1e9:.2f} GB")
    _, span_len, _ = idx.spans()
    # stored ranks per (b, l): [Hkv, N_S(b), 2]
    rk_all = idx.export(fields=["rank"])["rank"]
    ranks, o = [], 0
    for b in range(w.B):
        n = w.L * w.Hkv * int(idx.n_spans[b]) * 2
        ranks.append(rk_all[o:o + n].reshape(w.L, w.Hkv, int(idx.n_spans[b]), 2))
        o += n
    mean_rank = float(rk_all.mean()) if rk_all.size else 0.0

    tau = torch.empty(w.L, w.Hq, device=dev)
    if w.tau is not None:
        tau.fill_(w.tau)
    else:
        idx.calibrate_tau(0, w.L, synth.calibration_query(w, dev), w.frac, tau)
    cap = int(math.floor(w.cap_frac * int(idx.n_spans.min()))) if w.cap_frac else 0
    L, B, Hq, d, Wd = w.L, w.B, w.Hq, w.d, idx.mask_words
    nsteps = args.warmup + args.steps
    qs = [[synth.query(w, s, dev, layers=[l]).contiguous() for l in range(L)] for s in range(nsteps)]
    taus = [tau[l:l + 1].contiguous() for l in range(L)]
    masks = torch.zeros(nsteps, L, B, 1, Hq, Wd, dtype=torch.int64, device=dev)
    outs = [torch.zeros(B, 1, Hq, d, device=dev) for _ in range(L)]

    if args.pooled and cap <= 0:
        log("[bench] --pooled needs a workload with a cap")
        return 2
    budget = cap * Hq if args.pooled else 0

    def step(s, ix=idx):
        for l in range(L):
            if args.pooled:
                ix.route_pooled(l, 1, qs[s][l], taus[l], budget, masks[s, l], None)
            else:
                ix.route(l, 1, qs[s][l], taus[l], cap, masks[s, l], None)
            ix.decode_attend(l, 1, qs[s][l], masks[s, l], outs[l])

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()

    # per-step distribution: the same steps with one event after each (a pass
    # of its own, so that neither the timed region nor the kernel timing
    # carries the events)
    marks = [torch.cuda.Event(enable_timing=True)]
    marks[0].record()
    for s in range(args.warmup, nsteps):
        step(s)
        marks.append(torch.cuda.Event(enable_timing=True))
        marks[-1].record()
    torch.cuda.synchronize()
    dur = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(len(marks) - 1)])
    step_ms = {"p10": round(float(np.percentile(dur, 10)), 4), "median": round(float(np.median(dur)), 4),
               "p90": round(float(np.percentile(dur, 90)), 4)}

    # kernel durations: an instrumented eager pass over the timed steps
    ctx.timing(True)
    ctx.timing_read()
    for s in range(args.warmup, nsteps):
        step(s)
    torch.cuda.synchronize()
    route_ms, route_n, attend_ms, attend_n = ctx.timing_read()
    ctx.timing(False)
    assert attend_n == args.steps * L and route_n == args.steps * L

    # whole-step throughput: the step (copy of the step's queries into the
    # captured buffers, then route + attend for every layer) replayed as one
    # HIP graph, or launched eagerly with --eager
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    if not args.graph:
        torch.cuda.synchronize()
        e0.record()
        for s in range(args.warmup, nsteps):
            step(s)
        e1.record()
        torch.cuda.synchronize()
    else:
        # the captured step reads its queries from fixed buffers; each timed
        # step first copies its own queries there (part of the timed work)
        qbuf = [torch.empty_like(qs[0][l]) for l in range(L)]
        mbuf = torch.zeros_like(masks[0])
        for l in range(L):
            qbuf[l].copy_(qs[args.warmup][l])

        def gstep():
            for l in range(L):
                if args.pooled:
                    idx.route_pooled(l, 1, qbuf[l], taus[l], budget, mbuf[l], None)
                else:
                    idx.route(l, 1, qbuf[l], taus[l], cap, mbuf[l], None)
                idx.decode_attend(l, 1, qbuf[l], mbuf[l], outs[l])
        gstep()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            gstep()
        graph.replay()
        torch.cuda.synchronize()
        e0.record()
        for s in range(args.warmup, nsteps):
            for l in range(L):
                qbuf[l].copy_(qs[s][l])
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
    elapsed_ms = e0.elapsed_time(e1)
    value = B * args.steps / (elapsed_ms / 1e3)
    log(f"[bench] {args.steps} steps in {elapsed_ms:.2f} ms ({'graph' if args.graph else 'eager'}): "
        f"{value:.1f} query-tokens/s; attend {attend_ms / attend_n * 1e3:.1f} us/launch, "
        f"route call {route_ms / route_n * 1e3:.1f} us")

    # algorithmic bytes of the timed launches
    mk = masks[args.warmup:].cpu().numpy().view(np.uint64)     # [K, L, B, 1, Hq, Wd]
    res_rows = int((idx.n_spans + idx.n_raw).sum())
    res_bytes = w.Hkv * res_rows * d * 2 * 2
    small = B * Hq * d * 2 + B * Hq * Wd * 8
    fac_bytes, unions = 0, 0
    for s in range(args.steps):
        for l in range(L):
            fb, nu = union_alg_bytes(mk[s, l][:, 0], idx.n_spans, span_len, w.G, [r[l] for r in ranks], d)
            fac_bytes += fb
            unions += nu
    launches = args.steps * L
    attend_bytes = launches * (res_bytes + small) + fac_bytes
    per_launch = attend_bytes / launches
    achieved = attend_bytes / (attend_ms / 1e3) / 1e9
    route_bytes = launches * (Hq * w.dprime * int(idx.n_spans.sum()) * 4 + Hq * w.dprime * d * 4)
    route_gbs = route_bytes / (route_ms / 1e3) / 1e9
    traffic = traffic_from_profile(per_launch)
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "query-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(elapsed_ms / args.steps, 4),
        "step_ms": step_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": L, "query_heads": Hq, "kv_heads": w.Hkv, "head_dim": d,
                   "batch": B, "context": w.T, "R": w.R, "dprime": w.dprime, "gate_eps": args.gate_eps,
                   "mean_stored_rank": round(mean_rank, 2),
                   "expand_frac_target": w.frac if w.tau is None else None, "tau": w.tau,
                   "cap": 0 if args.pooled else cap, "pooled_budget_per_layer": budget or None,
                   "factor_tier": "hbm",
                   "launch": "per layer: " + ("route_pooled" if args.pooled else "route") + " + decode_attend"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "attend_kernel", "alg_bytes_per_launch": int(per_launch),
                     "mean_launch_us": round(attend_ms / attend_n * 1e3, 2)},
        "route_call": {"achieved": round(route_gbs, 1), "unit": "GB/s",
                       "mean_call_us": round(route_ms / route_n * 1e3, 2),
                       "covers": ("the sekv_route call by events around it: route kernel, then the cap kernel "
                                  "when cap > 0 (or the pool kernel), with the dispatch between them"),
                       "bytes": "the summary keys and W"},
        "index": {"build_s": round(build_s, 3), "spans": [int(x) for x in idx.n_spans[:4]],
                  "raw": [int(x) for x in idx.n_raw[:4]], "union_spans_per_launch": round(unions / launches, 1),
                  "resident_gb": round(info.resident_bytes / 1e9, 3),
                  "factor_gb": round(info.factor_bytes / 1e9, 3)},
    }

    if not args.no_pinned and w.tier == "pinned":
        # same decode with the factor pool in pinned host memory
        del idx
        torch.cuda.synchronize()
        t0 = time.time()
        pidx = ctx.build_index(sl.build_params(w, tier=sl.TIER_PINNED_HOST, gate_eps=args.gate_eps), K, V, H, W,
                               gates)
        pbuild_s = time.time() - t0
        log(f"[bench] pinned-tier index built in {pbuild_s:.2f} s")
        psteps = min(4, args.steps)
        ss = range(args.warmup, args.warmup + psteps)

        def wall_of(fn):
            torch.cuda.synchronize()
            t0 = time.time()
            for s in ss:
                fn(s)
            torch.cuda.synchronize()
            return time.time() - t0

        # (1) the model's loop: per layer, route then decode, no statistics
        # (no host synchronisation): each layer's gather, then its attention
        def per_layer(s):
            for l in range(L):
                pidx.route(l, 1, qs[s][l], taus[l], cap, masks[s, l], None)
                pidx.decode_attend(l, 1, qs[s][l], masks[s, l], outs[l])

        # (2) one call over all layers (queries of every layer at hand): the
        # gathers run one layer ahead of the attention on the index's copy
        # stream, two ring slots
        qall = {s: torch.cat(qs[s], dim=1).contiguous() for s in ss}
        mall = torch.zeros(B, L, Hq, Wd, dtype=torch.int64, device=dev)
        oall = torch.zeros(B, L, Hq, d, device=dev)

        def all_layers(s):
            pidx.route(0, L, qall[s], tau, cap, mall, None)
            pidx.decode_attend(0, L, qall[s], mall, oall)

        per_layer(args.warmup)
        all_layers(args.warmup)
        wall1 = wall_of(per_layer)
        wall2 = wall_of(all_layers)
        # statistics pass (reads back union sizes and gather times; syncs)
        pb = pc = 0
        pms = pms2 = 0.0
        ctx.timing(True)
        ctx.timing_read()
        for s in ss:
            for l in range(L):
                pidx.route(l, 1, qs[s][l], taus[l], cap, masks[s, l], None)
                st = pidx.decode_attend(l, 1, qs[s][l], masks[s, l], outs[l], stats=True)
                pb += st.pcie_bytes
                pc += st.pcie_copies
                pms += st.pcie_ms
        torch.cuda.synchronize()
        p_route_ms, p_route_n, p_attend_ms, p_attend_n = ctx.timing_read()
        ctx.timing(False)
        for s in ss:
            pidx.route(0, L, qall[s], tau, cap, mall, None)
            pms2 += pidx.decode_attend(0, L, qall[s], mall, oall, stats=True).pcie_ms
        torch.cuda.synchronize()
        result["pcie"] = {"build_s": round(pbuild_s, 3), "steps": psteps, "bytes_per_step": int(pb / psteps),
                          "copies_per_step": int(pc / psteps), "copy_ms_per_step": round(pms / psteps, 3),
                          "attend_us_per_launch_ring": round(p_attend_ms / max(p_attend_n, 1) * 1e3, 2),
                          "route_us_per_launch": round(p_route_ms / max(p_route_n, 1) * 1e3, 2),
                          "GB_per_s": round(pb / (pms / 1e3) / 1e9, 2) if pms > 0 else None,
                          "query_tokens_per_s_incl_pcie": round(B * psteps / wall1, 3),
                          "ms_per_step_incl_pcie": round(wall1 / psteps * 1e3, 3),
                          "all_layers_call": {
                              "query_tokens_per_s_incl_pcie": round(B * psteps / wall2, 3),
                              "ms_per_step_incl_pcie": round(wall2 / psteps * 1e3, 3),
                              "copy_ms_per_step": round(pms2 / psteps, 3),
                              "note": "one route and one decode call over all layers per step; gathers "
                                      "one layer ahead on a second stream"}}
        log(f"[bench] pinned tier: {pb / psteps / 1e9:.3f} GB and {pc / psteps:.0f} copies per step, "
            f"{pms / psteps:.1f} ms of copies per step; {B * psteps / wall1:.2f} query-tokens/s with PCIe "
            f"(per-layer calls), {B * psteps / wall2:.2f} (one call over all layers, gathers overlapped)")
        del pidx

    if not args.no_cpu_baseline:
        t0 = time.time()
        Hc = H.cpu()
        Kc = K[:, 0:1, 0:1].cpu()
        Vc = V[:, 0:1, 0:1].cpu()
        Wc = W.cpu()
        gc = None if gates is None else gates[:, 0:1, 0:1].cpu()
        qc = [qs[s][0].cpu() for s in range(args.warmup, nsteps)]
        result["cpu_baseline"] = cpu_baseline(w, Hc, Kc, Vc, Wc, gc, tau.cpu().numpy(), cap, qc)
        log(f"[bench] cpu baseline in {time.time() - t0:.1f} s: {result['cpu_baseline']['value']:.4f} query-tokens/s")

    print(json.dumps(result), flush=True)
    ctx.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
