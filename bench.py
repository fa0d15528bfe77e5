"""Benchmark of the SparsePR attention call on one MI355X.

One step = one whole SparsePR call in the fused order (partition, route, probe_fit,
attend_apply), which covers every stage the summary page of "Partition the Support,
Reconstruct the Residual" counts in its timed latency (partition, route, permutation,
sparse kernel, probes, fit, write-back); --unfused times partition, route, attend,
probe_fit, apply.  Workload: the HunyuanVideo-shaped 720p call, N = 118,800 tokens
(T=33, H=45, W=80), 24 heads, d = 128, bf16, target rho_exec = 22 %, seeded synthetic
inputs resident in HBM before the timed region.

Prints one JSON line: calls/s (value), the sparse kernel's effective TFLOP/s on executed
(unpadded) pairs and its fraction of the bf16 MFMA peak (roofline), the speedup over
the same-GPU dense attention, a per-stage breakdown, and the CPU oracle timed on a
bounded sample (cpu_baseline).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3] [--no-dense] [--no-cpu] [--unfused]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse attention calls/sec + effective TFLOPS (% bf16 MFMA peak) vs dense attn"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3
STAGES_FUSED = ["partition", "route", "probe_fit", "attend_apply"]
STAGES_UNFUSED = ["partition", "route", "attend", "probe_fit", "apply"]
STAGES_OVERLAPPED = ["partition", "gather_kv (second stream)", "route", "probe_fit (second stream)", "attend", "apply"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(cfg):
    """The oracle as it stands on one KV head of the workload, scaled to the call."""
    import numpy as np
    from oracle import sparsepr as O
    from sparsepr_workloads import generator as gen
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info] or [os.cpu_count() or 1])
        blas = ",".join(sorted({i.get("internal_api", "?") for i in info}))
    except Exception:  # pragma: no cover
        cores, blas = os.cpu_count() or 1, "?"
    q, k, v = gen.head_inputs(cfg, 0)
    p = O.Params(cfg.groups_q, cfg.groups_k, float(np.float32(cfg.rho_exec)), lam=float(np.float32(cfg.lam)))
    t0 = time.perf_counter()
    O.sparsepr_kv_head(q, k, v, p)
    dt = time.perf_counter() - t0
    per_call = dt * cfg.heads_kv
    return {"value": 1.0 / per_call, "unit": "calls/s", "cores": int(cores), "kind": "oracle",
            "sample": f"KV head 0 of {cfg.heads_kv} ({cfg.g} query head(s)): whole oracle call "
                      f"(partition, route, sparse attention of all {cfg.n} rows, probes, fit, apply) "
                      f"in {dt:.1f} s, scaled x{cfg.heads_kv}; float64 NumPy, BLAS {blas}, "
                      f"nproc {os.cpu_count()}"}


def dense_oracle_baseline(cfg, rows=1024):
    """The oracle's dense attention (float64, 1024-row chunks) on a bounded sample of query
    head 0 -- `rows` evenly spaced rows against all n keys -- scaled to every row of every
    query head of the call."""
    import numpy as np
    from oracle import sparsepr as O
    from sparsepr_workloads import generator as gen
    q, k, v = gen.head_inputs(cfg, 0)
    rows = min(rows, cfg.n)
    sel = (np.arange(rows) * cfg.n) // rows
    t0 = time.perf_counter()
    O.dense_attention(q[0], k, v, 1.0 / np.sqrt(cfg.d), rows=sel)
    dt = time.perf_counter() - t0
    per_call = dt * (cfg.n / rows) * cfg.heads_q
    return {"value": 1.0 / per_call, "unit": "calls/s", "kind": "oracle dense attention",
            "sample": f"{rows} evenly spaced rows of query head 0 against all {cfg.n} keys in {dt:.2f} s, "
                      f"scaled x{cfg.n / rows:.1f} rows x{cfg.heads_q} heads"}


def executed_tile_pairs(sp, cfg):
    """Query-key pairs the sparse kernel executes once its work is padded to tiles: per query
    group, the virtual rows (tokens x query heads of the KV head) rounded up to the 32 rows of
    one wave (waves past a group's rows skip the tile math), times the keys of the 64-key tiles
    its kept runs occupy (runs of adjacent kept key groups, each starting on a 16-key
    boundary), summed over KV heads."""
    import numpy as np
    rp = sp.route_buf["row_ptr"].cpu().numpy().astype(np.int64)
    cols = sp.route_buf["cols"].cpu().numpy().astype(np.int64)
    ko = sp.part["key_offsets"].cpu().numpy().astype(np.int64)
    qo = sp.part["query_offsets"].cpu().numpy().astype(np.int64)
    total = 0
    for kv in range(cfg.heads_kv):
        for a in range(cfg.groups_q):
            rows = (qo[kv, a + 1] - qo[kv, a]) * cfg.g
            if rows == 0:
                continue
            c = cols[kv, rp[kv, a]:rp[kv, a + 1]]
            keys, i = 0, 0
            while i < len(c):
                b = e = c[i]
                i += 1
                while i < len(c) and c[i] == e + 1:
                    e, i = c[i], i + 1
                k0, k1 = ko[kv, b], ko[kv, e + 1]
                if k1 > k0:
                    keys += (k1 - (k0 & ~15) + 63) // 64 * 64
            total += (rows + 31) // 32 * 32 * keys
    return int(total)


TRAFFIC_PROFILES = {   # call order -> counter summary of that order's attention kernel
    "fused": os.path.join(ROOT, "profiles", "sparse_attention_fused_720p_n118800_h24_hbm_traffic.md"),
    "overlapped": os.path.join(ROOT, "profiles", "sparse_attention_overlapped_720p_n118800_h24_hbm_traffic.md"),
}
KERNEL_SOURCES = ["free_block_sparse_sparsepr_amd/csrc/attend_mfma.hip", "free_block_sparse_sparsepr_amd/csrc/sp_attn.hpp",
                  "free_block_sparse_sparsepr_amd/csrc/sp_common.hpp"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload_name, order):
    """HBM bytes per launch of the attention kernel from the committed counter summary of
    this call order (FETCH_SIZE + WRITE_SIZE, each scaled against a plain copy of known
    size), or None when the summary is missing, covers another workload or order, or the
    kernel sources have changed since."""
    if order not in TRAFFIC_PROFILES:
        return None
    try:
        text = open(TRAFFIC_PROFILES[order]).read()
        block = text.split("```json", 1)[1].split("```", 1)[0]
        rec = json.loads(block)
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("workload") != workload_name or rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    if rec.get("call_order", "fused") != order:
        return None
    return rec.get("hbm_bytes_per_launch")


ABLATIONS = {   # summary page of "Partition the Support, Reconstruct the Residual", ablation paragraph
    "sparsepr": dict(),
    "hard_drop": dict(ablation=1),
    "semantic_hard_drop": dict(partition_mode=1, ablation=1),
    "semantic": dict(partition_mode=1),
    "ridge_only": dict(ablation=2),
    "uniform_probes": dict(probe_mode=1),
    "random_probes": dict(probe_mode=2),
    # budget variants (execution paragraph: the router spends a pair budget over cells)
    "tile_padded_costs": dict(cost_mode=1),
    "global_budget": dict(budget_mode=1),
    "global_budget_tile_padded": dict(budget_mode=1, cost_mode=1),
}


def ablation_report(workload):
    """Mean and 99th-percentile absolute error of the whole call's output against the
    same-GPU dense attention, for the method and each ablation switch, on one workload.
    The p99 is taken over a fixed stride of 2^24 elements; random probes are drawn with
    NumPy (seed 0) and passed in."""
    import numpy as np
    import torch

    import free_block_sparse_sparsepr_amd as S
    from sparsepr_workloads import CONFIGS, make_inputs

    cfg = CONFIGS[workload]
    dev = torch.device("cuda:0")
    Q, K, V = make_inputs(cfg, threads=16)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x).to(dev).to(tdt).contiguous() for x in (Q, K, V))
    del Q, K, V
    sp = S.SparsePR(S.config_from_workload(cfg), device=dev)
    dense = sp.dense(q, k, v).float()
    del sp
    rng = np.random.default_rng(0)
    given = np.stack([np.sort(rng.choice(cfg.n, cfg.n_probe, replace=False)) for _ in range(cfg.heads_kv)])
    stride = max(1, dense.numel() // (1 << 24))
    out = {}
    for name, kw in ABLATIONS.items():
        log(f"[ablations] {name}")
        sp = S.SparsePR(S.config_from_workload(cfg, **kw), device=dev)
        sp.partition(q, k, v)
        sp.route()
        if kw.get("probe_mode") == 2:
            sp.fit["probe_tokens"].copy_(torch.from_numpy(given.astype(np.int32)))
        sp.probe_fit(q)            # untimed first pass: the first launches load their kernels
        sp.attend_apply()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        sp.probe_fit(q)
        o = sp.attend_apply()
        torch.cuda.synchronize()
        err = (o.float() - dense).abs_().flatten()
        p99 = float(torch.quantile(err[::stride][: 1 << 24], 0.99))
        pairs = sp.route_buf["pairs"].cpu().numpy().astype(np.int64)
        out[name] = {"mean_abs_err": float(err.mean()), "p99_abs_err": p99,
                     "realised_rho_exec": float(pairs.mean()) / cfg.n ** 2 + cfg.n_probe / cfg.n,
                     "rho_exec_min_max_over_heads": [float(pairs.min()) / cfg.n ** 2 + cfg.n_probe / cfg.n,
                                                     float(pairs.max()) / cfg.n ** 2 + cfg.n_probe / cfg.n],
                     "probe_fit_plus_attend_ms": (time.perf_counter() - t0) * 1e3}
        del sp, o, err
        torch.cuda.empty_cache()
    print(json.dumps({"ablation_report": cfg.name, "reference": "same-GPU dense attention",
                      "data": "synthetic (seeded Fourier-feature Q/K, Gaussian V; no model weights)",
                      "variants": out}), flush=True)


def diagnostics_report(workload):
    """Per-head statistics of the hard-drop residual R = O_dense - O_sparse over every row, for
    the response-coupled and the semantic partition on one workload: the fraction of R's
    centred energy that is an affine function of the sparse output, and the energy left
    orthogonal to it (summary page of "Partition the Support, Reconstruct the Residual",
    partition paragraph)."""
    import numpy as np
    import torch

    import free_block_sparse_sparsepr_amd as S
    from sparsepr_workloads import CONFIGS, make_inputs

    cfg = CONFIGS[workload]
    dev = torch.device("cuda:0")
    Q, K, V = make_inputs(cfg, threads=16)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x).to(dev).to(tdt).contiguous() for x in (Q, K, V))
    del Q, K, V
    out = {}
    for name, mode in (("response", 0), ("semantic", 1)):
        log(f"[diagnostics] {name} partition")
        sp = S.SparsePR(S.config_from_workload(cfg, partition_mode=mode), device=dev)
        sp.partition(q, k, v)
        sp.route()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        st = sp.residual_diagnostics(q, k, v).cpu().numpy()
        ms = (time.perf_counter() - t0) * 1e3
        rows = cfg.n * cfg.d
        out[name] = {"explainable_frac_mean": float(st[:, 3].mean()),
                     "explainable_frac_min": float(st[:, 3].min()),
                     "explainable_frac_max": float(st[:, 3].max()),
                     "residual_energy_per_elem": float(st[:, 0].sum() / (rows * cfg.heads_q)),
                     "orthogonal_energy_per_elem": float(st[:, 2].sum() / (rows * cfg.heads_q)),
                     "per_head_frac": [round(float(x), 4) for x in st[:, 3]],
                     "call_ms": ms}
        del sp
        torch.cuda.empty_cache()
    print(json.dumps({"diagnostics_report": cfg.name,
                      "data": "synthetic (seeded Fourier-feature Q/K, Gaussian V; no model weights)",
                      "partitions": out}), flush=True)


def support_report(workload, n_sets=64, set_size=8):
    """Single-row and shared-route 90 %-mass supports on one workload (summary page of
    "Partition the Support, Reconstruct the Residual", support paragraph): per query head,
    n_sets sets of set_size queries, either consecutive raster tokens at seeded random
    starts or seeded random members of one query group of the response partition (group
    drawn in proportion to its size).  Reports medians as fractions of N."""
    import numpy as np
    import torch

    import free_block_sparse_sparsepr_amd as S
    from sparsepr_workloads import CONFIGS, make_inputs

    cfg = CONFIGS[workload]
    dev = torch.device("cuda:0")
    Q, K, V = make_inputs(cfg, threads=16)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x).to(dev).to(tdt).contiguous() for x in (Q, K, V))
    del Q, K, V
    sp = S.SparsePR(S.config_from_workload(cfg), device=dev)
    sp.partition(q, k, v)
    labels = sp.part["query_labels"].cpu().numpy()
    rng = np.random.default_rng(11)
    starts = rng.integers(0, cfg.n - set_size + 1, (cfg.heads_q, n_sets))
    kinds = {"consecutive_tokens": starts[..., None] + np.arange(set_size)}
    grp = np.empty((cfg.heads_q, n_sets, set_size), np.int64)
    for h in range(cfg.heads_q):
        lab = labels[h // cfg.g]
        for si in range(n_sets):
            members = np.flatnonzero(lab == lab[rng.integers(0, cfg.n)])
            grp[h, si] = rng.choice(members, set_size, replace=members.size < set_size)
    kinds["one_query_group"] = grp
    out = {}
    for name, sets in kinds.items():
        log(f"[support] {name}")
        st = torch.from_numpy(sets.astype(np.int32)).to(dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        rows, union = sp.support_diagnostics(q, k, st, 0.9)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3
        rows, union = rows.cpu().numpy() / cfg.n, union.cpu().numpy() / cfg.n
        out[name] = {"single_row_median": float(np.median(rows)), "shared_median": float(np.median(union)),
                     "single_row_median_per_head": [round(float(x), 4) for x in np.median(rows, axis=(1, 2))],
                     "shared_median_per_head": [round(float(x), 4) for x in np.median(union, axis=1)],
                     "call_ms": ms}
    print(json.dumps({"support_report": cfg.name, "mass": 0.9, "sets_per_head": n_sets, "set_size": set_size,
                      "data": "synthetic (seeded Fourier-feature Q/K, Gaussian V; no model weights)",
                      "sets": out}), flush=True)


def copy_probe(mib):
    """A plain copy of `mib` MiB (torch's device copy kernel), three launches on a source larger
    than the caches: each launch reads and writes exactly mib MiB."""
    import torch
    n = mib * (1 << 20)
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--dense-steps", type=int, default=None,
                    help="timed dense-attention calls (default: --steps, after --warmup untimed ones)")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--unfused", action="store_true",
                    help="time the unfused order (attend -> probe_fit -> apply) instead of the fused one")
    ap.add_argument("--chunks", type=int, default=4,
                    help="KV-head chunks of the pipelined order")
    ap.add_argument("--split-kv", type=int, default=None,
                    help="split order: KV heads whose attention runs beside the probe stage "
                         "(default: SparsePR.split_point())")
    ap.add_argument("--order", choices=["fused", "unfused", "overlapped", "pipelined", "split"], default=None,
                    help="call order to time: fused (probe_fit -> attend_apply), unfused (attend -> probe_fit "
                         "-> apply), overlapped (probe_fit on a second stream beside attend, then apply) or "
                         "pipelined (the fused order over --chunks chunks of KV heads on three streams, each "
                         "chunk's partition, route and probe stage beside the previous chunk's attention)")
    ap.add_argument("--budget-mode", type=int, default=0, choices=[0, 1],
                    help="route budget: 0 per KV head (the method), 1 one budget shared by all KV heads")
    ap.add_argument("--cost-mode", type=int, default=0, choices=[0, 1],
                    help="cell cost: 0 query-key pairs (the method), 1 tile-padded pairs")
    ap.add_argument("--graph", action="store_true",
                    help="after the eager timed region, capture one call of the same order in a HIP graph and "
                         "time the same number of replays (reported under \"graph\")")
    ap.add_argument("--ablations", action="store_true",
                    help="instead of timing, print the output error against dense attention of the method and "
                         "each ablation switch (hard drop, semantic partition, unprojected ridge, uniform and "
                         "random probes) and budget variant (tile-padded costs, global budget) on the workload")
    ap.add_argument("--diagnostics", action="store_true",
                    help="instead of timing, print the affine-explainable fraction and orthogonal energy of "
                         "the hard-drop residual for the response-coupled and semantic partitions")
    ap.add_argument("--support", action="store_true",
                    help="instead of timing, print the median single-row and shared-route 90%%-mass supports "
                         "for sets of 8 consecutive tokens and of 8 members of one query group")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (3 launches) and exit: the reference "
                         "kernel of known traffic for scaling the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    if args.ablations:
        ablation_report(args.workload)
        return
    if args.diagnostics:
        diagnostics_report(args.workload)
        return
    if args.support:
        support_report(args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for {args.gpus}); the SparsePR call "
              "shards by head with no exchange step, but no multi-GPU path is built.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import free_block_sparse_sparsepr_amd as S
    from sparsepr_workloads import CONFIGS, make_inputs

    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    log(f"[bench] generating {cfg.name} inputs")
    t0 = time.perf_counter()
    Q, K, V = make_inputs(cfg, threads=16)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x).to(dev).to(tdt).contiguous() for x in (Q, K, V))
    del Q, K, V
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s")
    sp = S.SparsePR(S.config_from_workload(cfg, budget_mode=args.budget_mode, cost_mode=args.cost_mode), device=dev)
    out = torch.empty((cfg.heads_q, cfg.n, cfg.d), dtype=tdt, device=dev)
    stream = torch.cuda.current_stream()

    order = args.order or ("unfused" if args.unfused else "overlapped")
    side = sp.side_stream() if order == "overlapped" else None
    pipe = None
    if order == "pipelined":
        pipe = S.PipelinedSparsePR(S.config_from_workload(cfg, budget_mode=args.budget_mode,
                                                          cost_mode=args.cost_mode),
                                   chunks=args.chunks, device=dev, fused=True)
        stages = STAGES_FUSED
        nch = len(pipe.parts)
    if order == "pipelined":
        pass
    elif order == "split":
        stages = S.SparsePR.SPLIT_STAGES
    elif order == "unfused":
        stages = STAGES_UNFUSED
        fns = [lambda: sp.partition(q, k, v), sp.route, sp.attend, lambda: sp.probe_fit(q), lambda: sp.apply(out)]
        streams = [stream] * 5
    elif order == "overlapped":   # as SparsePR.overlapped, stage by stage
        stages = STAGES_OVERLAPPED
        kv_ready = torch.cuda.Event()
        fns = [lambda: sp.partition(q, k, v, defer_kv=True), lambda: sp.gather_kv(k, v), sp.route,
               lambda: sp.probe_fit(q), sp.attend, lambda: sp.apply(out)]
        streams = [stream, side, stream, side, stream, stream]
    else:
        stages = STAGES_FUSED
        fns = [lambda: sp.partition(q, k, v), sp.route, lambda: sp.probe_fit(q), lambda: sp.attend_apply(out)]
        streams = [stream] * 4
    attn_stage = "attend_apply" if order in ("fused", "pipelined") else "attend"

    def step(ev=None):
        if pipe is not None:
            pipe(q, k, v, out, events=None if ev is None else {name: ev[i] for i, name in enumerate(stages)})
            return
        if order == "split":
            sp.split(q, k, v, out, first_kv=args.split_kv,
                     events=None if ev is None else {name: ev[i] for i, name in enumerate(stages)})
            return
        for i, fn in enumerate(fns):
            st = streams[i]
            if st is not stream:
                st.wait_stream(stream)      # a side stage starts after the main stream's work so far
            if side is not None and stages[i] == "attend":
                stream.wait_event(kv_ready)  # attend reads the gathered K and V
            with torch.cuda.stream(st):
                if ev is not None:
                    ev[i][0].record(st)
                fn()
                if ev is not None:
                    ev[i][1].record(st)
                if side is not None and stages[i].startswith("gather_kv"):
                    kv_ready.record(st)
            if i == len(fns) - 2 and side is not None:
                stream.wait_stream(side)    # apply waits for the fit

    for i in range(args.warmup):
        step()
        log(f"[bench] warmup {i + 1}/{args.warmup}")
    torch.cuda.synchronize()
    per = nch if pipe is not None else 1
    events = [[[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(per)]
               if pipe is not None else [torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
               for _ in stages] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"[bench] timed {args.steps} calls in {wall:.3f} s")
    if pipe is not None:    # stage time summed over the chunks (each on its own stream)
        stage_ms = {name: float(np.mean([sum(e0.elapsed_time(e1) for e0, e1 in events[s][i])
                                          for s in range(args.steps)])) for i, name in enumerate(stages)}
    else:
        stage_ms = {name: float(np.mean([events[s][i][0].elapsed_time(events[s][i][1]) for s in range(args.steps)]))
                    for i, name in enumerate(stages)}
    ms_per_step = wall * 1e3 / args.steps
    if order == "split":   # the attention's two launches, each timed on its own stream
        stage_ms["attend"] = stage_ms[stages[4]] + stage_ms[stages[5]]

    graph = None
    if args.graph:
        g = (pipe or sp).capture(q, k, v, out, order)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        gwall = time.perf_counter() - t0
        graph = {"ms_per_call": gwall * 1e3 / args.steps, "calls_per_s": args.steps / gwall}
        log(f"[bench] graph replays: {graph['ms_per_call']:.2f} ms/call")
        del g

    if pipe is not None:
        pairs_kv = np.concatenate([p.route_buf["pairs"].cpu().numpy() for _, _, p in pipe.parts]).astype(np.int64)
    else:
        pairs_kv = sp.route_buf["pairs"].cpu().numpy().astype(np.int64)
    routed = int(pairs_kv.sum()) * cfg.g                     # summed over query heads
    executed = routed + cfg.heads_q * cfg.n_probe * cfg.n
    flop_attend = 4.0 * cfg.d * routed
    flop_call = 4.0 * cfg.d * executed
    attend_tflops = flop_attend / (stage_ms[attn_stage] * 1e-3) / 1e12
    call_tflops = flop_call / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS
    rho_route = float(pairs_kv.mean()) / cfg.n ** 2
    rho_exec = rho_route + cfg.n_probe / cfg.n

    padded = executed_tile_pairs(sp, cfg) if pipe is None else None

    dense = None
    if not args.no_dense:
        dsteps = args.dense_steps or args.steps
        for _ in range(max(1, args.warmup)):
            sp.dense(q, k, v, out)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(dsteps):
            sp.dense(q, k, v, out)
        torch.cuda.synchronize()
        dense_ms = (time.perf_counter() - t0) * 1e3 / dsteps
        dense_flop = 4.0 * cfg.d * cfg.n * cfg.n * cfg.heads_q
        dense = {"ms_per_call": dense_ms, "steps": dsteps, "tflops": dense_flop / (dense_ms * 1e-3) / 1e12,
                 "speedup_sparsepr_vs_dense": dense_ms / ms_per_step}
        log(f"[bench] dense {dense_ms:.2f} ms/call")

    cpu = None
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on one head")
        cpu = cpu_baseline(cfg)
        log("[bench] timing the CPU oracle's dense attention on a sample of rows")
        cpu["dense_attention"] = dense_oracle_baseline(cfg)

    res = {
        "metric": METRIC, "value": args.steps / wall, "unit": "calls/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded Fourier-feature Q/K, Gaussian V; no model weights)",
        "config": {"workload": cfg.name, "grid_thw": list(cfg.grid), "n": cfg.n, "heads_q": cfg.heads_q,
                   "heads_kv": cfg.heads_kv, "d": cfg.d, "rho_exec_target": cfg.rho_exec,
                   "groups_q": cfg.groups_q, "groups_k": cfg.groups_k, "n_probe": cfg.n_probe,
                   "rank": cfg.rank, "r_k": cfg.r_k, "r_q": cfg.r_q, "lambda": cfg.lam},
        "call_order": (order if order != "split" else
                       f"split at KV head {args.split_kv or sp.split_point()} of {cfg.heads_kv}")
                      if pipe is None else f"pipelined over {nch} chunks of KV heads (fused order per chunk)",
        "route_variant": {"budget_mode": ["per_kv_head", "global"][args.budget_mode],
                          "cost_mode": ["pairs", "tile_padded"][args.cost_mode]},
        "roofline": {"bound": "mfma", "kernel": "sparse attention (" + (
                     "sparsepr_attend" if order not in ("fused", "split") else
                     "sparsepr_attend_apply: attention with the fused write-back epilogue, plus the 64-row probe "
                     "write-back kernel" if order == "fused" else
                     "sparsepr_attend on the first KV heads plus sparsepr_attend_apply on the others, their "
                     "durations on their own streams summed") + ")",
                     "achieved": attend_tflops, "peak": peak, "unit": "TFLOP/s", "frac": attend_tflops / peak,
                     "traffic": measured_traffic(cfg.name, order)},
        "graph": graph,
        "effective_tflops_call": call_tflops, "effective_frac_call": call_tflops / peak,
        "realised_rho_route": rho_route, "realised_rho_exec": rho_exec,
        "routed_pairs": routed,
        "tile_padded_pairs": None if padded is None else padded,
        "routed_over_padded": None if not padded else routed / padded,
        "attend_tflops_on_padded_pairs": None if not padded else 4.0 * cfg.d * padded / (stage_ms[attn_stage] * 1e-3) / 1e12,
        "stage_ms": stage_ms, "dense": dense, "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
