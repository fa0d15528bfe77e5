"""CPU study of the probe fit's conditioning (not collected as a test; run as a script).

    python tests/fit_conditioning_study.py [--workloads 2 4 5] [--heads 2]

For each KV head of a workload the oracle runs the partition, route and probe selection,
then the output error against dense attention (mean and 99th-percentile absolute error over
every row) is measured for hard drop and for the probe-fit correction under each reading of
the two points the probe-fit paragraph of the summary page of "Partition the Support,
Reconstruct the Residual" leaves open: the scale of the group-coverage weights (mean one, or
the tokens each probe stands for) and whether lambda = 0.1 is absolute or relative to the
weighted feature energy.  It also reports, per reading, the size of the correction against
the output's own spread and the affine-explainable fraction of the probe residuals in
sample against the whole sequence (fit on the probes, evaluated on every row).  Everything
is computed by the oracle; nothing here is compared with the GPU.
"""
import argparse
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from oracle import sparsepr as O  # noqa: E402
from sparsepr_workloads import CONFIGS, small  # noqa: E402
from sparsepr_workloads import generator as gen  # noqa: E402


def fit_variant(od, os_, w, lam, rank, lam_mode):
    R = od - os_
    xbar, ybar, Xt, Yt = O.weighted_center(os_, R, w)
    if lam_mode == "relative":      # lambda times the mean weighted feature energy per probe
        lam = lam * float((Xt * Xt).sum()) / Xt.shape[0]
    Z = np.linalg.solve(Xt @ Xt.T + lam * np.eye(Xt.shape[0]), Yt)
    W = Xt.T @ Z
    V, _ = O.output_subspace(Yt, rank)
    A, B = W @ V, V.T
    c0 = ybar - xbar @ A @ B
    cond = np.linalg.cond(Xt @ Xt.T + lam * np.eye(Xt.shape[0]))
    return A, B, c0, cond


def study(cfg, heads, rows=None):
    p = O.Params(cfg.groups_q, cfg.groups_k, float(np.float32(cfg.rho_exec)), lam=float(np.float32(cfg.lam)))
    scale = 1 / np.sqrt(cfg.d)
    variants = {
        "mean-one weights, absolute lambda (kept)": ("mean1", "absolute"),
        "weights = tokens per probe, absolute lambda": ("tokens", "absolute"),
        "mean-one weights, lambda relative to feature energy": ("mean1", "relative"),
        "unit weights, absolute lambda": ("unit", "absolute"),
    }
    acc = {k: [] for k in ["hard drop"] + list(variants)}
    extra = {k: [] for k in variants}
    for kv in range(min(heads, cfg.heads_kv)):
        qh, k, v = gen.head_inputs(cfg, kv)
        part = O.partition(qh, k, p)
        rt = O.route(part, p, cfg.n)
        pr = O.select_probes(part.xq, part.q_labels, part.q_centroids, np.diff(part.q_offsets), cfg.n_probe)
        counts = np.diff(part.q_offsets)
        for j in range(cfg.g):
            q = qh[j]
            od_all, _ = O.dense_attention(q, k, v, scale)
            os_all, _ = O.sparse_attention(q, k, v, scale, part.q_labels, part.k_labels, rt.kept)
            nonprobe = np.setdiff1d(np.arange(cfg.n), pr.tokens)
            err = np.abs(os_all[nonprobe] - od_all[nonprobe])
            acc["hard drop"].append((err.mean(), np.percentile(err, 99)))
            od, os_ = od_all[pr.tokens], os_all[pr.tokens]
            spread = np.sqrt(((os_all - os_all.mean(0)) ** 2).mean())
            for name, (wmode, lmode) in variants.items():
                if wmode == "mean1":
                    w = pr.weights
                elif wmode == "tokens":
                    w = pr.weights * cfg.n / cfg.n_probe
                else:
                    w = np.ones(cfg.n_probe)
                A, B, c0, cond = fit_variant(od, os_, w, p.lam, p.rank, lmode)
                corr = c0[None, :] + (os_all[nonprobe] @ A) @ B
                out = os_all[nonprobe] + corr
                e = np.abs(out - od_all[nonprobe])
                acc[name].append((e.mean(), np.percentile(e, 99)))
                R_all = od_all[nonprobe] - os_all[nonprobe]
                expl = 1 - ((R_all - corr) ** 2).sum() / max(((R_all - R_all.mean(0)) ** 2).sum(), 1e-300)
                extra[name].append((np.sqrt((corr ** 2).mean()) / spread, expl, cond))
        del counts
    return acc, extra


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", type=int, nargs="+", default=[2, 4, 5])
    ap.add_argument("--heads", type=int, default=2)
    args = ap.parse_args()
    shrink = {4: dict(grid=(6, 24, 32), heads_q=10, heads_kv=2), 5: dict(grid=(4, 24, 32), heads_q=4),
              3: dict(grid=(6, 24, 32), heads_q=6), 2: dict(grid=(8, 32, 32), heads_q=8)}
    for w in args.workloads:
        base = CONFIGS[w]
        kw = shrink.get(w, {})
        cfg = small(base, kw.get("grid", base.grid), heads_q=kw.get("heads_q"), heads_kv=kw.get("heads_kv"),
                    groups=64) if kw else base
        acc, extra = study(cfg, args.heads)
        print(f"\n== {base.name}: N={cfg.n}, {cfg.heads_q}q/{cfg.heads_kv}kv (first {args.heads} KV heads)")
        print(f"{'reading':55s} {'mean':>8s} {'p99':>8s} {'|corr|/spread':>14s} {'expl. frac':>10s} {'cond':>9s}")
        for name, vals in acc.items():
            m = np.mean([a for a, _ in vals]); q99 = np.mean([b for _, b in vals])
            if name in extra:
                r = np.mean([a for a, _, _ in extra[name]]); e = np.mean([b for _, b, _ in extra[name]])
                c = np.median([c for _, _, c in extra[name]])
                print(f"{name:55s} {m:8.4f} {q99:8.4f} {r:14.3f} {e:10.3f} {c:9.2e}")
            else:
                print(f"{name:55s} {m:8.4f} {q99:8.4f}")


if __name__ == "__main__":
    main()
