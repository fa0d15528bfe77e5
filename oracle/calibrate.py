"""Calibrate the signal amplitude of every workload head type (test infrastructure).

For each workload and head type, the amplitude a of Q = a s phi G + 0.3 eps (s = 1
during calibration) is found by 24 bisection steps on log a in [log 0.05, log 4] so that
the median single-row 90 %-mass support over 256 evenly spaced rows (float64, before
the bf16 cast) hits the type's target (PSRR support paragraph: 6.2 % for local and
cross-shaped heads, 56.5 % for global heads; 55 % for the world-model-shaped call).
The first KV head of each type is used.  Writes sparsepr_workloads/amplitudes.json.

Run: python -m oracle.calibrate
"""
import json
import os
import sys

import numpy as np

from sparsepr_workloads import CONFIGS
from sparsepr_workloads import generator as gen

from .diagnostics import median_support

STEPS = 24
LOG_LO, LOG_HI = np.log(0.05), np.log(4.0)


def calibrate_type(cfg, kv_head, target):
    sig = gen.signal(cfg, kv_head)
    qn = gen.NOISE_STD * gen.noise(cfg, kv_head * cfg.g, 2)
    kn = gen.NOISE_STD * gen.noise(cfg, kv_head, 3)
    scale = 1.0 / np.sqrt(cfg.d)
    lo, hi = LOG_LO, LOG_HI
    for _ in range(STEPS):
        mid = 0.5 * (lo + hi)
        a = np.exp(mid)
        sup = median_support(a * sig + qn, a * sig + kn, scale)
        if sup > target:
            lo = mid      # too diffuse: sharpen
        else:
            hi = mid
    a = float(np.exp(0.5 * (lo + hi)))
    return a, median_support(a * sig + qn, a * sig + kn, scale)


def main(cfg_ids=None):
    out_path = gen._AMP_FILE
    table = {}
    if os.path.exists(out_path):
        with open(out_path) as f:
            table = json.load(f)
    for cid in (cfg_ids or sorted(CONFIGS)):
        cfg = CONFIGS[cid]
        entry = {}
        for kind, target in cfg.support_target:
            kv = cfg.head_types.index(kind)
            a, sup = calibrate_type(cfg, kv, target)
            entry[kind] = a
            entry[kind + "_support"] = sup
            print(f"cfg {cid} {kind}: a = {a:.6f}, median support = {sup:.4f} (target {target})",
                  flush=True)
        table[str(cid)] = entry
        with open(out_path, "w") as f:
            json.dump(table, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main([int(x) for x in sys.argv[1:]] or None)
