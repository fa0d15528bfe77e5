"""The seeded workload generator (CPU): determinism, shapes, casting, page figures."""
import json
import os

import numpy as np
import pytest

from sparsepr_workloads import CONFIGS, round_to_bf16, small
from sparsepr_workloads import generator as gen

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def _bf16_neighbours(r):
    bits = r.astype(np.float32).view(np.uint32)
    up = (bits + (1 << 16)).view(np.float32)
    dn = (bits - (1 << 16)).view(np.float32)
    return dn, up


def test_round_to_bf16_is_nearest_even():
    x = np.random.default_rng(0).standard_normal(20000) * 3
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]   # exact ties
    r = round_to_bf16(x)
    assert not np.any(r.view(np.uint32) & 0xFFFF)           # representable in bf16
    nz = r != 0
    dn, up = _bf16_neighbours(r[nz])
    err = np.abs(x[nz] - r[nz].astype(np.float64))
    assert np.all(err <= np.abs(x[nz] - dn)) and np.all(err <= np.abs(x[nz] - up))
    assert r[0] == 1.0 and r[1] == 1.0 + 4 * 2 ** -8 and r[2] == -1.0 and r[3] == 0.0
    torch = pytest.importorskip("torch")
    t = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).float().numpy()
    # float32 -> bf16 in torch is also round-to-nearest-even; x was float64, so only
    # double-rounding cases may differ
    assert np.mean(t == r) > 0.999


def test_generator_is_deterministic_and_shaped():
    cfg = small(CONFIGS[4], (2, 8, 8), heads_q=10, heads_kv=2)
    q1, k1, v1 = gen.head_inputs(cfg, 1)
    q2, k2, v2 = gen.head_inputs(cfg, 1)
    assert q1.shape == (5, 128, 128) and k1.shape == (128, 128)
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(v1, v2)
    Q, K, V = gen.make_inputs(cfg, threads=2)
    np.testing.assert_array_equal(Q[5:10], q1)
    np.testing.assert_array_equal(K[1], k1)
    assert not np.array_equal(Q[5], Q[6])      # own noise and scale per query head


def test_config_shapes_and_probe_fraction_match_page():
    assert [CONFIGS[i].n for i in range(1, 6)] == [1024, 8192, 118800, 75600, 43200]
    c3 = CONFIGS[3]
    assert (c3.r_k, c3.r_q, c3.n_probe, c3.rank, c3.lam) == (
        GOLD["r_k"]["value"], GOLD["r_q"]["value"], GOLD["n_probe"]["value"],
        GOLD["rank"]["value"], GOLD["lambda"]["value"])
    lo, hi = GOLD["probe_pair_fraction_range_percent"]["value"]
    # 64 probe rows of a 118,800-token call are the page's 0.054 %
    assert round(100 * 64 / c3.n, 3) == lo
    for i in (3, 4, 5):
        assert lo - 1e-3 <= 100 * 64 / CONFIGS[i].n <= 0.15
    tgt = GOLD["target_density_percent"]["value"]
    assert CONFIGS[3].rho_exec * 100 == tgt["HunyuanVideo"]
    assert CONFIGS[5].rho_exec * 100 == tgt["Cosmos3-Nano"]


def test_calibrated_amplitudes_present():
    table = gen.load_amplitudes()
    for cid, cfg in CONFIGS.items():
        for kind, target in cfg.support_target:
            assert abs(table[str(cid)][kind + "_support"] - target) < 0.002
