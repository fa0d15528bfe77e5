"""GPU parity of the budget variants (summary page of "Partition the Support, Reconstruct
the Residual", execution paragraph: the router spends a pair budget over indivisible
cells): tile-padded cell costs, one budget shared by all KV heads, and both.  The route is
bit-exact against the oracle fed the GPU's response matrices.  The whole call's output
(overlapped and fused orders) is checked on sampled rows within the bf16 bar against the
oracle's own probe fit (float64 probe rows, ridge and subspace) on the GPU's labels, cells
and probes; the probe rows themselves within 1e-3 of the oracle's exact attention."""
import numpy as np
import pytest

from oracle import sparsepr as O
from sparsepr_workloads import CONFIGS, small

from gpu_harness import compare_float, device_tensor, host, kept_from_mask, oracle_inputs, oracle_params, gpu_coord_sum

pytestmark = pytest.mark.gpu

PROBE_ROW_MAX_ABS = 1e-3   # probe rows: fp32 scores, probabilities as a bf16 high + remainder pair

CASES = {
    "c2_bf16_mixed_scales": small(CONFIGS[2], (8, 16, 16), heads_q=4, groups=16),
    "c3_bf16_ragged": small(CONFIGS[3], (3, 15, 24), heads_q=3, groups=16),
    "c4_bf16_gqa_ragged": small(CONFIGS[4], (2, 15, 20), heads_q=10, heads_kv=2, groups=16),
}
MODES = {"tiles": (0, 1), "global": (1, 0), "global_tiles": (1, 1)}


@pytest.fixture(scope="module", params=[(c, m) for c in sorted(CASES) for m in MODES],
                ids=lambda t: f"{t[0]}-{t[1]}")
def run(request):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dataclasses
    import free_block_sparse_sparsepr_amd as S
    cname, mode = request.param
    cfg = CASES[cname]
    budget_mode, cost_mode = MODES[mode]
    print(f"\n[budget {cname} {mode}]", flush=True)
    Q, K, V = oracle_inputs(cfg)
    sp = S.SparsePR(S.config_from_workload(cfg, budget_mode=budget_mode, cost_mode=cost_mode))
    q, k, v = device_tensor(Q, cfg), device_tensor(K, cfg), device_tensor(V, cfg)
    out = host(sp.overlapped(q, k, v).clone())
    out_fused = host(sp.fused(q, k, v).clone())
    torch.cuda.synchronize()
    gpu = {n: host(t) for n, t in {**sp.part, **sp.route_buf, **sp.fit}.items()}
    p = dataclasses.replace(oracle_params(cfg), tile_cost=64 if cost_mode else 0, global_budget=bool(budget_mode))
    parts = [O.partition(Q[kv * cfg.g:(kv + 1) * cfg.g], K[kv], p, S=gpu["responses_s"][kv],
                         U=gpu["responses_u"][kv * cfg.g:(kv + 1) * cfg.g], U_sum=gpu_coord_sum(gpu, cfg, kv))
             for kv in range(cfg.heads_kv)]
    return dict(cfg=cfg, p=p, Q=Q, K=K, V=V, gpu=gpu, out=out, out_fused=out_fused, parts=parts)


def test_route_variant_bit_exact(run):
    cfg, gpu, p = run["cfg"], run["gpu"], run["p"]
    routes = O.route_heads(run["parts"], p, cfg.n)
    for kv, r in enumerate(routes):
        np.testing.assert_array_equal(gpu["cell_mass"][kv].astype(np.int64), r.mass)
        nnz = int(r.row_ptr[-1])
        np.testing.assert_array_equal(gpu["row_ptr"][kv], r.row_ptr)
        np.testing.assert_array_equal(gpu["cols"][kv][:nnz], r.cols)
        np.testing.assert_array_equal(kept_from_mask(gpu["kept_mask"][kv], cfg.groups_q, cfg.groups_k), r.kept)
        assert gpu["pairs"][kv] == r.pairs
    if p.global_budget:
        costs = [O.cell_costs(np.diff(pt.q_offsets), np.diff(pt.k_offsets), p.tile_cost) for pt in run["parts"]]
        spent = sum(int(c[r.kept].sum()) for c, r in zip(costs, routes))
        assert spent <= routes[0].budget or all((r.kept == r.mandatory).all() for r in routes)


def test_outputs_follow_the_variant_route(run):
    cfg, gpu, p = run["cfg"], run["gpu"], run["p"]
    scale = 1 / np.sqrt(cfg.d)
    rng = np.random.default_rng(cfg.cfg_id)
    for kv in sorted({0, cfg.heads_kv - 1}):
        ql, kl = gpu["query_labels"][kv], gpu["key_labels"][kv]
        kept = kept_from_mask(gpu["kept_mask"][kv], cfg.groups_q, cfg.groups_k)
        probes = O.Probes(gpu["probe_tokens"][kv].astype(np.int64), gpu["probe_groups"][kv].astype(np.int64),
                          gpu["probe_weights"][kv], None)
        rows = np.unique(np.concatenate([[0, cfg.n - 1], rng.choice(cfg.n, 96, replace=False)]))
        rows = np.setdiff1d(rows, probes.tokens)
        h = kv * cfg.g
        q, k, v = run["Q"][h], run["K"][kv], run["V"][kv]
        exact = O.probe_fit(q, k, v, scale, probes, ql, kl, kept, p)
        ok, mx, mean = compare_float(gpu["o_dense"][h], exact.o_dense, False)
        assert ok and mx <= PROBE_ROW_MAX_ABS, ("o_dense", h, mx, mean)
        ok, mx, mean = compare_float(gpu["o_sparse"][h], exact.o_sparse, False)
        assert ok and mx <= PROBE_ROW_MAX_ABS, ("o_sparse", h, mx, mean)
        o_s, _ = O.sparse_attention(q, k, v, scale, ql, kl, kept, rows=rows)
        want = O.correct_rows(o_s, exact)
        for name in ("out", "out_fused"):
            ok, mx, mean = compare_float(run[name][h][rows], want, False)
            assert ok, (name, h, mx, mean)
            ok, mx, mean = compare_float(run[name][h][probes.tokens], exact.o_dense, False)
            assert ok, (name, "probe rows", h, mx, mean)
