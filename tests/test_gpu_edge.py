"""Edge cases of the whole call on the GPU against the oracle: fewer tokens than one key
tile (n = 48, probe rows a third of the tokens), a token count that is not a multiple of
16 (n = 1025), the maximum density (rho_exec = 1: the budget is n^2 less the probe rows, so
all but the lightest cells are kept), bf16 with d = 64, and the largest GQA ratio (16 query heads on one KV head).  Integer stages
bit-exact given the GPU's response matrices (and head-summed U); probe rows against the
oracle's exact attention (within 1e-3: their probabilities enter the value product as a bf16
pair, high part and remainder), and every output row against the oracle's own probe fit
(float64 probe rows, ridge and subspace) within the bf16 bar; the overlapped order
bit-exact with the unfused one."""
import dataclasses

import numpy as np
import pytest

from oracle import sparsepr as O
from sparsepr_workloads import CONFIGS, small

from gpu_harness import compare_float, host, kept_from_mask, oracle_inputs, oracle_params, run_gpu, gpu_coord_sum

pytestmark = pytest.mark.gpu

PROBE_ROW_MAX_ABS = 1e-3   # probe rows: fp32 scores, probabilities as a bf16 high + remainder pair

CASES = {
    "n48_tiny": dataclasses.replace(small(CONFIGS[3], (1, 6, 8), heads_q=2, groups=4), n_probe=16, rank=4, r_k=8,
                                    rho_exec=0.6),
    "n1025_ragged": small(CONFIGS[3], (1, 25, 41), heads_q=2, groups=16),
    "max_density": dataclasses.replace(small(CONFIGS[3], (2, 15, 20), heads_q=2, groups=16), rho_exec=1.0),
    "bf16_d64": dataclasses.replace(small(CONFIGS[2], (4, 16, 16), heads_q=2, groups=16), d=64),
    "gqa_g16": small(CONFIGS[4], (2, 15, 20), heads_q=16, heads_kv=1, groups=16),
}


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = CASES[request.param]
    print(f"\n[edge {request.param}] N={cfg.n} Hq={cfg.heads_q} Hkv={cfg.heads_kv} d={cfg.d}", flush=True)
    Q, K, V = oracle_inputs(cfg)
    gpu, sp, (q, k, v) = run_gpu(cfg, Q, K, V)
    gpu["out_overlapped"] = host(sp.overlapped(q, k, v))
    torch.cuda.synchronize()
    p = oracle_params(cfg)
    p = dataclasses.replace(p, n_probe=cfg.n_probe, rank=cfg.rank, r_k=cfg.r_k)
    parts = [O.partition(Q[kv * cfg.g:(kv + 1) * cfg.g], K[kv], p, S=gpu["responses_s"][kv],
                         U=gpu["responses_u"][kv * cfg.g:(kv + 1) * cfg.g], U_sum=gpu_coord_sum(gpu, cfg, kv))
             for kv in range(cfg.heads_kv)]
    return dict(name=request.param, cfg=cfg, Q=Q, K=K, V=V, gpu=gpu, p=p, parts=parts)


def test_integer_stages_bit_exact(case):
    cfg, gpu, p = case["cfg"], case["gpu"], case["p"]
    for kv, part in enumerate(case["parts"]):
        np.testing.assert_array_equal(gpu["key_labels"][kv], part.k_labels)
        np.testing.assert_array_equal(gpu["query_labels"][kv], part.q_labels)
        np.testing.assert_array_equal(gpu["query_perm"][kv], part.q_perm)
        r = O.route(part, p, cfg.n)
        np.testing.assert_array_equal(kept_from_mask(gpu["kept_mask"][kv], cfg.groups_q, cfg.groups_k), r.kept)
        assert gpu["pairs"][kv] == r.pairs
        if cfg.rho_exec >= 1.0:
            assert r.budget == cfg.n * cfg.n - cfg.n_probe * cfg.n and r.pairs >= r.budget - cfg.n * cfg.n // 4
        pr = O.select_probes(part.xq, part.q_labels, part.q_centroids, np.diff(part.q_offsets), cfg.n_probe)
        np.testing.assert_array_equal(gpu["probe_tokens"][kv], pr.tokens)


def test_outputs_match_oracle(case):
    cfg, gpu, p = case["cfg"], case["gpu"], case["p"]
    scale = 1 / np.sqrt(cfg.d)
    for kv in range(cfg.heads_kv):
        ql, kl = gpu["query_labels"][kv], gpu["key_labels"][kv]
        kept = kept_from_mask(gpu["kept_mask"][kv], cfg.groups_q, cfg.groups_k)
        probes = O.Probes(gpu["probe_tokens"][kv].astype(np.int64), gpu["probe_groups"][kv].astype(np.int64),
                          gpu["probe_weights"][kv], None)
        for j in range(cfg.g):
            h = kv * cfg.g + j
            q, k, v = case["Q"][h], case["K"][kv], case["V"][kv]
            o_s, _ = O.sparse_attention(q, k, v, scale, ql, kl, kept)
            exact = O.probe_fit(q, k, v, scale, probes, ql, kl, kept, p)
            for name in ("o_dense", "o_sparse"):
                ok, mx, mean = compare_float(gpu[name][h], getattr(exact, name), False)
                assert ok and mx <= PROBE_ROW_MAX_ABS, (case["name"], name, h, mx, mean)
            want = O.apply_correction(o_s, exact, probes.tokens)
            want[probes.tokens] = exact.o_dense
            for name in ("out", "out_fused"):
                ok, mx, mean = compare_float(gpu[name][h], want, False)
                assert ok, (case["name"], name, h, mx, mean)
            od, _ = O.dense_attention(q, k, v, scale)
            ok, mx, mean = compare_float(gpu["dense"][h], od, False)
            assert ok, (case["name"], "dense", h, mx, mean)
    np.testing.assert_array_equal(gpu["out_overlapped"], gpu["out"])


def test_route_budget_at_the_largest_n():
    """The route's budget floor(rho_ppm n^2 / 10^6) - M n at the largest accepted n (2^22) and
    rho_exec = 1, where rho_ppm n^2 exceeds the 64-bit range: partition and route on seeded
    random bf16 inputs, then the kept cells and the realised pairs against the oracle's
    selection (Python integers) on the GPU's cell masses and group sizes."""
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import free_block_sparse_sparsepr_amd as S
    n, d = 1 << 22, 64
    print(f"\n[edge largest n] N={n} d={d} rho_exec=1", flush=True)
    cfg = S.Config(heads_q=1, heads_kv=1, n=n, d=d, rho_exec=1.0)
    sp = S.SparsePR(cfg)
    gen = torch.Generator(device="cuda").manual_seed(5)
    q, k, v = (torch.randn((1, n, d), generator=gen, device="cuda").to(torch.bfloat16) for _ in range(3))
    sp.partition(q, k, v)
    sp.route()
    torch.cuda.synchronize()
    m = host(sp.route_buf["cell_mass"])[0].astype(np.int64)      # cell masses < 2^42
    qc = np.diff(host(sp.part["query_offsets"])[0].astype(np.int64))
    kc = np.diff(host(sp.part["key_offsets"])[0].astype(np.int64))
    r = O.select_cells(m, qc, kc, 1.0, n, cfg.n_probe)
    assert r.budget == n * n - cfg.n_probe * n
    np.testing.assert_array_equal(kept_from_mask(host(sp.route_buf["kept_mask"])[0], 64, 64), r.kept)
    assert int(host(sp.route_buf["pairs"])[0]) == r.pairs
    assert r.pairs > r.budget - n * n // 8
