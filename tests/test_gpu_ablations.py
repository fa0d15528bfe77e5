"""GPU parity of the ablation switches (summary page of "Partition the Support, Reconstruct
the Residual", ablation paragraph) against the CPU oracle: hard drop, the ridge fit without
the rank-r projection, and probe rows drawn uniformly over the raster order or given by
the caller (here drawn at random on the host).  Partition and route are those of the
method; the oracle is fed the GPU's labels and kept cells.  Both call orders (fused and
unfused) are checked; bars as in test_gpu_parity (bf16 max-abs 2e-2, mean-abs 2e-3; fp32
max-abs 1e-4)."""
import numpy as np
import pytest

from oracle import sparsepr as O
from sparsepr_workloads import CONFIGS, small

from gpu_harness import compare_float, device_tensor, host, kept_from_mask, oracle_inputs, oracle_params, gpu_coord_sum

pytestmark = pytest.mark.gpu

CASES = {
    "c1_fp32_local": CONFIGS[1],
    "c3_bf16_local_cross_global_ragged": small(CONFIGS[3], (3, 15, 24), heads_q=3, groups=16),
    "c4_bf16_gqa_ragged": small(CONFIGS[4], (2, 15, 20), heads_q=10, heads_kv=2, groups=16),
}
VARIANTS = {
    "hard_drop": dict(ablation=1, probe_mode=0),
    "ridge_only": dict(ablation=2, probe_mode=0),
    "uniform_probes": dict(ablation=0, probe_mode=1),
    "random_probes": dict(ablation=0, probe_mode=2),
    "semantic": dict(partition_mode=1),
    "semantic_hard_drop": dict(partition_mode=1, ablation=1),
}


def _random_tokens(cfg, seed):
    rng = np.random.default_rng([seed, cfg.cfg_id])
    return np.stack([np.sort(rng.choice(cfg.n, cfg.n_probe, replace=False)) for _ in range(cfg.heads_kv)])


@pytest.fixture(scope="module", params=[(c, v) for c in sorted(CASES) for v in sorted(VARIANTS)],
                ids=lambda cv: f"{cv[0]}-{cv[1]}")
def r(request):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import free_block_sparse_sparsepr_amd as S
    cname, vname = request.param
    cfg = CASES[cname]
    print(f"\n[ablation {vname} on {cname}] N={cfg.n} Hq={cfg.heads_q} Hkv={cfg.heads_kv}", flush=True)
    Q, K, V = oracle_inputs(cfg)
    sp = S.SparsePR(S.config_from_workload(cfg, **VARIANTS[vname]))
    q, k, v = device_tensor(Q, cfg), device_tensor(K, cfg), device_tensor(V, cfg)
    given = _random_tokens(cfg, 7) if vname == "random_probes" else None

    def set_tokens():
        if given is not None:
            sp.fit["probe_tokens"].copy_(torch.from_numpy(given.astype(np.int32)))

    sp.partition(q, k, v)
    sp.route()
    sp.attend()
    set_tokens()
    sp.probe_fit(q)
    out = host(sp.apply())
    set_tokens()
    sp.probe_fit(q)
    out_fused = host(sp.attend_apply())
    torch.cuda.synchronize()
    gpu = {k_: host(t) for k_, t in {**sp.part, **sp.route_buf, **sp.fit}.items()}
    return dict(cfg=cfg, variant=vname, Q=Q, K=K, V=V, gpu=gpu, out=out, out_fused=out_fused, given=given,
                p=oracle_params(cfg))


def _expected(r, kv, j):
    """The oracle's output of query head kv*g+j for the variant, on the GPU's partition."""
    cfg, gpu, p, vname = r["cfg"], r["gpu"], r["p"], r["variant"]
    h = kv * cfg.g + j
    scale = 1 / np.sqrt(cfg.d)
    ql, kl = gpu["query_labels"][kv], gpu["key_labels"][kv]
    kept = kept_from_mask(gpu["kept_mask"][kv], cfg.groups_q, cfg.groups_k)
    q, k, v = r["Q"][h], r["K"][kv], r["V"][kv]
    o_s, _ = O.sparse_attention(q, k, v, scale, ql, kl, kept)
    if vname.endswith("hard_drop"):
        return O.hard_drop_rows(q, k, v, scale, ql, kl, kept), None, None
    if vname == "uniform_probes":
        probes = O.uniform_probes(cfg.n, ql, cfg.n_probe)
    elif vname == "random_probes":
        probes = O.given_probes(r["given"][kv], ql)
    else:
        probes = O.Probes(gpu["probe_tokens"][kv].astype(np.int64), gpu["probe_groups"][kv].astype(np.int64),
                          gpu["probe_weights"][kv], None)
    if vname == "ridge_only":
        fit = O.ridge_only_fit(q, k, v, scale, probes, ql, kl, kept, p)
    else:
        fit = O.probe_fit(q, k, v, scale, probes, ql, kl, kept, p)
    return O.apply_correction(o_s, fit, probes.tokens), fit, probes


def test_probe_rows_of_the_variant(r):
    cfg, gpu, vname = r["cfg"], r["gpu"], r["variant"]
    for kv in range(cfg.heads_kv):
        ql = gpu["query_labels"][kv]
        if vname.endswith("hard_drop"):
            assert (gpu["probe_tokens"][kv] == -1).all() and (gpu["r_eff"] == 0).all()
            assert not gpu["A"].any() and not gpu["B"].any() and not gpu["c0"].any()
            continue
        if vname == "uniform_probes":
            want = O.uniform_probes(cfg.n, ql, cfg.n_probe)
        elif vname == "random_probes":
            want = O.given_probes(r["given"][kv], ql)
        else:
            continue
        np.testing.assert_array_equal(gpu["probe_tokens"][kv], want.tokens)
        np.testing.assert_array_equal(gpu["probe_groups"][kv], want.groups)
        np.testing.assert_array_equal(gpu["probe_weights"][kv], want.weights)


def test_output_of_the_variant_matches_oracle(r):
    cfg, gpu, vname = r["cfg"], r["gpu"], r["variant"]
    fp32 = cfg.dtype == "fp32"
    for kv in range(cfg.heads_kv):
        for j in range(cfg.g):
            h = kv * cfg.g + j
            want, fit, probes = _expected(r, kv, j)
            ok, mx, mean = compare_float(r["out"][h], want, fp32)
            assert ok, (vname, "unfused", h, mx, mean)
            ok, mx, mean = compare_float(r["out_fused"][h], want, fp32)
            assert ok, (vname, "fused", h, mx, mean)
            if vname == "ridge_only":
                assert int(gpu["r_eff"][h]) == cfg.n_probe
                ok, mx, mean = compare_float(gpu["c0"][h], fit.c0, fp32)
                assert ok, ("c0", h, mx, mean)


def test_semantic_partition_bit_exact(r):
    """Semantic partition: the oracle, fed the GPU's query responses U (which only the route
    uses), reproduces the raw-activation features, both k-means, the permutations, the
    route and (with probes) the radial probe choice bit for bit."""
    cfg, gpu, p = r["cfg"], r["gpu"], r["p"]
    if not r["variant"].startswith("semantic"):
        pytest.skip("response-coupled partition (covered by test_gpu_parity)")
    for kv in range(cfg.heads_kv):
        qh = r["Q"][kv * cfg.g:(kv + 1) * cfg.g]
        part = O.partition_semantic(qh, r["K"][kv], p, U=gpu["responses_u"][kv * cfg.g:(kv + 1) * cfg.g],
                                    x_sum=gpu_coord_sum(gpu, cfg, kv))
        np.testing.assert_array_equal(gpu["key_labels"][kv], part.k_labels)
        np.testing.assert_array_equal(gpu["key_centroids_int"][kv], part.k_centroids_int)
        np.testing.assert_array_equal(gpu["key_perm"][kv], part.k_perm)
        np.testing.assert_array_equal(gpu["key_offsets"][kv], part.k_offsets)
        np.testing.assert_array_equal(gpu["query_features"][kv], part.xq)
        np.testing.assert_array_equal(gpu["query_labels"][kv], part.q_labels)
        np.testing.assert_array_equal(gpu["query_centroids"][kv], part.q_centroids)
        np.testing.assert_array_equal(gpu["query_perm"][kv], part.q_perm)
        np.testing.assert_array_equal(gpu["exponents"][kv], [part.e_s, part.e_u])
        rt = O.route(part, p, cfg.n)
        np.testing.assert_array_equal(gpu["cell_mass"][kv].astype(np.int64), rt.mass)
        np.testing.assert_array_equal(kept_from_mask(gpu["kept_mask"][kv], cfg.groups_q, cfg.groups_k), rt.kept)
        if r["variant"] == "semantic":
            pr = O.select_probes(part.xq, part.q_labels, part.q_centroids, np.diff(part.q_offsets), cfg.n_probe)
            np.testing.assert_array_equal(gpu["probe_tokens"][kv], pr.tokens)
