"""GPU parity of the partition's k-means for several iteration counts (no iteration, one,
and a few) on both assignment paths: feature widths 16 and 48 use the matrix-core
assignment, whose centroid update is folded into the next assignment; widths 20 and 36 the
vector one with a separate update.  Labels and integer centroids must be bit-exact with the
oracle fed the GPU's response matrices."""
import dataclasses

import numpy as np
import pytest

from oracle import sparsepr as O
from sparsepr_workloads import CONFIGS, small

from gpu_harness import device_tensor, host, oracle_inputs, oracle_params, gpu_coord_sum

pytestmark = pytest.mark.gpu

BASE = small(CONFIGS[3], (3, 15, 24), heads_q=3, groups=16)
CASES = [("mfma", it, dataclasses.replace(BASE, kmeans_iters=it)) for it in (0, 1, 2, 3)] + \
        [("vector", it, dataclasses.replace(BASE, kmeans_iters=it, groups_q=20, groups_k=20, r_k=36))
         for it in (1, 3)]


@pytest.mark.parametrize("path,iters,cfg", CASES, ids=[f"{p}_iters{i}" for p, i, _ in CASES])
def test_kmeans_iterations_bit_exact(path, iters, cfg):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import free_block_sparse_sparsepr_amd as S
    print(f"\n[kmeans {path} iters={iters}] N={cfg.n} G={cfg.groups_q} r_k={cfg.r_k}", flush=True)
    Q, K, V = oracle_inputs(cfg)
    sp = S.SparsePR(S.config_from_workload(cfg))
    sp(device_tensor(Q, cfg), device_tensor(K, cfg), device_tensor(V, cfg))
    torch.cuda.synchronize()
    gpu = {k: host(t) for k, t in sp.part.items()}
    p = oracle_params(cfg)
    assert p.kmeans_iters == iters
    for kv in range(cfg.heads_kv):
        qh = Q[kv * cfg.g:(kv + 1) * cfg.g]
        part = O.partition(qh, K[kv], p, S=gpu["responses_s"][kv], U=gpu["responses_u"][kv * cfg.g:(kv + 1) * cfg.g],
                           U_sum=gpu_coord_sum(gpu, cfg, kv))
        np.testing.assert_array_equal(gpu["key_labels"][kv], part.k_labels)
        np.testing.assert_array_equal(gpu["key_centroids_int"][kv], part.k_centroids_int[:, :cfg.r_k])
        np.testing.assert_array_equal(gpu["query_labels"][kv], part.q_labels)
        np.testing.assert_array_equal(gpu["query_centroids"][kv], part.q_centroids)
