"""GPU parity of the residual diagnostics (summary page of "Partition the Support,
Reconstruct the Residual", partition paragraph: the share of the hard-drop residual that is
an affine function of the sparse output and the energy orthogonal to it) against the
oracle's least-squares statistics, computed in float64 from the oracle's dense and sparse
outputs on the GPU's labels and kept cells, for both partitions.  Bars: explainable
fraction within 1e-2 (bf16) / 1e-6 (fp32) absolute, energies within 3 % (bf16) / 1e-5
(fp32) relative (the GPU's outputs carry the attention kernels' rounding)."""
import numpy as np
import pytest

from oracle import diagnostics as Dg
from oracle import sparsepr as O
from sparsepr_workloads import CONFIGS, small

from gpu_harness import device_tensor, host, kept_from_mask, oracle_inputs

pytestmark = pytest.mark.gpu

CASES = {
    "c1_fp32_local": CONFIGS[1],
    "c3_bf16_local_cross_global_ragged": small(CONFIGS[3], (3, 15, 24), heads_q=3, groups=16),
    "c4_bf16_gqa_ragged": small(CONFIGS[4], (2, 15, 20), heads_q=10, heads_kv=2, groups=16),
}


@pytest.mark.parametrize("partition_mode", [0, 1], ids=["response", "semantic"])
@pytest.mark.parametrize("cname", sorted(CASES))
def test_residual_diagnostics_match_oracle(cname, partition_mode):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import free_block_sparse_sparsepr_amd as S
    cfg = CASES[cname]
    print(f"\n[diagnostics {cname} partition_mode={partition_mode}]", flush=True)
    Q, K, V = oracle_inputs(cfg)
    sp = S.SparsePR(S.config_from_workload(cfg, partition_mode=partition_mode))
    q, k, v = device_tensor(Q, cfg), device_tensor(K, cfg), device_tensor(V, cfg)
    sp.partition(q, k, v)
    sp.route()
    got = host(sp.residual_diagnostics(q, k, v))
    torch.cuda.synchronize()
    ql_all, kl_all, km_all = host(sp.part["query_labels"]), host(sp.part["key_labels"]), host(sp.route_buf["kept_mask"])
    fp32 = cfg.dtype == "fp32"
    scale = 1 / np.sqrt(cfg.d)
    for h in range(cfg.heads_q):
        kv = h // cfg.g
        kept = kept_from_mask(km_all[kv], cfg.groups_q, cfg.groups_k)
        o_s, _ = O.sparse_attention(Q[h], K[kv], V[kv], scale, ql_all[kv], kl_all[kv], kept)
        o_d, _ = O.dense_attention(Q[h], K[kv], V[kv], scale)
        want = np.array(Dg.affine_residual_stats(o_s, o_d))
        rel = 1e-5 if fp32 else 3e-2
        np.testing.assert_allclose(got[h][:3], want[:3], rtol=rel, err_msg=f"energies h={h}")
        assert abs(got[h][3] - want[3]) <= (1e-6 if fp32 else 1e-2), (h, got[h][3], want[3])
