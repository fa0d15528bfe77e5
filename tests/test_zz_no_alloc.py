"""The allocation-free attention entry point (sparsepr_attend_noalloc) against sparsepr_attend,
called through the C ABI: two calls in a row on one GPU, the second with a smaller input,
each bit-identical to sparsepr_attend on the same partition and route (same kernels, same
schedule; only where the schedule is kept differs)."""
import pytest

from sparsepr_workloads import CONFIGS, small

from gpu_harness import device_tensor, oracle_inputs

pytestmark = pytest.mark.gpu

SHAPES = [  # larger first, then smaller: the second call reuses the array the first one filled
    ("bf16 GQA 10q/2kv", small(CONFIGS[4], (3, 15, 24), heads_q=10, heads_kv=2, groups=16)),
    ("bf16 ragged 3 heads", small(CONFIGS[3], (2, 13, 17), heads_q=3, groups=16)),
]


def test_noalloc_attend_matches_attend_twice():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import free_block_sparse_sparsepr_amd as S
    for name, cfg in SHAPES:
        print(f"\n[noalloc {name}] N={cfg.n} Hq={cfg.heads_q} Hkv={cfg.heads_kv}", flush=True)
        Q, K, V = oracle_inputs(cfg)
        sp = S.SparsePR(S.config_from_workload(cfg))
        q, k, v = device_tensor(Q, cfg), device_tensor(K, cfg), device_tensor(V, cfg)
        sp.partition(q, k, v)
        sp.route()
        sp.attend()
        ref_o, ref_lse = sp.o_gm.clone(), sp.lse.clone()
        sp.o_gm.fill_(float("nan"))
        sp.lse.fill_(float("nan"))
        sp.attend_noalloc()
        torch.cuda.synchronize()
        assert torch.equal(sp.o_gm, ref_o), name
        assert torch.equal(sp.lse, ref_lse), name
