"""GPU parity of the support diagnostics (summary page of "Partition the Support,
Reconstruct the Residual", support paragraph: single-row 90 %-mass supports and their
union over queries that share a route) against the oracle.

The counts are integers decided from floating-point scores, so they are checked the way the
partition's integer stages are: the GPU's fp32 scores (read back from the workspace) are
within 1e-5 relative of the oracle's float64 scores, and given those scores the oracle's
integer decisions (fixed-point masses formed in double precision,
``supports_from_scores``) give every row count and every union bit-exact.  Each count is
also checked to be a valid float64 answer within 2e-5 of the mass.  Exact ties
(identical keys) are checked against their closed form."""
import math

import numpy as np
import pytest

from oracle import diagnostics as Dg
from sparsepr_workloads import CONFIGS, small

from gpu_harness import device_tensor, host, oracle_inputs

pytestmark = pytest.mark.gpu

TOL = 2e-5


def _sorted_probs(q, k, scale):
    s = (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T) * scale
    p = np.exp(s - s.max())
    p /= p.sum()
    return -np.sort(-p)


def _check(cfg, Q, K, sets, rows_gpu, union_gpu, mass):
    scale = 1 / math.sqrt(cfg.d)
    equal = total = 0
    for h in range(cfg.heads_q):
        kv = h // cfg.g
        for si in range(sets.shape[1]):
            toks = sets[h, si]
            valid = (toks >= 0) & (toks < cfg.n)
            assert (rows_gpu[h, si][~valid] == -1).all()
            if not valid.any():
                assert union_gpu[h, si] == 0
                continue
            cnt_ref, member = Dg.row_supports(Q[h], K[kv], scale, toks[valid], mass)
            budget = 0
            for r, t in enumerate(toks[valid]):
                kg = int(rows_gpu[h, si][valid][r])
                p = _sorted_probs(Q[h][t], K[kv], scale)
                c = np.cumsum(p)
                assert 1 <= kg <= cfg.n, (h, si, t, kg)
                assert c[kg - 1] >= mass - TOL and (kg == 1 or c[kg - 2] < mass + TOL), (h, si, t, kg, cnt_ref[r])
                budget += abs(kg - int(cnt_ref[r]))
                kr = int(cnt_ref[r])
                if kr < cfg.n and p[kr - 1] - p[kr] < 1e-5 * p[kr - 1]:
                    budget += 1
                equal += kg == cnt_ref[r]
                total += 1
            u_ref = int(member.any(axis=0).sum())
            assert abs(int(union_gpu[h, si]) - u_ref) <= budget, (h, si, union_gpu[h, si], u_ref, budget)
    assert equal >= 0.95 * total, (equal, total)


def _run(cfg, Q, K, sets, mass, with_scores=False):
    import torch
    import free_block_sparse_sparsepr_amd as S
    sp = S.SparsePR(S.config_from_workload(cfg))
    q, k = device_tensor(Q, cfg), device_tensor(K, cfg)
    res = sp.support_diagnostics(q, k, torch.from_numpy(sets.astype(np.int32)).cuda(), mass, with_scores=with_scores)
    torch.cuda.synchronize()
    return tuple(host(t) for t in res)


def _check_exact(cfg, Q, K, sets, rows_gpu, union_gpu, scores, mass):
    """Bit-exact counts and unions given the GPU's fp32 scores; the scores themselves against
    the float64 dot products."""
    scale = np.float32(1 / math.sqrt(cfg.d))
    for h in range(cfg.heads_q):
        kv = h // cfg.g
        for si in range(sets.shape[1]):
            toks = sets[h, si]
            valid = (toks >= 0) & (toks < cfg.n)
            if not valid.any():
                continue
            f = scores[h, si][valid]
            ref = np.asarray(Q[h], np.float64)[toks[valid]] @ np.asarray(K[kv], np.float64).T
            np.testing.assert_allclose(f, ref, rtol=1e-5, atol=1e-5 * np.abs(ref).max())
            cnt, member = Dg.supports_from_scores(f, scale, mass)
            np.testing.assert_array_equal(rows_gpu[h, si][valid], cnt)
            assert int(union_gpu[h, si]) == int(member.any(axis=0).sum()), (h, si)


def _consecutive_sets(cfg, n_sets, s, rng):
    starts = rng.integers(0, cfg.n - s + 1, (cfg.heads_q, n_sets))
    return starts[..., None] + np.arange(s)


CASES = {
    "c1_fp32": (CONFIGS[1], 24, 8),
    "c2_bf16_mixed_scales": (CONFIGS[2], 4, 8),
    "c4_bf16_gqa_ragged": (small(CONFIGS[4], (2, 15, 20), heads_q=10, heads_kv=2, groups=16), 6, 8),
    "c5_bf16_dense_support": (small(CONFIGS[5], (3, 16, 24), heads_q=2, groups=16), 5, 16),
}


@pytest.mark.parametrize("mass", [0.9, 0.5])
@pytest.mark.parametrize("kind", ["consecutive", "random"])
@pytest.mark.parametrize("cname", sorted(CASES))
def test_support_matches_oracle(cname, kind, mass):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg, n_sets, s = CASES[cname]
    print(f"\n[support {cname} {kind} mass={mass}]", flush=True)
    Q, K, _ = oracle_inputs(cfg)
    rng = np.random.default_rng(7)
    if kind == "consecutive":
        sets = _consecutive_sets(cfg, n_sets, s, rng)
    else:
        sets = rng.integers(0, cfg.n, (cfg.heads_q, n_sets, s))
    rows, union, scores = _run(cfg, Q, K, sets, mass, with_scores=True)
    _check_exact(cfg, Q, K, sets, rows, union, scores, mass)
    _check(cfg, Q, K, sets, rows, union, mass)


def test_support_invalid_tokens_and_many_items():
    """Tokens outside [0, n) give -1 and stay out of the union; more (head, set) items than
    concurrent slots (600 sets of 2 rows) exercise the work loop; set sizes 1 and 16."""
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = CONFIGS[1]
    print("\n[support invalid tokens, 600 items]", flush=True)
    Q, K, _ = oracle_inputs(cfg)
    rng = np.random.default_rng(3)
    sets = rng.integers(0, cfg.n, (1, 600, 2))
    sets[0, 5] = [-1, cfg.n]
    sets[0, 9, 1] = -7
    sets[0, 11, 0] = cfg.n + 3
    rows, union = _run(cfg, Q, K, sets, 0.9)
    assert union[0, 5] == 0
    _check(cfg, Q, K, sets, rows, union, 0.9)
    for s in (1, 16):
        sets = rng.integers(0, cfg.n, (1, 5, s))
        rows, union, scores = _run(cfg, Q, K, sets, 0.9, with_scores=True)
        _check_exact(cfg, Q, K, sets, rows, union, scores, 0.9)
        _check(cfg, Q, K, sets, rows, union, 0.9)
        if s == 1:
            np.testing.assert_array_equal(union[0], rows[0, :, 0])


@pytest.mark.parametrize("dtype_cfg", [1, 2])
def test_support_exact_ties(dtype_cfg):
    """Identical keys: every probability is 1/n, so each row needs ceil(0.9 n) keys, the
    lowest indices, and any union equals that count (the tie path of the select)."""
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = CONFIGS[dtype_cfg]
    print(f"\n[support ties {cfg.name}]", flush=True)
    Q, K, _ = oracle_inputs(cfg)
    K = np.ascontiguousarray(np.broadcast_to(K[:, :1, :], K.shape))
    rng = np.random.default_rng(5)
    sets = rng.integers(0, cfg.n, (cfg.heads_q, 3, 8))
    rows, union = _run(cfg, Q, K, sets, 0.9)
    want = math.ceil(0.9 * cfg.n)
    assert (rows == want).all(), np.unique(rows)
    assert (union == want).all(), np.unique(union)
