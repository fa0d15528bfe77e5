"""Overlapped and graph-captured execution of the whole call (the K/V gathers on a second
stream beside the route, the probe stage there beside the sparse attention; one HIP graph
per call).  Every kernel of the call is
deterministic (integer atomics only, fixed reduction orders), so both must reproduce the
eager unfused / fused outputs bit for bit.  Graph replays are interleaved with eager work
and synchronisations, each replay is checked, and a replay after the inputs are overwritten
in place must match an eager call on the new inputs."""
import numpy as np
import pytest

from sparsepr_workloads import CONFIGS, small

from gpu_harness import device_tensor, host, oracle_inputs

pytestmark = pytest.mark.gpu

CASES = {
    "c1_fp32": CONFIGS[1],
    "c3_bf16_ragged": small(CONFIGS[3], (3, 15, 24), heads_q=3, groups=16),
    "c4_bf16_gqa_ragged": small(CONFIGS[4], (2, 15, 20), heads_q=10, heads_kv=2, groups=16),
}


def _setup(cname, seed_shift=0):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import free_block_sparse_sparsepr_amd as S
    cfg = CASES[cname]
    Q, K, V = oracle_inputs(cfg)
    if seed_shift:
        rng = np.random.default_rng(seed_shift)
        Q = Q[:, rng.permutation(cfg.n)]
        K = K[:, rng.permutation(cfg.n)]
    sp = S.SparsePR(S.config_from_workload(cfg))
    return cfg, sp, device_tensor(Q, cfg), device_tensor(K, cfg), device_tensor(V, cfg)


@pytest.mark.parametrize("cname", sorted(CASES))
def test_deferred_kv_gather_is_bit_identical(cname):
    """A partition that leaves the K/V gathers to gather_kv (the key centroids then read K
    through the permutation, in the same order) gives the same buffers bit for bit."""
    import torch
    print(f"\n[deferred gathers {cname}]", flush=True)
    cfg, sp, q, k, v = _setup(cname)
    sp.partition(q, k, v)
    torch.cuda.synchronize()
    want = {n: host(t.clone()) for n, t in sp.part.items()}
    for n in ("k_gm", "v_gm", "key_centroids"):
        sp.part[n].zero_()
    sp.partition(q, k, v, defer_kv=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(sp.part["key_centroids"]), want["key_centroids"])
    sp.gather_kv(k, v)
    torch.cuda.synchronize()
    for n, t in sp.part.items():
        np.testing.assert_array_equal(host(t), want[n], err_msg=n)


def test_deferred_gathers_are_required():
    """A partition that defers the K/V gathers is refused by the entry points that read the
    gathered K and V (SPARSEPR_ERR_PARAM) until sparsepr_gather_kv has been enqueued."""
    import torch
    print("\n[deferred gathers required]", flush=True)
    cfg, sp, q, k, v = _setup("c3_bf16_ragged")
    sp.partition(q, k, v, defer_kv=True)
    sp.route()
    for name, call in (("attend", sp.attend), ("attend_apply", sp.attend_apply),
                       ("probe_fit", lambda: sp.probe_fit(q))):
        with pytest.raises(RuntimeError, match="status -6"):
            call()
    sp.gather_kv(k, v)
    sp.probe_fit(q)
    out = sp.attend_apply()
    torch.cuda.synchronize()
    want = host(sp.fused(q, k, v).clone())
    np.testing.assert_array_equal(host(out), want)


@pytest.mark.parametrize("cname", sorted(CASES))
def test_overlapped_order_matches_unfused(cname):
    import torch
    print(f"\n[overlapped {cname}]", flush=True)
    cfg, sp, q, k, v = _setup(cname)
    want = host(sp(q, k, v).clone())
    fit_want = {n: host(t.clone()) for n, t in sp.fit.items()}
    for _ in range(2):
        got = sp.overlapped(q, k, v)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(got), want)
        for n, t in sp.fit.items():
            np.testing.assert_array_equal(host(t), fit_want[n], err_msg=n)


@pytest.mark.parametrize("order", ["fused", "unfused", "overlapped"])
@pytest.mark.parametrize("cname", sorted(CASES))
def test_graph_replays_match_eager(cname, order):
    import torch
    print(f"\n[graph {cname} {order}]", flush=True)
    cfg, sp, q, k, v = _setup(cname)
    fn = {"fused": sp.fused, "unfused": sp.__call__, "overlapped": sp.overlapped}[order]
    out = torch.empty((cfg.heads_q, cfg.n, cfg.d), dtype=q.dtype, device=q.device)
    want = host(fn(q, k, v, out).clone())
    pairs = host(sp.route_buf["pairs"].clone())
    graph = sp.capture(q, k, v, out, order)
    # eager work between replays: another call shape on its own buffers and a torch op
    _, sp2, q2, k2, v2 = _setup(cname, seed_shift=5)
    for rep in range(3):
        out.zero_()
        sp.route_buf["pairs"].zero_()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(out), want, err_msg=f"replay {rep}")
        np.testing.assert_array_equal(host(sp.route_buf["pairs"]), pairs)
        other = sp2.fused(q2, k2, v2)
        (other.float() * 2).sum().item()
        torch.cuda.synchronize()
    # new input values in the same buffers: the replay must follow them
    want2 = host(sp2.fused(q2, k2, v2).clone())
    q.copy_(q2)
    k.copy_(k2)
    v.copy_(v2)
    graph.replay()
    torch.cuda.synchronize()
    if order == "fused":
        np.testing.assert_array_equal(host(out), want2)
    else:
        want2u = host(sp2(q2, k2, v2).clone())
        np.testing.assert_array_equal(host(out), want2u)


@pytest.mark.parametrize("cname", sorted(CASES))
def test_split_order_matches_overlapped_and_fused(cname):
    """The split order (the first KV heads' attention beside the probe stage, the other heads'
    attention with the fused write-back on a third stream once the fit is done): the first
    heads equal the overlapped call and the others the fused call, bit for bit, at every
    split point, eager (twice) and as graph replays with eager work between them."""
    import torch
    print(f"\n[split {cname}]", flush=True)
    cfg, sp, q, k, v = _setup(cname)
    if cfg.heads_kv < 2:
        pytest.skip("one KV head: nothing to split")
    over = host(sp.overlapped(q, k, v).clone())
    fused = host(sp.fused(q, k, v).clone())
    for first in range(1, cfg.heads_kv):
        h0 = first * cfg.g
        for _ in range(2):
            got = host(sp.split(q, k, v, first_kv=first))
            torch.cuda.synchronize()
            np.testing.assert_array_equal(got[:h0], over[:h0], err_msg=f"first heads, split {first}")
            np.testing.assert_array_equal(got[h0:], fused[h0:], err_msg=f"other heads, split {first}")
    out = torch.empty((cfg.heads_q, cfg.n, cfg.d), dtype=q.dtype, device=q.device)
    graph = sp.capture(q, k, v, out, "split")
    h0 = sp.split_point() * cfg.g
    _, sp2, q2, k2, v2 = _setup(cname, seed_shift=5)
    for rep in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        got = host(out)
        np.testing.assert_array_equal(got[:h0], over[:h0], err_msg=f"replay {rep}")
        np.testing.assert_array_equal(got[h0:], fused[h0:], err_msg=f"replay {rep}")
        (sp2.fused(q2, k2, v2).float() * 2).sum().item()
        torch.cuda.synchronize()


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "unfused"])
@pytest.mark.parametrize("cname", sorted(CASES))
def test_head_chunk_pipeline_matches_one_call(cname, fused):
    """The call split over chunks of KV heads on three streams gives the one-call output
    bit for bit (each head's arithmetic is unchanged), for every chunk count."""
    import torch
    import free_block_sparse_sparsepr_amd as S
    print(f"\n[pipelined {cname} fused={fused}]", flush=True)
    cfg, sp, q, k, v = _setup(cname)
    want = host((sp.fused(q, k, v) if fused else sp(q, k, v)).clone())
    for chunks in sorted({1, 2, cfg.heads_kv}):
        pipe = S.PipelinedSparsePR(S.config_from_workload(cfg), chunks=chunks, fused=fused)
        for _ in range(2):
            got = pipe(q, k, v)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(host(got), want, err_msg=f"chunks={chunks}")


def test_head_chunk_pipeline_graph_replays():
    """The pipelined call captured in one HIP graph (three streams joined into the capture)
    replays to the eager result, with eager work between replays."""
    import torch
    import free_block_sparse_sparsepr_amd as S
    print("\n[pipelined graph]", flush=True)
    cfg, sp, q, k, v = _setup("c3_bf16_ragged")
    want = host(sp.fused(q, k, v).clone())
    pipe = S.PipelinedSparsePR(S.config_from_workload(cfg), chunks=2, fused=True)
    out = torch.empty_like(q)
    graph = pipe.capture(q, k, v, out)
    for rep in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(out), want, err_msg=f"replay {rep}")
        sp.fused(q, k, v)
        torch.cuda.synchronize()
