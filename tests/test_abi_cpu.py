"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every entry
point include/sparsepr.h declares, and rejects bad arguments before touching a device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparsepr.h")

B = pytest.importorskip("free_block_sparse_sparsepr_amd._binding")


def lib_or_skip():
    try:
        return B.load()
    except ImportError as e:
        pytest.skip(str(e))


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:sparsepr_status|const char\*)\s+(sparsepr_\w+)\(", text, re.M)))


def test_header_declares_the_five_calls_and_helpers():
    names = declared_functions()
    for n in ["sparsepr_partition", "sparsepr_route", "sparsepr_attend", "sparsepr_probe_fit",
              "sparsepr_apply", "sparsepr_workspace_size", "sparsepr_dense_attention",
              "sparsepr_status_string"]:
        assert n in names
    assert sorted(B.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    lib = lib_or_skip()
    for n in declared_functions():
        assert hasattr(lib, n), n


def _params(**kw):
    base = dict(heads_q=4, heads_kv=2, n=4096, d=128, dtype=B.BF16, groups_q=64, groups_k=64, r_k=48,
                r_q=64, n_probe=64, rank=16, lam=0.1, rho_exec=0.22, block=64, kmeans_iters=10,
                softmax_scale=0.0)
    base.update(kw)
    return B.Params(**base)


def _ws(p):
    lib = lib_or_skip()
    out = ctypes.c_size_t(0)
    return lib.sparsepr_workspace_size(ctypes.byref(p), ctypes.byref(out)), out.value


def test_workspace_size_valid():
    st, n = _ws(_params())
    assert st == 0 and n > 0


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), -2), (dict(n=0), -2), (dict(n=(1 << 22) + 1), -2), (dict(heads_q=3), -2),
    (dict(heads_q=34, heads_kv=2), -2), (dict(groups_q=65), -2), (dict(groups_k=0), -2),
    (dict(n=32, groups_q=33, n_probe=16, rho_exec=0.9), -2), (dict(dtype=7), -3),
    (dict(groups_k=64, r_q=32), -6), (dict(r_k=65), -6), (dict(n_probe=65), -6),
    (dict(n=60, groups_q=8, groups_k=8, n_probe=61, rank=4), -6), (dict(rank=33), -6),
    (dict(rank=17, n_probe=16), -6), (dict(lam=0.0), -6), (dict(lam=float("nan")), -6),
    (dict(rho_exec=1.5), -6), (dict(rho_exec=0.01, n=4096), -6), (dict(kmeans_iters=-1), -6),
    (dict(block=32), -6), (dict(softmax_scale=-1.0), -6), (dict(ablation=3), -6), (dict(ablation=-1), -6),
    (dict(probe_mode=3), -6), (dict(partition_mode=2), -6), (dict(budget_mode=2), -6), (dict(cost_mode=-1), -6),
])
def test_invalid_params_rejected(kw, code):
    st, _ = _ws(_params(**kw))
    assert st == code


@pytest.mark.parametrize("ablation", [B.ABLATE_NONE, B.ABLATE_HARD_DROP, B.ABLATE_RIDGE_ONLY])
@pytest.mark.parametrize("probe_mode", [B.PROBES_RADIAL, B.PROBES_UNIFORM, B.PROBES_GIVEN])
@pytest.mark.parametrize("partition_mode", [B.PARTITION_RESPONSE, B.PARTITION_SEMANTIC])
def test_ablation_switches_accepted(ablation, probe_mode, partition_mode):
    st, n = _ws(_params(ablation=ablation, probe_mode=probe_mode, partition_mode=partition_mode))
    assert st == 0 and n > 0


def test_entry_points_reject_before_any_launch():
    lib = lib_or_skip()
    bad = _params(d=96)
    good = _params()
    part, route, fit = B.PartitionT(), B.RouteT(), B.FitT()
    nul = ctypes.c_void_p(0)
    # invalid params
    assert lib.sparsepr_partition(ctypes.byref(bad), nul, nul, nul, ctypes.byref(part), nul, 0, nul) == -2
    # null inputs / outputs
    assert lib.sparsepr_partition(ctypes.byref(good), nul, nul, nul, ctypes.byref(part), nul, 0, nul) == -1
    assert lib.sparsepr_route(ctypes.byref(good), ctypes.byref(part), ctypes.byref(route), nul, 0, nul) == -1
    assert lib.sparsepr_attend(ctypes.byref(good), ctypes.byref(part), ctypes.byref(route), nul, nul, nul, 0,
                               nul) == -1
    assert lib.sparsepr_probe_fit(ctypes.byref(good), nul, ctypes.byref(part), ctypes.byref(route),
                                  ctypes.byref(fit), nul, 0, nul) == -1
    assert lib.sparsepr_apply(ctypes.byref(good), nul, ctypes.byref(part), ctypes.byref(fit), nul, nul) == -1
    assert lib.sparsepr_dense_attention(ctypes.byref(good), nul, nul, nul, nul, nul, 0, nul) == -1
    # misaligned pointer, and a workspace that is too small (fake non-null pointers are
    # never dereferenced: validation fails first)
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1008)
    fields = {f: 0x2000 for f in B.PARTITION_FIELDS}
    full = B.PartitionT(**fields)
    assert lib.sparsepr_partition(ctypes.byref(good), odd, fake, fake, ctypes.byref(full), fake, 1 << 40,
                                  nul) == -4
    assert lib.sparsepr_partition(ctypes.byref(good), fake, fake, fake, ctypes.byref(full), fake, 16,
                                  nul) == -5
    assert lib.sparsepr_status_string(-5) == b"workspace too small"
    # attend and attend_apply keep their tile schedule in the workspace: a missing or short
    # one is rejected before anything is launched
    rfields = {f: 0x2000 for f in B.ROUTE_FIELDS}
    froute = B.RouteT(**rfields)
    ffit = B.FitT(**{f: 0x2000 for f in B.FIT_FIELDS})
    assert lib.sparsepr_attend(ctypes.byref(good), ctypes.byref(full), ctypes.byref(froute), fake, fake, nul, 0,
                               nul) == -1
    assert lib.sparsepr_attend(ctypes.byref(good), ctypes.byref(full), ctypes.byref(froute), fake, fake, fake, 16,
                               nul) == -5
    assert lib.sparsepr_attend_apply(ctypes.byref(good), ctypes.byref(full), ctypes.byref(froute),
                                     ctypes.byref(ffit), fake, fake, 16, nul) == -5
    need = ctypes.c_size_t(0)
    assert lib.sparsepr_workspace_size(ctypes.byref(good), ctypes.byref(need)) == 0
    assert lib.sparsepr_attend(ctypes.byref(good), ctypes.byref(full), ctypes.byref(froute), fake, fake, odd,
                               need.value, nul) == -4


def test_support_diagnostics_validation():
    """Set sizes 1..16, n_sets >= 0 and 0 < mass <= 1 are checked on the host; zero sets is a
    no-op that touches no pointer."""
    lib = lib_or_skip()
    p = _params()
    out = ctypes.c_size_t(0)
    assert lib.sparsepr_support_workspace_size(ctypes.byref(p), 8, 8, ctypes.byref(out)) == 0
    assert out.value == 4 * 8 * 8 * p.n * 4          # 32 items, each 8 rows of n fp32 scores
    assert lib.sparsepr_support_workspace_size(ctypes.byref(p), 1000, 8, ctypes.byref(out)) == 0
    assert out.value == 512 * 8 * p.n * 4            # at most 512 concurrent items
    for n_sets, s in [(-1, 8), (4, 0), (4, 17)]:
        assert lib.sparsepr_support_workspace_size(ctypes.byref(p), n_sets, s, ctypes.byref(out)) == -6
    nul = ctypes.c_void_p(0)
    assert lib.sparsepr_support_diagnostics(ctypes.byref(p), nul, nul, nul, 0, 8, 0.9, nul, nul, nul, 0, nul) == 0
    assert lib.sparsepr_support_diagnostics(ctypes.byref(p), nul, nul, nul, 4, 8, 0.9, nul, nul, nul, 0, nul) == -1
    for mass in (0.0, 1.5, float("nan")):
        assert lib.sparsepr_support_diagnostics(ctypes.byref(p), nul, nul, nul, 4, 8, mass, nul, nul, nul, 0,
                                                nul) == -6
    fake = ctypes.c_void_p(0x1000)
    assert lib.sparsepr_support_diagnostics(ctypes.byref(p), fake, fake, fake, 4, 8, 0.9, fake, fake, fake, 16,
                                            nul) == -5


def test_global_budget_route_needs_its_workspace():
    """The shared budget keeps per-head sorted cells in the workspace; the per-head route
    needs none."""
    lib = lib_or_skip()
    _, n0 = _ws(_params(groups_q=64, groups_k=64, n=1 << 20))
    st, n1 = _ws(_params(groups_q=64, groups_k=64, n=1 << 20, budget_mode=B.BUDGET_GLOBAL))
    assert st == 0 and n1 >= n0
    nul = ctypes.c_void_p(0)
    fields = {f: 0x2000 for f in B.PARTITION_FIELDS}
    part = B.PartitionT(**fields)
    route = B.RouteT(**{f: 0x3000 for f in B.ROUTE_FIELDS})
    g = _params(budget_mode=B.BUDGET_GLOBAL, cost_mode=B.COST_TILES)
    assert lib.sparsepr_route(ctypes.byref(g), ctypes.byref(part), ctypes.byref(route), nul, 0, nul) == -1
    assert lib.sparsepr_route(ctypes.byref(g), ctypes.byref(part), ctypes.byref(route), ctypes.c_void_p(0x1000), 16,
                              nul) == -5


def test_noalloc_attend_rejects_before_any_launch():
    """The allocation-free attention takes no workspace: it checks its pointers and rejects a
    schedule larger than its fixed device array before it looks anything up or launches."""
    lib = lib_or_skip()
    nul = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1008)
    part = B.PartitionT(**{f: 0x2000 for f in B.PARTITION_FIELDS})
    route = B.RouteT(**{f: 0x3000 for f in B.ROUTE_FIELDS})
    good = _params()
    assert lib.sparsepr_attend_noalloc(ctypes.byref(_params(d=96)), ctypes.byref(part), ctypes.byref(route), fake,
                                       fake, nul) == -2
    assert lib.sparsepr_attend_noalloc(ctypes.byref(good), ctypes.byref(part), ctypes.byref(route), nul, fake,
                                       nul) == -1
    assert lib.sparsepr_attend_noalloc(ctypes.byref(good), ctypes.byref(part), ctypes.byref(route), odd, fake,
                                       nul) == -4
    # 16 query heads on each of 8 KV heads at the largest n: the schedule needs
    # 4 (2 (2^22 16 / 256 + 64) 8 + 64 + 8) bytes, more than the 4 MiB array
    big = _params(heads_q=128, heads_kv=8, n=1 << 22)
    assert 4 * (2 * ((1 << 22) * 16 // 256 + 64) * 8 + 64 + 8) > 4 << 20
    assert lib.sparsepr_attend_noalloc(ctypes.byref(big), ctypes.byref(part), ctypes.byref(route), fake, fake,
                                       nul) == -5
