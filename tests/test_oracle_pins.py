"""Pins of the CPU oracle against facts fixed outside it: library routines, closed forms,
invariants stated on the pages, and brute force on tiny inputs.  CPU only."""
import decimal
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

from oracle import diagnostics as Dg
from oracle import sparsepr as O

RNG = np.random.default_rng(1234)


def rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


# ----------------------------------------------------------------------------- dense
def test_dense_attention_matches_library_softmax():
    q, k, v = rand(7, 5), rand(11, 5), rand(11, 3)
    s = q @ k.T * 0.37
    o, lse = O.dense_attention(q, k, v, 0.37, chunk=3)
    np.testing.assert_allclose(o, softmax(s, axis=1) @ v, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, logsumexp(s, axis=1), rtol=1e-13)


def test_dense_attention_identical_keys_gives_mean_of_values():
    q = rand(4, 6)
    k = np.repeat(rand(1, 6), 9, axis=0)
    v = rand(9, 2)
    o, _ = O.dense_attention(q, k, v, 1.0)
    np.testing.assert_allclose(o, np.repeat(v.mean(0, keepdims=True), 4, 0), atol=1e-14)


# ----------------------------------------------------------------------------- sparse
def _tiny_partition(n=40, gq=3, gk=4):
    ql = RNG.integers(0, gq, n)
    kl = RNG.integers(0, gk, n)
    return ql, kl


def test_sparse_all_cells_equals_dense():
    q, k, v = rand(40, 8), rand(40, 8), rand(40, 4)
    ql, kl = _tiny_partition()
    kept = np.ones((3, 4), bool)
    o_s, l_s = O.sparse_attention(q, k, v, 0.5, ql, kl, kept)
    o_d, l_d = O.dense_attention(q, k, v, 0.5)
    np.testing.assert_allclose(o_s, o_d, atol=1e-12)
    np.testing.assert_allclose(l_s, l_d, atol=1e-12)


def test_sparse_renormalised_over_kept_groups_and_residual_identity():
    """Hard drop + renormalisation: the residual equals the dropped mass times
    (output on the dropped support - sparse output) (PSRR hard-drop residual paragraph);
    the kept-set probabilities sum to one."""
    q, k, v = rand(40, 8), rand(40, 8), rand(40, 4)
    ql, kl = _tiny_partition()
    kept = np.array([[1, 0, 1, 0], [0, 1, 0, 0], [1, 1, 1, 0]], bool)
    o_s, l_s = O.sparse_attention(q, k, v, 0.5, ql, kl, kept)
    o_d, l_d = O.dense_attention(q, k, v, 0.5)
    p = softmax(q @ k.T * 0.5, axis=1)
    for i in range(40):
        keep = kept[ql[i]][kl]
        ps = p[i, keep] / p[i, keep].sum()
        assert abs(ps.sum() - 1) < 1e-14
        np.testing.assert_allclose(o_s[i], ps @ v[keep], atol=1e-13)
        m_drop = p[i, ~keep].sum()
        o_drop = p[i, ~keep] @ v[~keep] / m_drop
        np.testing.assert_allclose(o_d[i] - o_s[i], m_drop * (o_drop - o_s[i]), atol=1e-12)
        # exp(L_sparse - L_dense) is the kept mass
        assert abs(math.exp(l_s[i] - l_d[i]) - (1 - m_drop)) < 1e-12


def test_probe_rows_reproduce_residual_exactly():
    q, k, v = rand(40, 8), rand(40, 8), rand(40, 4)
    ql, kl = _tiny_partition()
    kept = np.array([[1, 0, 0, 0], [0, 1, 1, 0], [0, 0, 1, 1]], bool)
    toks = np.array([3, 17, 29, 30])
    od, os_, R, _, _ = O.probe_rows(q, k, v, 0.5, toks, ql, kl, kept)
    full_d, _ = O.dense_attention(q, k, v, 0.5)
    full_s, _ = O.sparse_attention(q, k, v, 0.5, ql, kl, kept)
    np.testing.assert_array_equal(R, od - os_)
    np.testing.assert_allclose(od, full_d[toks], atol=1e-14)
    np.testing.assert_allclose(os_, full_s[toks], atol=1e-14)


# ----------------------------------------------------------------------------- features
def test_div_rhaz_matches_decimal_half_up():
    for a in range(-50, 51):
        for b in range(1, 12):
            want = int(decimal.Decimal(a / 1) .__truediv__(decimal.Decimal(b))
                       .quantize(decimal.Decimal(1), rounding=decimal.ROUND_HALF_UP))
            assert int(O.div_rhaz(a, b)) == want, (a, b)


def test_pow2_exponent_is_largest():
    for m in [1e-9, 0.3, 1.0, 126.9, 127.0, 127.1, 5e6]:
        e = O.pow2_exponent(m, 127)
        assert m * 2.0 ** e <= 127 < m * 2.0 ** (e + 1)
    assert O.pow2_exponent(0.0, 127) == 0


def test_key_features_scale_invariance_and_range():
    S = rand(48, 300, scale=3.0)
    X, e = O.key_features(S)
    assert X.shape == (300, 48)
    assert 63 < np.abs(X).max() <= 127
    X2, e2 = O.key_features(4.0 * S)
    np.testing.assert_array_equal(X, X2)
    assert e2 == e - 2
    # rounding is to nearest: |X - S 2^e| <= 1/2
    assert np.abs(X.T - S * 2.0 ** e).max() <= 0.5


def test_query_features_shift_and_scale_invariance():
    U = RNG.uniform(-0.45, 0.45, (1, 50, 16))
    U[0, 0, 0] = 0.45
    x, e = O.query_features(U)
    assert e == 15
    x2, _ = O.query_features(2.0 * U)
    np.testing.assert_array_equal(x, x2)
    # an exactly representable per-row shift that keeps the head maximum's binade
    shift = (RNG.integers(-100, 100, (1, 50, 1)) * 2.0 ** -15)
    x3, e3 = O.query_features(U + shift)
    assert e3 == e
    np.testing.assert_array_equal(x, x3)
    assert np.abs(x).max(axis=1).min() == 127
    # constant rows give the zero direction
    U[0, 7] = 0.25
    assert not O.query_features(U)[0][7].any()


def test_query_features_head_sum_for_gqa():
    """Under GQA the coordinate is the float64 head sum: values whose float32 sum loses
    the small term keep it, and a supplied U_sum replaces the sum."""
    U = RNG.uniform(-1, 1, (3, 20, 8))
    x, _ = O.query_features(U)
    x1, _ = O.query_features((U[0] + U[1] + U[2])[None])
    np.testing.assert_array_equal(x, x1)
    tiny = np.zeros((3, 1, 4))
    tiny[0, 0] = [1.0, 1.0, 0.0, 0.0]
    tiny[1, 0] = [2.0 ** -30, 0.0, 0.0, 0.0]
    tiny[2, 0] = [-1.0, -1.0, 0.0, 0.0]
    np.testing.assert_array_equal(O.summed_response(tiny)[0], [2.0 ** -30, 0.0, 0.0, 0.0])
    assert np.float32(np.float32(1.0) + np.float32(2.0 ** -30)) - np.float32(1.0) == 0.0
    np.testing.assert_array_equal(O.summed_response(U[:1]), U[0])
    # the supplied sum is what gets quantised
    other = U[0] - U[1]
    np.testing.assert_array_equal(O.query_features(U, U_sum=other)[0], O.query_features(other[None])[0])


# ----------------------------------------------------------------- sampled responses
def test_sample_queries_hand_values():
    """r_K evenly strided sampled rows, token floor((2s+1) N / (2 r_K)), head s mod g
    (values worked by hand for N = 100, r_K = 4, g = 3)."""
    tok, hd = O.sample_queries(100, 4, 3)
    np.testing.assert_array_equal(tok, [12, 37, 62, 87])
    np.testing.assert_array_equal(hd, [0, 1, 2, 0])
    tok, hd = O.sample_queries(7, 3, 1)
    np.testing.assert_array_equal(tok, [1, 3, 5])
    np.testing.assert_array_equal(hd, [0, 0, 0])


def test_key_responses_decode_the_sampled_rows():
    """A planted one-hot code: query (h, t) is the unit vector e_{h N + t}, and key j answers
    head 0's token j with 1 and head 1's token j with 2, so row s of S is non-zero only at
    the sampled token, with a value that names the sampled head, times scale.  A wrong
    head cycle, stride or scale changes the decoded rows or the value."""
    scale = 1 / np.sqrt(7.0)
    g, n, r_k = 2, 12, 4
    d = g * n
    q = np.zeros((g, n, d))
    for h in range(g):
        for t in range(n):
            q[h, t, h * n + t] = 1.0
    k = np.zeros((n, d))
    for j in range(n):              # key j answers to both heads' token j
        k[j, j] = 1.0
        k[j, n + j] = 2.0
    S = O.key_responses(q, k, scale, r_k)
    # sampled tokens floor((2s+1) 12 / 8) = 1, 4, 7, 10; heads 0, 1, 0, 1
    want = np.zeros((r_k, n))
    for s, (t, h) in enumerate([(1, 0), (4, 1), (7, 0), (10, 1)]):
        want[s, t] = scale * (1.0 if h == 0 else 2.0)
    np.testing.assert_array_equal(S, want)


def test_key_responses_explicit_dot_products():
    """S[s, j] = scale * sum_c Q[h_s, t_s, c] K[j, c], written as plain loops over the
    hand-computed sampled rows of N = 9, r_K = 3, g = 2 (tokens 1, 4, 7; heads 0, 1, 0)."""
    g, n, d = 2, 9, 5
    q, k = rand(g, n, d), rand(n, d)
    scale = 0.3141
    S = O.key_responses(q, k, scale, 3)
    for s, (t, h) in enumerate([(1, 0), (4, 1), (7, 0)]):
        for j in range(n):
            acc = 0.0
            for c in range(d):
                acc += q[h, t, c] * k[j, c]
            assert abs(S[s, j] - scale * acc) < 1e-12


def test_query_responses_explicit_dot_products_and_unit_centroids():
    """U^(h)[i, b] = scale * <q^(h)_i, C^K_b>: plain loops, and unit-vector centroids pick
    the query's coordinates."""
    g, n, d, G = 2, 6, 4, 3
    q, C = rand(g, n, d), rand(G, d)
    scale = 0.777
    U = O.query_responses(q, C, scale)
    assert U.shape == (g, n, G)
    for h in range(g):
        for i in range(n):
            for b in range(G):
                acc = 0.0
                for c in range(d):
                    acc += q[h, i, c] * C[b, c]
                assert abs(U[h, i, b] - scale * acc) < 1e-12
    E = np.eye(d)[[2, 0, 3]]
    np.testing.assert_array_equal(O.query_responses(q, E, 1.0), q[:, :, [2, 0, 3]])


# ----------------------------------------------------------------------------- k-means
def _brute_kmeans(X, G, iters):
    """Lloyd's algorithm written with explicit squared Euclidean distances and exact
    rational means (Python Fractions), rounded half away from zero."""
    from fractions import Fraction
    X = [list(map(int, r)) for r in X]
    n = len(X)
    C = [list(X[(2 * g + 1) * n // (2 * G)]) for g in range(G)]

    def assign():
        lab = []
        for x in X:
            dist = [sum((xi - ci) ** 2 for xi, ci in zip(x, c)) for c in C]
            lab.append(min(range(G), key=lambda g: (dist[g], g)))
        return lab

    def rnd(fr):
        s = 1 if fr >= 0 else -1
        fr = abs(fr)
        fl = fr.numerator // fr.denominator
        return s * (fl + (1 if fr - fl >= Fraction(1, 2) else 0))

    for _ in range(iters):
        lab = assign()
        for g in range(G):
            mem = [X[j] for j in range(n) if lab[j] == g]
            if mem:
                C[g] = [rnd(Fraction(sum(col), len(mem))) for col in zip(*mem)]
    return np.array(assign()), np.array(C)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_kmeans_matches_bruteforce_lloyd(seed):
    r = np.random.default_rng(seed)
    X = r.integers(-127, 128, (90, 6))
    X[::7] = X[3]           # duplicate points -> ties and possibly empty groups
    lab, C = O.kmeans(X, 5, 4)
    blab, bC = _brute_kmeans(X, 5, 4)
    np.testing.assert_array_equal(lab, blab)
    np.testing.assert_array_equal(C, bC)


def test_kmeans_exactness_bound():
    # the largest |<x, c>| the GPU accumulates in float32 stays below 2**24
    assert 64 * 127 * 127 < 2 ** 24 and 2 * 64 * 127 * 127 + 64 * 127 * 127 < 2 ** 24 * 2


def test_group_major_is_stable_bijection():
    lab = RNG.integers(0, 5, 60)
    lab[lab == 3] = 4          # an empty group
    perm, inv, off = O.group_major(lab, 6)
    want = [i for _, i in sorted((int(l), i) for i, l in enumerate(lab))]
    np.testing.assert_array_equal(perm, want)
    np.testing.assert_array_equal(inv[perm], np.arange(60))
    assert off[0] == 0 and off[-1] == 60 and off[4] == off[3]
    for g in range(6):
        assert (lab[perm[off[g]:off[g + 1]]] == g).all()


def test_key_centroids_are_group_means():
    k = rand(30, 5)
    lab = RNG.integers(0, 4, 30)
    lab[lab == 2] = 1
    C = O.key_centroids(k, lab, 4)
    for b in range(4):
        if (lab == b).any():
            np.testing.assert_allclose((k[lab == b] - C[b]).sum(0), 0, atol=1e-13)
        else:
            assert not C[b].any()


# ----------------------------------------------------------------------------- route
def test_exp_table_matches_high_precision_exp():
    decimal.getcontext().prec = 50
    E = O.exp_table()
    for kk in range(1024):
        x = decimal.Decimal(2 ** 20) * (decimal.Decimal(-kk) / decimal.Decimal(64)).exp()
        want = int(x.quantize(decimal.Decimal(1), rounding=decimal.ROUND_HALF_EVEN))
        assert E[kk] == want, kk
    assert E[0] == 2 ** 20 and E[931] == 1 and E[932] == 0


def test_row_masses_approximate_size_weighted_centroid_softmax():
    U = rand(25, 16, scale=2.0)
    counts = RNG.integers(1, 300, 16)
    counts[5] = 0
    P = O.row_masses(U, counts)
    w = counts * np.exp(U - U.max(1, keepdims=True))
    w[:, 5] = 0
    ref = w / w.sum(1, keepdims=True)
    # 1/64-logit rounding and a 2^20 table: within ~2 % relative (+ fixed-point floor)
    assert np.all(np.abs(P / 2 ** 20 - ref) <= 0.02 * ref + 2e-6)
    tot = P.sum(1)
    assert np.all(tot <= 2 ** 20) and np.all(tot > 2 ** 20 - 16)
    assert not P[:, 5].any()


def test_block_mass_sums_over_group_rows_and_heads():
    U = rand(2, 30, 4)
    ql = RNG.integers(0, 3, 30)
    kc = np.array([5, 0, 7, 9])
    m = O.block_mass(U, ql, kc, 3)
    want = np.zeros((3, 4), np.int64)
    for h in range(2):
        P = O.row_masses(U[h], kc)
        for i in range(30):
            want[ql[i]] += P[i]
    np.testing.assert_array_equal(m, want)
    assert not m[:, 1].any()


def _check_selection(r, m, qc, kc, budget):
    cost = np.outer(qc, kc)
    # mandatory: each non-empty query group keeps its heaviest key group
    for a in range(len(qc)):
        if qc[a]:
            b = max((b for b in range(len(kc)) if kc[b]), key=lambda b: (m[a, b], -b))
            assert r.mandatory[a, b] and r.kept[a, b]
        else:
            assert not r.kept[a].any()
    left = budget - cost[r.mandatory].sum()
    opt = r.kept & ~r.mandatory
    assert cost[opt].sum() <= max(left, 0) or not opt.any()
    kap = {}
    for a, b in itertools.product(range(len(qc)), range(len(kc))):
        if cost[a, b] and not r.mandatory[a, b]:
            # mass per pair compared by cross-multiplication (exact)
            kap[(a, b)] = (MassPerPair(int(m[a, b]), int(cost[a, b])), -(a * len(kc) + b))
    kept_keys = [kap[c] for c in kap if r.kept[c]]
    drop_keys = [kap[c] for c in kap if not r.kept[c]]
    if kept_keys and drop_keys:
        assert min(kept_keys) > max(drop_keys)       # a prefix of the ranking
    if drop_keys:
        first = max(drop_keys)
        cell = [c for c in kap if kap[c] == first][0]
        assert cost[opt].sum() + cost[cell] > left   # maximal prefix


class MassPerPair:
    def __init__(self, m, c):
        self.m, self.c = m, c

    def __lt__(self, o):
        return self.m * o.c < o.m * self.c

    def __eq__(self, o):
        return self.m * o.c == o.m * self.c


@pytest.mark.parametrize("rho", [0.05, 0.22, 0.5, 0.9])
def test_select_cells_invariants(rho):
    n = 500
    qc = np.bincount(RNG.integers(0, 6, n), minlength=7)
    kc = np.bincount(RNG.integers(0, 5, n), minlength=5)
    m = RNG.integers(0, 10 ** 9, (7, 5))
    r = O.select_cells(m, qc, kc, rho, n, 8)
    _check_selection(r, m, qc, kc, r.budget)
    assert r.pairs == int(np.outer(qc, kc)[r.kept].sum())
    assert r.row_ptr[-1] == r.cols.size
    for a in range(7):
        cols = r.cols[r.row_ptr[a]:r.row_ptr[a + 1]]
        assert list(cols) == sorted(cols) and all(r.kept[a, cols])


def test_select_cells_full_density_keeps_everything():
    n = 300
    qc = np.bincount(RNG.integers(0, 4, n), minlength=4)
    kc = np.bincount(RNG.integers(0, 4, n), minlength=4)
    r = O.select_cells(RNG.integers(0, 99, (4, 4)), qc, kc, 1.0, n, 0)
    assert r.pairs == n * n and r.kept[np.outer(qc, kc) > 0].all()


def test_route_budget_accounting():
    """rho_exec = rho_route + M/N with the probe cost subtracted first (PSRR execution
    paragraph)."""
    for n, rho in [(118800, 0.22), (75600, 0.22), (43200, 0.26), (1024, 0.25)]:
        B = O.route_budget(rho, n, 64)
        assert abs((B + 64 * n) / n ** 2 - rho) < 1e-6
    assert O.route_budget(0.22, 118800, 64) == 3_097_353_600


# ----------------------------------------------------------------------------- probes
def test_probe_allocation_equal_with_remainder_to_larger_groups():
    qc = np.array([10, 0, 3, 50, 50, 1, 20])
    m = O.probe_allocation(qc, 20)
    assert m.sum() == 20 and np.all(m <= qc) and m[1] == 0 and m[5] == 1
    un = [a for a in range(7) if qc[a] > m[a]]
    assert max(m[un]) - min(m[un]) <= 1
    for a, b in itertools.product(un, un):
        if qc[a] > qc[b]:
            assert m[a] >= m[b]
    # 64 probes over 64 large groups: one each
    assert (O.probe_allocation(np.full(64, 100), 64) == 1).all()
    with pytest.raises(ValueError):
        O.probe_allocation(np.array([2, 3]), 6)


def test_select_probes_bruteforce_radial_ranks():
    n, F, G = 120, 5, 4
    x = RNG.integers(-3, 4, (n, F))          # small range -> many radius ties
    lab = RNG.integers(0, G, n)
    C = RNG.integers(-2, 3, (G, F))
    qc = np.bincount(lab, minlength=G)
    pr = O.select_probes(x, lab, C, qc, 10)
    got = {}
    for t, g in zip(pr.tokens, pr.groups):
        got.setdefault(int(g), []).append(int(t))
    for a in range(G):
        mem = sorted(((int(((x[i] - C[a]) ** 2).sum()), i) for i in range(n) if lab[i] == a))
        ma = pr.alloc[a]
        want = [mem[(2 * kk + 1) * len(mem) // (2 * ma)][1] for kk in range(ma)]
        assert got.get(a, []) == want
    assert abs(pr.weights.sum() - 10) < 1e-12
    assert (pr.weights > 0).all()


# ----------------------------------------------------------------------------- fit
def _fit_data(M=20, d=6):
    X = rand(M, d)
    Y = 0.3 * X @ rand(d, d) + 0.05 * rand(M, d)
    w = RNG.uniform(0.2, 3.0, M)
    return X, Y, w * M / w.sum()


def test_ridge_normal_equations_and_primal_form():
    X, Y, w = _fit_data()
    W, xbar, ybar, _, _ = O.ridge_fit(X, Y, w, 0.1)
    Xc, Yc = X - xbar, Y - ybar
    lhs = (Xc.T * w) @ Xc @ W + 0.1 * W
    rhs = (Xc.T * w) @ Yc
    assert np.abs(lhs - rhs).max() <= 1e-10 * np.abs(rhs).max()
    # weighted means make the weighted residual of the affine fit zero
    res = Y - (ybar + (X - xbar) @ W)
    np.testing.assert_allclose(w @ res, 0, atol=1e-12)
    # intercept is unpenalised: the weighted mean of X maps to the weighted mean of Y
    np.testing.assert_allclose(xbar, (w @ X) / w.sum())


def test_ridge_reduces_to_least_squares():
    X, Y, _ = _fit_data(M=40, d=5)
    w = np.ones(40)
    # lambda -> 0: the ridge solution approaches ordinary least squares with an
    # intercept (the dual M x M system has condition ~ 1/lambda, hence the tolerance)
    W, xbar, ybar, _, _ = O.ridge_fit(X, Y, w, 1e-8)
    Xa = np.hstack([X, np.ones((40, 1))])
    sol = np.linalg.lstsq(Xa, Y, rcond=None)[0]
    np.testing.assert_allclose(W, sol[:5], atol=1e-6)
    np.testing.assert_allclose(ybar - xbar @ W, sol[5], atol=1e-6)


def test_output_subspace_matches_svd_and_is_a_projector():
    _, Y, w = _fit_data(M=30, d=24)
    Y = Y + 0.2 * rand(30, 24)
    _, _, _, _, Yt = O.ridge_fit(rand(30, 24), Y, w, 0.1)
    V, eig = O.output_subspace(Yt, 4)
    assert V.shape == (24, 4)
    np.testing.assert_allclose(V.T @ V, np.eye(4), atol=1e-12)
    P = V @ V.T
    np.testing.assert_allclose(P, P.T, atol=1e-13)
    np.testing.assert_allclose(P @ P, P, atol=1e-12)
    _, sv, vt = np.linalg.svd(Yt)
    np.testing.assert_allclose(P, vt[:4].T @ vt[:4], atol=1e-10)
    np.testing.assert_allclose(eig[:5], sv[:5] ** 2, rtol=1e-10)


def test_projection_is_noop_when_residual_rank_within_r():
    M, d = 20, 10
    X = rand(M, d)
    Y = rand(M, 3) @ rand(3, d)           # residuals of rank 3 (<= r)
    w = np.ones(M)
    W, xbar, ybar, Xt, Yt = O.ridge_fit(X, Y, w, 0.1)
    V, _ = O.output_subspace(Yt, 16)
    assert V.shape[1] <= 3 + 1
    np.testing.assert_allclose(W @ V @ V.T, W, atol=1e-10)


def test_apply_full_route_is_dense_and_probe_rows_exact():
    """With every cell kept the residual is zero, the fit is zero and the corrected
    output is dense attention."""
    n, d = 64, 8
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    p = O.Params(groups_q=4, groups_k=4, rho_exec=1.0, n_probe=8, rank=4)
    part = O.partition(q[None], k, p)
    kept = np.ones((4, 4), bool)
    rt = O.Route(kept, kept, None, None, n * n, n * n, None)
    res = O.sparsepr_kv_head(q[None], k, v, p, part=part, route_=rt)
    od, _ = O.dense_attention(q, k, v, p.softmax_scale(d))
    np.testing.assert_allclose(res.o[0], od, atol=1e-12)


def test_apply_correction_lies_in_mean_plus_subspace():
    n, d = 96, 8
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    p = O.Params(groups_q=4, groups_k=4, rho_exec=0.4, n_probe=16, rank=3)
    res = O.sparsepr_kv_head(q[None], k, v, p)
    fit = res.fits[0]
    os_, _ = O.sparse_attention(q, k, v, p.softmax_scale(d), res.part.q_labels,
                                res.part.k_labels, res.route.kept)
    delta = res.o[0] - os_ - fit.ybar
    nonprobe = np.setdiff1d(np.arange(n), res.probes.tokens)
    P = fit.V @ fit.V.T
    np.testing.assert_allclose(delta[nonprobe] @ P, delta[nonprobe], atol=1e-12)
    od, _ = O.dense_attention(q, k, v, p.softmax_scale(d))
    np.testing.assert_allclose(res.o[0][res.probes.tokens], od[res.probes.tokens], atol=1e-13)


def test_weighted_ridge_matches_scikit_learn():
    """Library pin: weighted ridge with an unpenalised intercept is sklearn's Ridge with
    sample weights (objective sum_i w_i ||y_i - b - x_i W||^2 + lambda ||W||_F^2)."""
    from sklearn.linear_model import Ridge
    X, Y, w = _fit_data(M=64, d=16)
    W, xbar, ybar, _, _ = O.ridge_fit(X, Y, w, 0.1)
    sk = Ridge(alpha=0.1, fit_intercept=True, solver="cholesky").fit(X, Y, sample_weight=w)
    np.testing.assert_allclose(W, sk.coef_.T, atol=1e-10)
    np.testing.assert_allclose(ybar - xbar @ W, sk.intercept_, atol=1e-10)
    # M < d (the dual form's regime, as at d = 128 with 64 probes)
    X, Y, w = _fit_data(M=12, d=30)
    W, xbar, ybar, _, _ = O.ridge_fit(X, Y, w, 0.1)
    sk = Ridge(alpha=0.1, fit_intercept=True, solver="svd").fit(X, Y, sample_weight=w)
    np.testing.assert_allclose(W, sk.coef_.T, atol=1e-9)


def test_fit_and_apply_recover_a_planted_affine_residual():
    """When the residual really is an affine function of the sparse output with rank
    <= r, the probe fit recovers it for every row (up to ridge shrinkage)."""
    n, d, M = 400, 32, 64
    o_s = rand(n, d, scale=0.5)
    W0 = rand(d, 4) @ rand(4, d) * 0.2
    b0 = rand(d) * 0.1
    R_all = o_s @ W0 + b0
    toks = np.sort(RNG.choice(n, M, replace=False))
    w = np.ones(M)
    W, xbar, ybar, Xt, Yt = O.ridge_fit(o_s[toks], R_all[toks], w, 1e-6)
    V, _ = O.output_subspace(Yt, 16)
    A, B = W @ V, V.T
    fit = O.Fit(A, B, ybar - xbar @ A @ B, W, xbar, ybar, V, None,
                o_s[toks] + R_all[toks], o_s[toks], R_all[toks])
    out = O.apply_correction(o_s, fit, toks)
    np.testing.assert_allclose(out, o_s + R_all, atol=1e-5)


# ----------------------------------------------------------------------------- ablations
def test_hard_drop_is_the_renormalised_sparse_output_and_dense_on_full_route():
    q, k, v = rand(40, 8), rand(40, 8), rand(40, 4)
    ql, kl = _tiny_partition()
    kept = np.array([[1, 0, 1, 0], [0, 1, 0, 0], [1, 1, 1, 0]], bool)
    p = softmax(q @ k.T * 0.5, axis=1)
    got = O.hard_drop_rows(q, k, v, 0.5, ql, kl, kept)
    for i in range(40):
        keep = kept[ql[i]][kl]
        np.testing.assert_allclose(got[i], p[i, keep] @ v[keep] / p[i, keep].sum(), atol=1e-13)
    full = O.hard_drop_rows(q, k, v, 0.5, ql, kl, np.ones((3, 4), bool))
    np.testing.assert_allclose(full, softmax(q @ k.T * 0.5, axis=1) @ v, atol=1e-13)


@pytest.mark.parametrize("n,m", [(118800, 64), (1000, 64), (64, 64), (100, 7)])
def test_uniform_probes_are_evenly_spaced_and_unit_weight(n, m):
    labels = RNG.integers(0, 5, n)
    pr = O.uniform_probes(n, labels, m)
    t = pr.tokens
    assert t.size == m and np.all(np.diff(t) > 0) and t[0] >= 0 and t[-1] < n
    gaps = np.diff(t)
    assert gaps.min() >= n // m - 1 and gaps.max() <= -(-n // m) + 1
    # symmetric about the middle of the clip: t_k + t_{M-1-k} is n - 1 or n - 2 ... n
    s = t + t[::-1]
    assert np.all(np.abs(s - (n - 1)) <= 1)
    # the first probe sits half a spacing in
    assert abs(t[0] - n / (2 * m)) <= 1
    np.testing.assert_array_equal(pr.groups, labels[t])
    np.testing.assert_array_equal(pr.weights, np.ones(m))


def test_ridge_only_factors_the_weighted_ridge_map():
    """A B of the ridge-only fit is the weighted ridge map that scikit-learn pins above;
    the correction ybar + (o - xbar) W is written as o A B + c0."""
    n, d, M = 120, 12, 16
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    ql, kl = RNG.integers(0, 3, n), RNG.integers(0, 4, n)
    kept = np.array([[1, 0, 1, 0], [0, 1, 0, 1], [1, 1, 0, 0]], bool)
    toks = np.sort(RNG.choice(n, M, replace=False))
    pr = O.given_probes(toks, ql)
    p = O.Params(groups_q=3, groups_k=4, rho_exec=0.5, n_probe=M, rank=4, lam=0.1)
    fit = O.ridge_only_fit(q, k, v, 0.3, pr, ql, kl, kept, p)
    W, xbar, ybar, _, _ = O.ridge_fit(fit.o_sparse, fit.R, pr.weights, 0.1)
    np.testing.assert_allclose(fit.A @ fit.B, W, atol=1e-12)
    o = rand(5, d)
    np.testing.assert_allclose(O.correct_rows(o, fit), o + ybar + (o - xbar) @ W, atol=1e-12)


def test_ridge_only_with_vanishing_lambda_interpolates_the_probe_residuals():
    """With M < d and lambda -> 0 the unprojected ridge map interpolates: every probe row's
    corrected sparse output equals its exact dense output (least squares with more unknowns
    than equations); the rank-r projected fit does not when R has rank > r."""
    n, d, M = 200, 24, 12
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    ql, kl = RNG.integers(0, 3, n), RNG.integers(0, 4, n)
    kept = np.array([[1, 0, 0, 0], [0, 1, 0, 0], [0, 0, 1, 0]], bool)
    pr = O.given_probes(np.sort(RNG.choice(n, M, replace=False)), ql)
    p = O.Params(groups_q=3, groups_k=4, rho_exec=0.5, n_probe=M, rank=2, lam=1e-9)
    fit = O.ridge_only_fit(q, k, v, 0.3, pr, ql, kl, kept, p)
    np.testing.assert_allclose(O.correct_rows(fit.o_sparse, fit), fit.o_dense, atol=1e-6)
    proj = O.probe_fit(q, k, v, 0.3, pr, ql, kl, kept, p)
    assert np.abs(O.correct_rows(proj.o_sparse, proj) - proj.o_dense).max() > 1e-3


def test_semantic_features_quantise_raw_rows_and_recover_planted_clusters():
    """Semantic partition: features are the raw rows on one power-of-two scale (invariant
    to scaling the activations by a power of two); planted, well separated clusters of
    raw keys and queries are recovered exactly."""
    n, d, G = 256, 16, 4
    centres = rand(G, d, scale=4.0)
    truth = np.repeat(np.arange(G), n // G)
    k = centres[truth] + 0.05 * rand(n, d)
    x, e = O.semantic_features(k[None])
    assert np.abs(x).max() <= 127 and np.abs(x).max() >= 64
    x2, e2 = O.semantic_features(4.0 * k[None])
    np.testing.assert_array_equal(x2, x)
    assert e2 == e - 2
    q = centres[truth[::-1]] + 0.05 * rand(n, d)
    p = O.Params(groups_q=G, groups_k=G, rho_exec=0.5, n_probe=8, rank=2)
    part = O.partition_semantic(np.stack([q, q]), k, p)
    # every planted cluster is one group (labels are a relabelling of the truth)
    for lab, tr in ((part.k_labels, truth), (part.q_labels, truth[::-1])):
        pairs = set(zip(lab.tolist(), tr.tolist()))
        assert len(pairs) == G and len({a for a, _ in pairs}) == G
    # the GQA query coordinate is the float64 head sum; a supplied sum replaces it
    xq, _ = O.semantic_features(np.stack([q, 0.5 * q]))
    xs, _ = O.semantic_features((1.5 * q)[None])
    np.testing.assert_array_equal(xq, xs)
    np.testing.assert_array_equal(O.semantic_features(np.stack([q, 0.5 * q]), x_sum=-q)[0],
                                  O.semantic_features(-q[None])[0])


def test_affine_residual_stats_pins():
    """Explainable fraction = scikit-learn's variance-weighted R^2 of a linear regression of
    R on the sparse output; 1 for an exactly affine residual; orthogonal energy = the
    least-squares residual energy."""
    from sklearn.linear_model import LinearRegression
    from sklearn.metrics import r2_score
    from oracle import diagnostics as D
    n, d = 500, 8
    o_s = rand(n, d)
    R = 0.3 * o_s @ rand(d, d) + 0.1 * rand(n, d) + 0.2
    tot, cen, orth, frac = D.affine_residual_stats(o_s, o_s + R)
    lr = LinearRegression().fit(o_s, R)
    assert abs(frac - r2_score(R, lr.predict(o_s), multioutput="variance_weighted")) < 1e-12
    assert abs(orth - ((R - lr.predict(o_s)) ** 2).sum()) < 1e-9 * orth
    assert abs(tot - (R * R).sum()) < 1e-9 * tot and cen <= tot
    W0, c0 = rand(d, d), rand(d)
    _, _, orth1, frac1 = D.affine_residual_stats(o_s, o_s + (o_s @ W0 + c0))
    assert frac1 > 1 - 1e-12 and orth1 < 1e-18 * n * d


# ----------------------------------------------------------------------------- support diagnostics
def test_row_support_brute_force_over_subsets():
    """The single-row support count is the size of the smallest key subset reaching the mass
    (every subset enumerated), and the chosen members form such a subset."""
    from oracle import diagnostics as D
    n = 10
    for trial in range(6):
        q, k = rand(3, 4), rand(n, 4, scale=1.5)
        for mass in (0.5, 0.9, 0.99):
            count, member = D.row_supports(q, k, 0.8, np.arange(3), mass)
            p = softmax(q @ k.T * 0.8, axis=1)
            for r in range(3):
                best = min(len(c) for m in range(1, n + 1) for c in itertools.combinations(range(n), m)
                           if p[r, list(c)].sum() >= mass)
                assert count[r] == best == member[r].sum()
                assert p[r, member[r]].sum() >= mass


def test_row_support_closed_forms():
    """Identical keys: every probability is 1/N, the count is ceil(mass N) and the ties go to
    the lowest key indices.  Two levels (a keys e^delta times likelier than the other b):
    the count follows from the mass arithmetic by hand."""
    from oracle import diagnostics as D
    n = 1001
    k = np.repeat(rand(1, 6), n, axis=0)
    count, member = D.row_supports(rand(5, 6), k, 1.0, np.arange(5), 0.9)
    assert (count == math.ceil(0.9 * n)).all()
    assert member[:, :901].all() and not member[:, 901:].any()
    _, union = D.shared_supports(rand(8, 6), k, 1.0, np.arange(8).reshape(2, 4), 0.9)
    assert (union == 901).all()
    a, b, delta = 7, 300, 4.0
    k = np.zeros((a + b, 2))
    k[RNG.choice(a + b, a, replace=False), 0] = delta
    q = np.array([[1.0, 0.0]])
    w = math.exp(delta)
    total = a * w + b
    count, _ = D.row_supports(q, k, 1.0, [0], 0.9)
    want = math.ceil(0.9 * total / w) if a * w >= 0.9 * total else a + math.ceil(0.9 * total - a * w)
    assert count[0] == want


def test_shared_support_dominant_keys_and_bounds():
    """A row whose key j scores far above the rest needs that one key; a route shared by rows
    with distinct dominant keys keeps one key per distinct dominant key.  For any set the
    union lies between the largest single-row count and the sum of them, and a set of one
    repeated row keeps exactly that row's support."""
    from oracle import diagnostics as D
    n, d = 64, 16
    k = rand(n, d) * 0.1
    k[:d] += 40 * np.eye(d)
    q = np.eye(d)
    sets = np.array([[0, 1, 2, 3, 4, 5, 6, 7], [3, 3, 3, 9, 9, 11, 3, 9]])
    count, union = D.shared_supports(q, k, 1.0, sets, 0.9)
    assert (count == 1).all()
    assert list(union) == [8, 3]
    q, k = rand(40, 8), rand(300, 8)
    sets = RNG.integers(0, 40, (12, 8))
    count, union = D.shared_supports(q, k, 0.5, sets, 0.9)
    assert (union >= count.max(axis=1)).all() and (union <= count.sum(axis=1)).all()
    c1, u1 = D.shared_supports(q, k, 0.5, np.full((1, 8), 5), 0.9)
    assert u1[0] == c1[0, 0]


# ----------------------------------------------------------------------------- budget variants
def test_tile_padded_costs_and_ranking_by_hand():
    """Tile-padded cost: ceil(n/64)*64 per side, empty groups free.  Worked by hand: one
    query group of 64 rows, key groups of 10, 64 and 70 keys with masses 100, 500, 600 and a
    budget of 9000 pairs.  Unpadded: the mandatory cell is b=2 (4480 pairs), then b=0
    (ratio 100/640) fits and b=1 (4096) does not.  Padded: b=2 costs 8192, b=1 now ranks
    first (500/4096 > 100/4096) and does not fit in the 808 left, so the prefix stops."""
    np.testing.assert_array_equal(O.cell_costs([65, 64, 0], [1, 128], tile=64),
                                  [[128 * 64, 128 * 128], [64 * 64, 64 * 128], [0, 0]])
    np.testing.assert_array_equal(O.cell_costs([65, 3], [7], tile=0), [[455], [21]])
    m = np.array([[100, 500, 600]])
    assert O.route_budget(0.009, 1000, 0) == 9000
    r0 = O.select_cells(m, [64], [10, 64, 70], 0.009, 1000, 0)
    r1 = O.select_cells(m, [64], [10, 64, 70], 0.009, 1000, 0, tile=64)
    assert list(r0.kept[0]) == [True, False, True] and r0.pairs == 640 + 4480
    assert list(r1.kept[0]) == [False, False, True] and r1.pairs == 4480


def test_tile_padded_equals_unpadded_on_whole_tiles():
    """Group sizes that are multiples of 64 make the two cost models identical."""
    qc = 64 * RNG.integers(0, 4, 6)
    kc = 64 * RNG.integers(0, 4, 5)
    n = int(qc.sum())
    m = RNG.integers(0, 10 ** 9, (6, 5))
    for rho in (0.1, 0.3, 0.6):
        a = O.select_cells(m, qc, kc, rho, n, 4)
        b = O.select_cells(m, qc, kc, rho, n, 4, tile=64)
        np.testing.assert_array_equal(a.kept, b.kept)


def test_global_budget_single_head_is_the_per_head_route():
    n = 400
    qc = np.bincount(RNG.integers(0, 6, n), minlength=6)
    kc = np.bincount(RNG.integers(0, 5, n), minlength=5)
    m = RNG.integers(0, 10 ** 9, (6, 5))
    for rho in (0.05, 0.3):
        for tile in (0, 64):
            a = O.select_cells(m, qc, kc, rho, n, 8, tile)
            (b,) = O.select_cells_global([m], [qc], [kc], rho, n, 8, tile)
            np.testing.assert_array_equal(a.kept, b.kept)


def test_global_budget_moves_budget_to_the_concentrated_head():
    """Two heads, one query group, four key groups of 50 keys and 100 queries (cells of
    5000 pairs), per-head budget 3 cells.  Head 0's masses all beat head 1's: per head each
    keeps its mandatory cell plus two; with the shared budget of 6 cells head 0 keeps all
    four and head 1 its mandatory cell plus one (the best of its remaining three)."""
    n = 1000
    qc, kc = np.array([100]), np.array([50, 50, 50, 50])
    m0, m1 = np.array([[900, 800, 700, 600]]), np.array([[40, 10, 30, 20]])
    rho = 0.015          # 15000 pairs per head with no probes
    assert O.route_budget(rho, n, 0) == 15000
    per = [O.select_cells(m, qc, kc, rho, n, 0) for m in (m0, m1)]
    assert [list(r.kept[0]) for r in per] == [[True, True, True, False], [True, False, True, True]]
    glob = O.select_cells_global([m0, m1], [qc, qc], [kc, kc], rho, n, 0)
    assert [list(r.kept[0]) for r in glob] == [[True, True, True, True], [True, False, True, False]]
    assert sum(r.pairs for r in glob) == 6 * 5000


@pytest.mark.parametrize("tile", [0, 64])
def test_global_budget_is_a_feasible_maximal_prefix(tile):
    """Over random heads: the kept cost fits the shared budget, every kept optional cell
    precedes every dropped one in the shared order (ratio, then head, then cell), and the
    first dropped cell would not fit."""
    H, n = 3, 600
    qcs = [np.bincount(RNG.integers(0, 5, n), minlength=5) for _ in range(H)]
    kcs = [np.bincount(RNG.integers(0, 6, n), minlength=6) for _ in range(H)]
    ms = [RNG.integers(0, 10 ** 8, (5, 6)) for _ in range(H)]
    rs = O.select_cells_global(ms, qcs, kcs, 0.2, n, 4, tile)
    costs = [O.cell_costs(qcs[h], kcs[h], tile) for h in range(H)]
    total = sum(int(costs[h][rs[h].kept].sum()) for h in range(H))
    assert total <= 3 * O.route_budget(0.2, n, 4) or all(
        (rs[h].kept == rs[h].mandatory).all() for h in range(H))
    opt = [(Fraction(int(ms[h][a, b]), int(costs[h][a, b])), h, a * 6 + b, bool(rs[h].kept[a, b]))
           for h in range(H) for a in range(5) for b in range(6)
           if costs[h][a, b] > 0 and not rs[h].mandatory[a, b]]
    opt.sort(key=lambda t: (-t[0], t[1], t[2]))
    flags = [t[3] for t in opt]
    first_drop = flags.index(False) if False in flags else len(flags)
    assert all(flags[:first_drop]) and not any(flags[first_drop:])
    if first_drop < len(opt):
        _, h, c, _ = opt[first_drop]
        assert total + int(costs[h][c // 6, c % 6]) > 3 * O.route_budget(0.2, n, 4)


# ------------------------------------------------------------ support from given scores
def test_supports_from_scores_closed_forms_and_subset_brute_force():
    """Integer-mass supports on given float32 scores: uniform scores need ceil(mass n) keys
    (the lowest indices), a dominant score needs one key, and on tiny random rows the count
    is the smallest k for which some k-subset's integer mass reaches the target (subset
    enumeration, no sorting), with members the highest scores, ties to lower indices."""
    f = np.zeros((1, 8), np.float32)
    cnt, mem = Dg.supports_from_scores(f, 1.0, 0.75)
    assert cnt[0] == 6 and mem[0].tolist() == [True] * 6 + [False] * 2
    f = np.array([[0.0, 100.0, 0.0, 0.0]], np.float32)
    cnt, mem = Dg.supports_from_scores(f, 1.0, 0.9)
    assert cnt[0] == 1 and mem[0].tolist() == [False, True, False, False]
    rng = np.random.default_rng(11)
    for _ in range(40):
        n = int(rng.integers(2, 8))
        row = (rng.integers(-3, 4, n) * 0.5).astype(np.float32)   # repeated values -> ties
        scale = float(np.float32(rng.uniform(0.3, 2.0)))
        mass = float(rng.choice([0.5, 0.75, 0.9]))
        cnt, mem = Dg.supports_from_scores(row[None], scale, mass)
        x = (row.astype(np.float64) - float(row.max())) * scale
        m = [int(v) for v in np.floor(np.ldexp(np.exp(x), 40))]
        total = sum(m)
        want = math.ceil(float(total) * mass)
        tgt = max(total if want >= total else want, 1)
        best = min(k for k in range(1, n + 1)
                   if max(sum(m[i] for i in c) for c in itertools.combinations(range(n), k)) >= tgt)
        assert cnt[0] == best, (row, mass, cnt[0], best)
        keep = sorted(range(n), key=lambda i: (-float(row[i]), i))[:best]
        assert sorted(np.nonzero(mem[0])[0].tolist()) == sorted(keep)


def test_supports_from_scores_agree_with_float64_probabilities():
    """On random float32 scores the integer-mass count equals the float64-probability count
    except where the mass threshold falls within the 2^-40 quantisation of a boundary."""
    rng = np.random.default_rng(12)
    q, k = rng.standard_normal((40, 16)), rng.standard_normal((300, 16))
    scale = 0.25
    f = (q @ k.T).astype(np.float32)
    cnt, _ = Dg.supports_from_scores(f, scale, 0.9)
    p = np.exp((f.astype(np.float64) - f.max(axis=1, keepdims=True)) * scale)
    p /= p.sum(axis=1, keepdims=True)
    for r in range(40):
        srt = -np.sort(-p[r])
        c = np.cumsum(srt)
        want = int((c < 0.9).sum()) + 1
        assert abs(int(cnt[r]) - want) <= 1 and (cnt[r] == want or abs(c[want - 1] - 0.9) < 1e-9)
