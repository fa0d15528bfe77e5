"""Plain CPU oracle of the SparsePR attention call (float64 NumPy).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything under ``oracle/``.
The GPU library never calls it, and it shares no code with the GPU library.

Citation key.  PSRR = the summary page of "Partition the Support, Reconstruct the
Residual: Training-Free Sparse Attention for Video Generation and World Models"
(Taghavi, Langari, Pandey).  Its paragraphs are cited by topic: *support* (single-row
and shared-route 90 %-mass support), *hard-drop residual*, *response-coupled partition*,
*probe-fit residual reconstruction*, *execution* (group-major layout, varlen block-sparse
kernel, GQA sharing, rho_exec accounting, what is timed), *ablation*.  LMNT = the
lmnt.cn SparsePR article; its section 2.1 gives dense softmax attention.

The page states what each stage computes but leaves counts, rules and precisions open.
Every reading taken here is marked "Reading:" and is the same one the GPU library
implements.  Integer stages (features, k-means, permutation, routing, probes) are exact
integer arithmetic given the response matrices S and U, so they can be compared
bit for bit.  Where a float decides an integer (the rounding of S and U to integer
features and route logits) the oracle takes the decision on the same float values
the kernel produced when it is fed them.

Parity pins: see tests/test_oracle_*.py.  The whole call has no printed worked
example on the pages; beyond the closed forms, reductions and brute-force checks
listed there, end-to-end values are parity unpinned.
"""
from dataclasses import dataclass
from fractions import Fraction

import numpy as np

FEATURE_MAX = 127           # integer feature range [-127, 127]
QUERY_RESP_LIMIT = 2 ** 14  # integer resolution of the query response profile
ROUTE_LOGIT_UNITS = 64      # route logits in 1/64-logit units
EXP_TABLE_SIZE = 1024
MASS_ONE = 2 ** 20          # fixed-point one for per-row masses
EIG_REL_TOL = 1e-8


@dataclass(frozen=True)
class Params:
    """Hyper-parameters; defaults are the values the PSRR partition / probe-fit
    paragraphs fix (r_K=48, r_Q=64, M=64, r=16, lambda=0.1)."""
    groups_q: int
    groups_k: int
    rho_exec: float
    r_k: int = 48
    r_q: int = 64
    n_probe: int = 64
    rank: int = 16
    lam: float = 0.1
    kmeans_iters: int = 10
    scale: float = 0.0       # 0 -> 1/sqrt(d)
    tile_cost: int = 0       # 0: cell cost n_a n_b; 64: tile-padded cost (budget variant)
    global_budget: bool = False   # one budget shared by all KV heads (budget variant)

    def softmax_scale(self, d):
        return self.scale if self.scale > 0 else 1.0 / np.sqrt(d)


def f64(x):
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------------------
# dense attention (LMNT section 2.1): O = softmax(Q K^T / sqrt(d_k)) V
# --------------------------------------------------------------------------------------
def dense_attention(q, k, v, scale, rows=None, chunk=1024):
    """Exact softmax attention of the given rows against all keys; returns (O, LSE)."""
    q, k, v = f64(q), f64(k), f64(v)
    if rows is not None:
        q = q[np.asarray(rows)]
    out = np.empty((q.shape[0], v.shape[1]))
    lse = np.empty(q.shape[0])
    for c0 in range(0, q.shape[0], chunk):
        s = (q[c0:c0 + chunk] @ k.T) * scale
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l_ = e.sum(axis=1)
        out[c0:c0 + chunk] = (e @ v) / l_[:, None]
        lse[c0:c0 + chunk] = m[:, 0] + np.log(l_)
    return out, lse


# --------------------------------------------------------------------------------------
# response-coupled partition (PSRR, response-coupled partition paragraph)
# --------------------------------------------------------------------------------------
def sample_queries(n, r_k, g):
    """Reading: the page samples "a batch of the current call's queries" without a
    count or rule.  r_K = 48 rows, evenly strided in raster order (token
    floor((2s+1) N / (2 r_K))), cycling over the g query heads of the KV head."""
    s = np.arange(r_k)
    return (2 * s + 1) * n // (2 * r_k), s % g


def key_responses(q_heads, k, scale, r_k):
    """S [r_K, N]: pre-softmax responses of the sampled queries to every key."""
    q_heads = f64(q_heads)
    tok, hd = sample_queries(k.shape[0], r_k, q_heads.shape[0])
    return (q_heads[hd, tok] @ f64(k).T) * scale


def pow2_exponent(maxabs, limit):
    """Largest integer e with maxabs * 2**e <= limit (0 when maxabs == 0)."""
    maxabs = float(maxabs)
    if maxabs == 0.0:
        return 0
    e = int(np.floor(np.log2(limit / maxabs)))
    while maxabs * 2.0 ** (e + 1) <= limit:
        e += 1
    while maxabs * 2.0 ** e > limit:
        e -= 1
    return e


def key_features(S):
    """Integer key features X^K [N, r_K] from the response matrix.

    Reading: the distance between keys is the Euclidean distance of their raw response
    curves (no per-key centring: a per-query shift moves every key alike and softmax
    ignores it).  The curves are scaled by one power of two per head so that the
    largest magnitude is at most 127, then rounded half-to-even, which makes the
    k-means exact integer arithmetic."""
    S = f64(S)
    e = pow2_exponent(np.abs(S).max() if S.size else 0.0, FEATURE_MAX)
    X = np.clip(np.rint(S * 2.0 ** e), -FEATURE_MAX, FEATURE_MAX).astype(np.int64)
    return X.T.copy(), e


def div_rhaz(a, b):
    """Integer a / b (b > 0) rounded half away from zero."""
    a = np.asarray(a, dtype=np.int64)
    b = np.asarray(b, dtype=np.int64)
    return np.sign(a) * ((2 * np.abs(a) + b) // (2 * b))


def kmeans_init_tokens(n, groups):
    return (2 * np.arange(groups) + 1) * n // (2 * groups)


def kmeans_assign(X, C):
    """argmin_g ||c_g||^2 - 2 <x, c_g>; ties go to the smallest g.  All values are
    integers far below 2**53, so the float64 products are exact."""
    Xf, Cf = X.astype(np.float64), C.astype(np.float64)
    score = (Cf * Cf).sum(axis=1)[None, :] - 2.0 * (Xf @ Cf.T)
    return np.argmin(score, axis=1).astype(np.int64)


def kmeans_update(X, labels, C):
    """c_g = rounded mean of its members; an empty group keeps its centroid."""
    G, F = C.shape
    counts = np.bincount(labels, minlength=G)
    sums = np.stack([np.bincount(labels, weights=X[:, f].astype(np.float64), minlength=G)
                     for f in range(F)], axis=1).astype(np.int64)
    newC = C.copy()
    ne = counts > 0
    newC[ne] = div_rhaz(sums[ne], counts[ne][:, None])
    return newC


def kmeans(X, groups, iters):
    """Online Lloyd k-means (PSRR, response-coupled partition paragraph; the accounting
    paragraph counts this online k-means inside the call).

    Reading: initial centroids are the features of tokens floor((2g+1) N / (2 G)); a fixed
    number of iterations (each an assignment then an update) followed by a final
    assignment.  Returns (labels, centroids the final assignment used)."""
    X = np.asarray(X, dtype=np.int64)
    C = X[kmeans_init_tokens(X.shape[0], groups)].copy()
    for _ in range(iters):
        C = kmeans_update(X, kmeans_assign(X, C), C)
    return kmeans_assign(X, C), C


def group_major(labels, groups):
    """Stable group-major order (PSRR, execution paragraph: Q, K, V laid out group-major).

    Reading: within a group, tokens keep their original order.  Returns
    (perm, inverse perm, offsets): perm[p] is the token at group-major position p."""
    labels = np.asarray(labels, dtype=np.int64)
    counts = np.bincount(labels, minlength=groups)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    perm = np.argsort(labels, kind="stable").astype(np.int64)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    return perm, inv, offsets


def key_centroids(k, labels, groups):
    """C^K_b = mean of the original key vectors of group b (0 for an empty group)."""
    k = f64(k)
    counts = np.bincount(labels, minlength=groups)
    C = np.zeros((groups, k.shape[1]))
    for b in range(groups):
        if counts[b]:
            C[b] = k[labels == b].mean(axis=0)
    return C


def query_responses(q_heads, Ck, scale):
    """U^(h) = Q^(h) C^K^T * scale for every query head of the KV head: [g, N, G_K]."""
    return np.einsum("hnd,bd->hnb", f64(q_heads), f64(Ck)) * scale


def summed_response(U_heads):
    """Reading: under GQA the route is shared by the KV head's query heads (PSRR,
    execution paragraph), so the query coordinate is the response summed over those heads:
    sum_h U^(h), formed in float64 in ascending head order (for g = 1 the single response
    as given)."""
    U_heads = np.asarray(U_heads)
    acc = f64(U_heads[0]).copy()
    for j in range(1, U_heads.shape[0]):
        acc = acc + f64(U_heads[j])
    return acc


def query_features(U_heads, U_sum=None):
    """Integer response-direction features X^Q [N, G_K].

    Reading: queries "whose response directions are alike" share a route.  A direction
    is taken invariant to a per-row shift (softmax ignores it) and to a positive
    per-row scale: quantise the summed response at 2**14 levels of the head maximum,
    centre each row (G_K u - sum u), and divide by the row's largest magnitude onto
    [-127, 127] with round-half-away integer division.  The feature width is
    min(r_Q, G_K) = G_K (G_K > r_Q is rejected).

    ``U_sum`` [N, G_K], when given, is the head-summed coordinate to quantise in place of
    summed_response(U_heads): the float values another implementation formed, so that the
    integer decisions below are taken on identical inputs."""
    U = summed_response(U_heads) if U_sum is None else f64(U_sum)
    e = pow2_exponent(np.abs(U).max() if U.size else 0.0, QUERY_RESP_LIMIT)
    u = np.rint(U * 2.0 ** e).astype(np.int64)
    c = U.shape[1] * u - u.sum(axis=1, keepdims=True)
    mx = np.abs(c).max(axis=1, keepdims=True)
    x = np.where(mx > 0, div_rhaz(FEATURE_MAX * c, np.maximum(mx, 1)), 0)
    return x.astype(np.int64), e


@dataclass
class Partition:
    S: np.ndarray            # [r_K, N]
    e_s: int
    xk: np.ndarray           # [N, r_K] int
    k_labels: np.ndarray
    k_centroids_int: np.ndarray
    k_perm: np.ndarray
    k_inv: np.ndarray
    k_offsets: np.ndarray
    k_centroids: np.ndarray  # [G_K, d] original space
    U: np.ndarray            # [g, N, G_K]
    e_u: int
    xq: np.ndarray           # [N, G_K] int
    q_labels: np.ndarray
    q_centroids: np.ndarray  # [G_Q, G_K] int (the ones the final assignment used)
    q_perm: np.ndarray
    q_inv: np.ndarray
    q_offsets: np.ndarray


def partition(q_heads, k, p: Params, S=None, U=None, U_sum=None):
    """Response-coupled partition of one KV head (PSRR, response-coupled partition
    paragraph): keys first, then queries, one asymmetric pass.  S, U and the head-summed
    U_sum may be supplied (e.g. the GPU's) to take every integer decision on identical
    responses."""
    q_heads, k = f64(q_heads), f64(k)
    n, d = k.shape
    scale = p.softmax_scale(d)
    if p.groups_k > p.r_q:
        raise ValueError("G_K > r_Q")
    if S is None:
        S = key_responses(q_heads, k, scale, p.r_k)
    xk, e_s = key_features(S)
    k_labels, kc = kmeans(xk, p.groups_k, p.kmeans_iters)
    k_perm, k_inv, k_off = group_major(k_labels, p.groups_k)
    Ck = key_centroids(k, k_labels, p.groups_k)
    if U is None:
        U = query_responses(q_heads, Ck, scale)
    xq, e_u = query_features(U, U_sum)
    q_labels, qc = kmeans(xq, p.groups_q, p.kmeans_iters)
    q_perm, q_inv, q_off = group_major(q_labels, p.groups_q)
    return Partition(np.asarray(S), e_s, xk, k_labels, kc, k_perm, k_inv, k_off, Ck,
                     np.asarray(U), e_u, xq, q_labels, qc, q_perm, q_inv, q_off)


# --------------------------------------------------------------------------------------
# routing to a target execution density (PSRR, execution paragraph)
# --------------------------------------------------------------------------------------
def exp_table():
    """E[k] = rint(2**20 exp(-k/64)), k = 0..1023 (E[k] = 0 from k = 932 on)."""
    k = np.arange(EXP_TABLE_SIZE, dtype=np.float64)
    return np.rint(MASS_ONE * np.exp(-k / ROUTE_LOGIT_UNITS)).astype(np.int64)


def row_masses(U_head, k_counts, table=None):
    """Fixed-point per-row key-group masses P_i(b) [N, G_K] for one query head.

    Reading (the block score is not on the page): each query's mass on key group b is
    estimated by treating b's keys as copies of its centroid, i.e. the size-weighted
    softmax of the centroid responses, n_b exp(U_ib) / sum_b' n_b' exp(U_ib').  Logits
    are rounded to 1/64 units and exponentiated through a 1024-entry table so every
    later decision is integer; P sums to at most 2**20 per row."""
    table = exp_table() if table is None else table
    k_counts = np.asarray(k_counts, dtype=np.int64)
    ne = k_counts > 0
    z = np.rint(ROUTE_LOGIT_UNITS * f64(U_head)).astype(np.int64)
    mu = np.where(ne[None, :], z, np.iinfo(np.int64).min).max(axis=1)
    dz = np.minimum(mu[:, None] - z, EXP_TABLE_SIZE - 1)
    dz = np.where(ne[None, :], dz, EXP_TABLE_SIZE - 1)
    e = np.where(ne[None, :], k_counts[None, :] * table[dz], 0)
    tot = e.sum(axis=1)
    return (e << 20) // tot[:, None]


def block_mass(U_heads, q_labels, k_counts, groups_q, table=None):
    """Cell mass m_ab = sum over the KV head's query heads and over the queries i of
    group a of P_i(b) (exact integers)."""
    U_heads = np.asarray(U_heads)
    Gk = U_heads.shape[2]
    m = np.zeros((groups_q, Gk), dtype=np.int64)
    for h in range(U_heads.shape[0]):
        P = row_masses(U_heads[h], k_counts, table)
        for b in range(Gk):
            m[:, b] += np.bincount(q_labels, weights=P[:, b].astype(np.float64),
                                   minlength=groups_q).astype(np.int64)
    return m


def route_budget(rho, n, n_probe):
    """Route budget in pairs per head: rho_exec = rho_route + M/N, with the probe cost
    subtracted first (PSRR, execution paragraph).  rho is taken as the float32 value the
    library receives, converted once to integer parts per million."""
    rho_ppm = int(np.floor(float(np.float32(rho)) * 1e6 + 0.5))
    return (rho_ppm * n * n) // 1_000_000 - n_probe * n


@dataclass
class Route:
    kept: np.ndarray         # [G_Q, G_K] bool
    mandatory: np.ndarray    # [G_Q, G_K] bool
    row_ptr: np.ndarray      # [G_Q + 1]
    cols: np.ndarray         # ascending per row
    pairs: int               # routed (unpadded) pairs
    budget: int
    mass: np.ndarray         # [G_Q, G_K]


def cell_costs(q_counts, k_counts, tile=0):
    """Cost of every cell (a, b) in query-key pairs: n_a n_b, or with ``tile`` > 0 the
    pairs of the tiles it occupies, ceil(n_a / tile) tile x ceil(n_b / tile) tile (a cell is
    an indivisible routing unit and the kernel executes whole tiles; execution paragraph).
    Empty groups cost 0."""
    qc = np.asarray(q_counts, dtype=np.int64)
    kc = np.asarray(k_counts, dtype=np.int64)
    if tile > 0:
        qc = (qc + tile - 1) // tile * tile
        kc = (kc + tile - 1) // tile * tile
    return qc[:, None] * kc[None, :]


def _mandatory(m, q_counts, k_counts):
    """Every non-empty query group keeps its heaviest non-empty key group (ties: smaller b),
    so the renormalised set is never empty."""
    qc, kc = np.asarray(q_counts), np.asarray(k_counts)
    mand = np.zeros(m.shape, dtype=bool)
    for a in range(m.shape[0]):
        if qc[a] == 0 or not np.any(kc > 0):
            continue
        mand[a, int(np.argmax(np.where(kc > 0, m[a], -1)))] = True
    return mand


def _route_of(kept, mand, m, q_counts, k_counts, budget):
    Gq = kept.shape[0]
    row_ptr = np.concatenate([[0], np.cumsum(kept.sum(axis=1))]).astype(np.int64)
    cols = np.concatenate([np.nonzero(kept[a])[0] for a in range(Gq)]).astype(np.int64) \
        if kept.any() else np.zeros(0, np.int64)
    pairs = int(cell_costs(q_counts, k_counts)[kept].sum())
    return Route(kept, mand, row_ptr, cols, pairs, budget, m)


def select_cells(m, q_counts, k_counts, rho, n, n_probe, tile=0):
    """Top-cell selection to the target execution density.

    Reading (the order and the overshoot rule are not on the page; cells are
    indivisible so the realised density deviates from the target, and the page reports
    realised values): every non-empty query group keeps its heaviest non-empty key
    group (ties: smaller b) so the renormalised set is never empty; the remaining
    non-empty cells are ranked by mass per unit cost m_ab / c_ab (exact rational
    comparison), larger first, ties to smaller a*G_K + b, and the longest prefix whose
    cost fits the budget left after the mandatory cells is kept (a fractional-knapsack
    order for retained mass).  c_ab = n_a n_b, or tile-padded with ``tile`` > 0; the
    reported pairs are always the unpadded n_a n_b of the kept cells."""
    m = np.asarray(m, dtype=np.int64)
    Gq, Gk = m.shape
    cost = cell_costs(q_counts, k_counts, tile)
    B = route_budget(rho, n, n_probe)
    mand = _mandatory(m, q_counts, k_counts)
    kept = mand.copy()
    left = B - int(cost[mand].sum())
    ranked = []
    for a in range(Gq):
        for b in range(Gk):
            if cost[a, b] > 0 and not mand[a, b]:
                ranked.append((-Fraction(int(m[a, b]), int(cost[a, b])), a * Gk + b, a, b))
    ranked.sort()
    used = 0
    for _, _, a, b in ranked:
        c = int(cost[a, b])
        if used + c > left:
            break
        kept[a, b] = True
        used += c
    return _route_of(kept, mand, m, q_counts, k_counts, B)


def select_cells_global(ms, q_counts, k_counts, rho, n, n_probe, tile=0):
    """Budget shared by all KV heads of the call (a variant the page leaves open: heads
    whose mass is concentrated can take budget from diffuse ones).  The mandatory cells
    stay per head; the budget is H_kv times the per-head budget; the remaining cells of
    all heads are ranked together by m_ab / c_ab, larger first, ties to the smaller
    (head, a*G_K + b), and the longest prefix that fits is kept.  Returns one Route per
    head (each reports the shared budget)."""
    H = len(ms)
    B = route_budget(rho, n, n_probe) * H
    costs = [cell_costs(q_counts[h], k_counts[h], tile) for h in range(H)]
    mands = [_mandatory(np.asarray(ms[h], np.int64), q_counts[h], k_counts[h]) for h in range(H)]
    kepts = [mk.copy() for mk in mands]
    left = B - sum(int(costs[h][mands[h]].sum()) for h in range(H))
    ranked = []
    for h in range(H):
        m = np.asarray(ms[h], np.int64)
        Gq, Gk = m.shape
        for a in range(Gq):
            for b in range(Gk):
                if costs[h][a, b] > 0 and not mands[h][a, b]:
                    ranked.append((-Fraction(int(m[a, b]), int(costs[h][a, b])), h, a * Gk + b, a, b))
    ranked.sort()
    used = 0
    for _, h, _, a, b in ranked:
        c = int(costs[h][a, b])
        if used + c > left:
            break
        kepts[h][a, b] = True
        used += c
    return [_route_of(kepts[h], mands[h], np.asarray(ms[h], np.int64), q_counts[h], k_counts[h], B)
            for h in range(H)]


def route(part: Partition, p: Params, n):
    """Route of one KV head with its own budget (the global budget needs every head: see
    route_heads)."""
    qc = np.diff(part.q_offsets)
    kc = np.diff(part.k_offsets)
    m = block_mass(part.U, part.q_labels, kc, p.groups_q)
    return select_cells(m, qc, kc, p.rho_exec, n, p.n_probe, p.tile_cost)


def route_heads(parts, p: Params, n):
    """Routes of all KV heads of a call: per head, or with p.global_budget one shared
    budget."""
    if not p.global_budget:
        return [route(part, p, n) for part in parts]
    qcs = [np.diff(part.q_offsets) for part in parts]
    kcs = [np.diff(part.k_offsets) for part in parts]
    ms = [block_mass(part.U, part.q_labels, kc, p.groups_q) for part, kc in zip(parts, kcs)]
    return select_cells_global(ms, qcs, kcs, p.rho_exec, n, p.n_probe, p.tile_cost)


# --------------------------------------------------------------------------------------
# block-sparse attention renormalised over the kept K/V groups (PSRR, execution paragraph)
# --------------------------------------------------------------------------------------
def sparse_attention(q, k, v, scale, q_labels, k_labels, kept, rows=None):
    """For a query of group a, softmax over the keys of the key groups kept in row a
    only; exact within those cells.  Returns (O, LSE) for the requested rows."""
    q, k, v = f64(q), f64(k), f64(v)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    out = np.empty((rows.size, v.shape[1]))
    lse = np.empty(rows.size)
    ql = np.asarray(q_labels)[rows]
    for a in np.unique(ql):
        sel = np.nonzero(ql == a)[0]
        keys = np.nonzero(kept[a][np.asarray(k_labels)])[0]
        o, l_ = dense_attention(q[rows[sel]], k[keys], v[keys], scale)
        out[sel], lse[sel] = o, l_
    return out, lse


# --------------------------------------------------------------------------------------
# probe-fit residual reconstruction (PSRR, probe-fit residual reconstruction paragraph)
# --------------------------------------------------------------------------------------
def probe_allocation(q_counts, n_probe):
    """Reading: M probes are spread equally over the non-empty query groups, one at a
    time in the order (larger group first, then smaller index), skipping a group once
    every member is a probe.  So each group gets floor or ceil of M / G', the larger
    groups take the remainder, and a full group passes its share on."""
    qc = np.asarray(q_counts, dtype=np.int64)
    order = sorted([a for a in range(qc.size) if qc[a] > 0], key=lambda a: (-qc[a], a))
    m = np.zeros(qc.size, dtype=np.int64)
    total = 0
    while total < n_probe:
        moved = False
        for a in order:
            if total < n_probe and m[a] < qc[a]:
                m[a] += 1
                total += 1
                moved = True
        if not moved:
            raise ValueError("more probes than queries")
    return m


@dataclass
class Probes:
    tokens: np.ndarray   # [M] token indices, group ascending, radial rank ascending
    groups: np.ndarray   # [M]
    weights: np.ndarray  # [M] group-coverage weights, sum = M
    alloc: np.ndarray    # [G_Q]


def select_probes(xq, q_labels, q_centroids, q_counts, n_probe):
    """Probe rows stratified by query group and drawn in radial order about the group
    centroid.

    Reading: within group a the members are ordered by the integer squared distance of
    their direction features to the group's centroid (the one its final assignment
    used), ties by token index, and the m_a probes are the evenly spaced ranks
    floor((2k+1) n_a / (2 m_a)).  Group-coverage weight w = n_a / m_a (the tokens each
    probe stands for), scaled to mean 1 so lambda keeps its unweighted meaning."""
    xq = np.asarray(xq, dtype=np.int64)
    q_labels = np.asarray(q_labels)
    n = xq.shape[0]
    alloc = probe_allocation(q_counts, n_probe)
    toks, grps, wts = [], [], []
    for a in range(alloc.size):
        ma = int(alloc[a])
        if ma == 0:
            continue
        mem = np.nonzero(q_labels == a)[0]
        na = mem.size
        diff = xq[mem] - np.asarray(q_centroids[a], dtype=np.int64)[None, :]
        rad = (diff * diff).sum(axis=1)
        order = np.lexsort((mem, rad))
        for kk in range(ma):
            toks.append(int(mem[order[(2 * kk + 1) * na // (2 * ma)]]))
            grps.append(a)
            wts.append(n_probe * na / (ma * n))
    return Probes(np.array(toks, np.int64), np.array(grps, np.int64), np.array(wts), alloc)


def probe_rows(q, k, v, scale, tokens, q_labels, k_labels, kept):
    """Exact probe rows against all keys, their sparse outputs, and R = O_dense - O_sparse."""
    od, lse_d = dense_attention(q, k, v, scale, rows=tokens)
    os_, lse_s = sparse_attention(q, k, v, scale, q_labels, k_labels, kept, rows=tokens)
    return od, os_, od - os_, lse_d, lse_s


def weighted_center(X, Y, w):
    w = f64(w)
    sw = w.sum()
    xbar = (w @ f64(X)) / sw
    ybar = (w @ f64(Y)) / sw
    r = np.sqrt(w)[:, None]
    return xbar, ybar, r * (f64(X) - xbar), r * (f64(Y) - ybar)


def ridge_fit(X, Y, w, lam):
    """Group-coverage-weighted ridge fit of the residual as an affine function of the
    sparse output.

    Reading: textbook weighted ridge with a centred, unpenalised intercept; lambda is
    absolute with mean-one weights.  Solved in the dual (M x M) form
    W = Xt^T (Xt Xt^T + lambda I_M)^{-1} Yt with Xt = Omega^1/2 X_c, Yt = Omega^1/2 Y_c.
    Returns (W [d, d], xbar, ybar, Xt, Yt)."""
    xbar, ybar, Xt, Yt = weighted_center(X, Y, w)
    Kmat = Xt @ Xt.T + lam * np.eye(Xt.shape[0])
    Z = np.linalg.solve(Kmat, Yt)
    return Xt.T @ Z, xbar, ybar, Xt, Yt


def output_subspace(Yt, rank, rel_tol=EIG_REL_TOL):
    """Rank-r output subspace observed in the weighted, centred probe residuals.

    Reading: the top-r eigenpairs (lambda_k, a_k) of Yt Yt^T (M x M) with
    lambda_k > rel_tol * lambda_1 give orthonormal output directions
    V_r[:, k] = Yt^T a_k / sqrt(lambda_k).  Returns (V_r [d, r_eff], top r+1 eigenvalues)."""
    Yt = f64(Yt)
    ev, vec = np.linalg.eigh(Yt @ Yt.T)
    ev, vec = ev[::-1], vec[:, ::-1]
    top = ev[:rank + 1].copy()
    lam1 = ev[0] if ev.size else 0.0
    keep = [i for i in range(min(rank, ev.size)) if lam1 > 0 and ev[i] > rel_tol * lam1]
    if not keep:
        return np.zeros((Yt.shape[1], 0)), top
    a = vec[:, keep]
    return (Yt.T @ a) / np.sqrt(ev[keep])[None, :], top


@dataclass
class Fit:
    A: np.ndarray       # [d, r_eff]
    B: np.ndarray       # [r_eff, d]
    c0: np.ndarray      # [d]
    W: np.ndarray
    xbar: np.ndarray
    ybar: np.ndarray
    V: np.ndarray
    eig: np.ndarray
    o_dense: np.ndarray  # probe rows [M, d]
    o_sparse: np.ndarray
    R: np.ndarray


def probe_fit(q, k, v, scale, probes: Probes, q_labels, k_labels, kept, p: Params):
    """Probe rows, weighted ridge and rank-r projection for one query head.  Only the
    feature-dependent part of the correction is projected: the correction of a row is
    ybar + (o - xbar) W V_r V_r^T = o A B + c0 with A = W V_r, B = V_r^T,
    c0 = ybar - xbar A B."""
    od, os_, R, _, _ = probe_rows(q, k, v, scale, probes.tokens, q_labels, k_labels, kept)
    return fit_from_probe_rows(od, os_, probes.weights, p)


def fit_from_probe_rows(o_dense, o_sparse, weights, p: Params):
    """The weighted ridge and rank-r projection given the probe rows' dense and sparse
    outputs (R = O_dense - O_sparse)."""
    od, os_ = f64(o_dense), f64(o_sparse)
    R = od - os_
    W, xbar, ybar, Xt, Yt = ridge_fit(os_, R, weights, p.lam)
    V, eig = output_subspace(Yt, p.rank)
    A = W @ V
    B = V.T
    c0 = ybar - xbar @ A @ B
    return Fit(A, B, c0, W, xbar, ybar, V, eig, od, os_, R)


def apply_correction(o_sparse, fit: Fit, probe_tokens):
    """o_hat = o + c0 + (o A) B for every row; probe rows take their exact dense output."""
    o = f64(o_sparse)
    out = o + fit.c0[None, :] + (o @ fit.A) @ fit.B
    out[np.asarray(probe_tokens)] = fit.o_dense
    return out


def correct_rows(o_rows, fit: Fit):
    o = f64(o_rows)
    return o + fit.c0[None, :] + (o @ fit.A) @ fit.B


# --------------------------------------------------------------------------------------
# ablations (PSRR, ablation paragraph): hard drop, ridge without the projection, and
# probe rows drawn uniformly over space-time or by the caller instead of stratified
# radially.  The page names the variants and reports their ordering; how each is built
# is a reading.
# --------------------------------------------------------------------------------------
def hard_drop_rows(q, k, v, scale, q_labels, k_labels, kept, rows=None):
    """Hard drop: the output is the renormalised sparse attention itself (no probes, no
    fit, no correction)."""
    o, _ = sparse_attention(q, k, v, scale, q_labels, k_labels, kept, rows=rows)
    return o


def semantic_features(x_heads, x_sum=None):
    """Integer features of raw activations for the semantic-partition ablation (the page
    contrasts its response-coupled partition with clustering the activations
    themselves).  Reading: keys use their own rows; queries under GQA use the rows summed
    over the KV head's query heads (as the query coordinate is: float64, ascending head
    order); one power of two per head scales the largest magnitude to at most 127, then
    round half-to-even, as for the key response features.  Width d.  ``x_sum`` [N, d],
    when given, replaces the head sum (another implementation's float values, so the
    integer decisions are taken on identical inputs)."""
    X = summed_response(x_heads) if x_sum is None else f64(x_sum)
    e = pow2_exponent(np.abs(X).max() if X.size else 0.0, FEATURE_MAX)
    return np.clip(np.rint(X * 2.0 ** e), -FEATURE_MAX, FEATURE_MAX).astype(np.int64), e


def partition_semantic(q_heads, k, p: Params, U=None, x_sum=None):
    """Semantic partition: the same k-means, permutation and key centroids as the method,
    but keys clustered on their raw vectors and queries on their raw vectors (not on
    response curves and response directions).  The route still scores cells with the
    query responses U to the key centroids.  S is not formed (None)."""
    q_heads, k = f64(q_heads), f64(k)
    scale = p.softmax_scale(k.shape[1])
    xk, e_k = semantic_features(k[None])
    k_labels, kc = kmeans(xk, p.groups_k, p.kmeans_iters)
    k_perm, k_inv, k_off = group_major(k_labels, p.groups_k)
    Ck = key_centroids(k, k_labels, p.groups_k)
    if U is None:
        U = query_responses(q_heads, Ck, scale)
    xq, e_q = semantic_features(q_heads, x_sum)
    q_labels, qc = kmeans(xq, p.groups_q, p.kmeans_iters)
    q_perm, q_inv, q_off = group_major(q_labels, p.groups_q)
    return Partition(None, e_k, xk, k_labels, kc, k_perm, k_inv, k_off, Ck,
                     np.asarray(U), e_q, xq, q_labels, qc, q_perm, q_inv, q_off)


def uniform_probes(n, q_labels, n_probe):
    """Uniform spatiotemporal probes.  Reading: the tokens floor((2k+1) N / (2M)), k < M,
    of the raster (t, h, w) order, i.e. evenly spaced over the clip; each stands for N / M
    tokens, so every mean-one weight is 1; a probe's group is its query label (it selects
    the kept cells of the probe's sparse row)."""
    k = np.arange(n_probe, dtype=np.int64)
    toks = (2 * k + 1) * n // (2 * n_probe)
    return given_probes(toks, q_labels)


def given_probes(tokens, q_labels):
    """Probe rows chosen by the caller (e.g. drawn uniformly at random with a seeded
    generator): weight 1 each, group = query label."""
    toks = np.asarray(tokens, dtype=np.int64)
    grps = np.asarray(q_labels)[toks].astype(np.int64)
    return Probes(toks, grps, np.ones(toks.size), None)


def ridge_only_fit(q, k, v, scale, probes: Probes, q_labels, k_labels, kept, p: Params):
    """Ridge without the rank-r projection: the correction of a row is
    ybar + (o - xbar) W with the full weighted ridge map W = Xt^T Z,
    Z = (Xt Xt^T + lambda I_M)^{-1} Yt.  Factored through the M probes as A = Xt^T [d, M],
    B = Z [M, d] (so A B = W) and c0 = ybar - xbar A B, the same form the projected fit
    is applied in."""
    od, os_, R, _, _ = probe_rows(q, k, v, scale, probes.tokens, q_labels, k_labels, kept)
    xbar, ybar, Xt, Yt = weighted_center(os_, R, probes.weights)
    Z = np.linalg.solve(Xt @ Xt.T + p.lam * np.eye(Xt.shape[0]), Yt)
    A = Xt.T
    B = Z
    c0 = ybar - xbar @ A @ B
    return Fit(A, B, c0, A @ B, xbar, ybar, None, np.zeros(p.rank + 1), od, os_, R)


# --------------------------------------------------------------------------------------
# whole call
# --------------------------------------------------------------------------------------
@dataclass
class KVHeadResult:
    part: Partition
    route: Route
    probes: Probes
    fits: list          # one Fit per query head
    o: np.ndarray       # [g, N, d] token order (None when rows were sampled)


def sparsepr_kv_head(q_heads, k, v, p: Params, S=None, U=None, with_output=True,
                     part=None, route_=None, probes=None):
    """The whole SparsePR call for one KV head and its g query heads.  Intermediate
    stages may be supplied (e.g. the GPU's labels, CSR and probes) to check the float
    stages on identical integer decisions."""
    q_heads, k, v = f64(q_heads), f64(k), f64(v)
    n, d = k.shape
    scale = p.softmax_scale(d)
    if part is None:
        part = partition(q_heads, k, p, S=S, U=U)
    if route_ is None:
        route_ = route(part, p, n)
    if probes is None:
        probes = select_probes(part.xq, part.q_labels, part.q_centroids,
                               np.diff(part.q_offsets), p.n_probe)
    fits, outs = [], []
    for j in range(q_heads.shape[0]):
        fit = probe_fit(q_heads[j], k, v, scale, probes, part.q_labels, part.k_labels,
                        route_.kept, p)
        fits.append(fit)
        if with_output:
            os_, _ = sparse_attention(q_heads[j], k, v, scale, part.q_labels, part.k_labels,
                                      route_.kept)
            outs.append(apply_correction(os_, fit, probes.tokens))
    return KVHeadResult(part, route_, probes, fits, np.stack(outs) if with_output else None)


def executed_pairs(route_: Route, n, n_probe):
    """Executed pairs per head: routed (unpadded) pairs plus the probe rows."""
    return route_.pairs + n_probe * n
