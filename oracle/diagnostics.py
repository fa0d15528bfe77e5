"""Attention-support and residual statistics (test infrastructure only; see
oracle/sparsepr.py).

The support paragraph of the summary page of "Partition the Support, Reconstruct the
Residual" measures how many keys a single query row needs to keep 90 % of its attention
mass and how much that grows when several queries share one route; its partition
paragraph measures how much of the hard-drop residual is an affine function of the sparse
output.  Each function here writes out one of those definitions in float64.
"""
import numpy as np

from .sparsepr import f64


def support_rows(n, count=256):
    """Evenly spaced rows floor((2r+1) N / (2 count))."""
    r = np.arange(min(count, n))
    return (2 * r + 1) * n // (2 * r.size)


def row_supports(q, k, scale, rows, mass=0.9):
    """The 90 %-mass support of single query rows (summary page of "Partition the Support,
    Reconstruct the Residual", support paragraph): for each row, the fewest keys whose
    softmax probabilities sum to at least ``mass``, taken in order of decreasing probability
    with ties broken by the smaller key index.  Returns (count per row [R] int64, member mask
    [R, N] bool); float64 throughout."""
    q, k = f64(q)[np.asarray(rows)], f64(k)
    s = (q @ k.T) * scale
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    n = k.shape[0]
    count = np.empty(p.shape[0], dtype=np.int64)
    member = np.zeros(p.shape, dtype=bool)
    for r in range(p.shape[0]):
        order = np.lexsort((np.arange(n), -p[r]))
        c = np.cumsum(p[r][order])
        need = int((c < mass).sum()) + 1
        count[r] = min(need, n)
        member[r, order[:count[r]]] = True
    return count, member


def supports_from_scores(scores, scale, mass=0.9):
    """The same support definition with each key's probability taken as an integer mass,
    decided in double precision from given float32 scores f (e.g. another implementation's):
    m = floor(2^40 exp((f - f_max) scale)) with the difference and product as float64
    operations; the target is min(ceil(mass * S), S) with S = sum m as a float64, at least 1;
    keys by decreasing score, ties by the smaller index, and the count is the shortest
    prefix whose integer sum reaches the target.  ``scores`` [R, N]; returns (count per row
    [R] int64, member mask [R, N] bool)."""
    f = np.asarray(scores, dtype=np.float32)
    count = np.empty(f.shape[0], dtype=np.int64)
    member = np.zeros(f.shape, dtype=bool)
    n = f.shape[1]
    for r in range(f.shape[0]):
        fr = f[r].astype(np.float64) + 0.0          # -0 and +0 are one score
        x = (fr - fr.max()) * float(np.float32(scale))
        m = np.floor(np.ldexp(np.exp(x), 40)).astype(np.int64)
        total = int(m.sum())
        want = float(np.ceil(float(total) * mass))
        tgt = total if want >= float(total) else int(want)
        tgt = max(tgt, 1)
        order = np.lexsort((np.arange(n), -fr))
        c = np.cumsum(m[order])
        k = int(np.searchsorted(c, tgt, side="left")) + 1
        count[r] = min(k, n)
        member[r, order[:count[r]]] = True
    return count, member


def shared_supports(q, k, scale, sets, mass=0.9):
    """Queries that share one route must keep the union of their single-row supports (same
    paragraph: eight queries per route).  ``sets`` [S, s] holds token indices; returns
    (count per row [S, s], union size per set [S]) as int64."""
    sets = np.asarray(sets)
    count, member = row_supports(q, k, scale, sets.reshape(-1), mass)
    union = member.reshape(sets.shape[0], sets.shape[1], -1).any(axis=1).sum(axis=1)
    return count.reshape(sets.shape), union.astype(np.int64)


def support_fraction(q, k, scale, rows, mass=0.9):
    """Per row: the single-row support as a fraction of N (float64).  The page reports
    medians of 6.2 % (Wan2.2) and 56.5 % (Cosmos-Predict2.5); the synthetic workloads are
    shaped to span that range."""
    return row_supports(q, k, scale, rows, mass)[0] / f64(k).shape[0]


def median_support(q, k, scale, count=256, mass=0.9):
    return float(np.median(support_fraction(q, k, scale, support_rows(k.shape[0], count), mass)))


def affine_residual_stats(o_sparse, o_dense):
    """How much of the hard-drop residual R = O_dense - O_sparse is an affine function of
    the sparse output, over every row of one query head (the page's partition paragraph
    reports this share, and the energy orthogonal to it, for its oracle diagnostic).

    Reading: ordinary least squares R ~ c + O_sparse W over all n rows (unweighted, no
    penalty).  Returns (||R||_F^2, ||R - mean R||_F^2, ||R - (c + O_sparse W)||_F^2,
    explainable fraction = 1 - third / second)."""
    X = f64(o_sparse)
    R = f64(o_dense) - X
    Xa = np.hstack([X, np.ones((X.shape[0], 1))])
    coef = np.linalg.lstsq(Xa, R, rcond=None)[0]
    res = R - Xa @ coef
    tot = float((R * R).sum())
    cen = float(((R - R.mean(axis=0)) ** 2).sum())
    orth = float((res * res).sum())
    return tot, cen, orth, 1.0 - orth / cen if cen > 0 else 0.0
