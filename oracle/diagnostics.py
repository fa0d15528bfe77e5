"""Attention-support statistics (test infrastructure only; see oracle/sparsepr.py).

The PSRR support paragraph measures how many keys a single query row needs to keep
90 % of its attention mass (median 6.2 % on Wan2.2, 56.5 % on Cosmos-Predict2.5) and how
that grows when queries share a route.  The synthetic workloads are calibrated to those
single-row medians with ``support_fraction``.
"""
import numpy as np

from .sparsepr import f64


def support_rows(n, count=256):
    """Evenly spaced rows floor((2r+1) N / (2 count))."""
    r = np.arange(min(count, n))
    return (2 * r + 1) * n // (2 * r.size)


def support_fraction(q, k, scale, rows, mass=0.9):
    """Per row: the smallest number of keys whose softmax mass reaches ``mass``,
    as a fraction of N (float64)."""
    q, k = f64(q)[np.asarray(rows)], f64(k)
    s = (q @ k.T) * scale
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    p = -np.sort(-p, axis=1)
    c = np.cumsum(p, axis=1)
    need = (c < mass).sum(axis=1) + 1
    return need / k.shape[0]


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
