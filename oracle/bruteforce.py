"""Brute-force MoGE routing for tiny inputs (NumPy only, independent of moge_oracle.c).

TEST INFRASTRUCTURE (see the oracle package header).

Reading of the method (Pangu Pro MoE pages: lsdiaocha.cn summary, section 1; hyper.ai
abstract): a token must activate the same number K' of experts in every one of the M
equal groups, and the gate of an expert is its probability under a softmax over all N
experts.  Among all such balanced selections, the router keeps the K' most probable
experts of each group, i.e. the balanced selection of largest total probability.  This
module finds that selection by enumerating every balanced selection, which checks the
oracle's per-group rank rule from a different angle (an optimisation over subsets rather
than a per-expert rank count).
"""
from __future__ import annotations

import itertools

import numpy as np


def softmax64(lg: np.ndarray) -> np.ndarray:
    z = lg.astype(np.float64)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def balanced_selections(N: int, M: int, Kp: int):
    """Every selection with exactly Kp experts from each of the M contiguous groups of N/M experts."""
    G = N // M
    per_group = [list(itertools.combinations(range(g * G, (g + 1) * G), Kp)) for g in range(M)]
    for combo in itertools.product(*per_group):
        yield tuple(e for grp in combo for e in grp)


def route_bruteforce(lg: np.ndarray, M: int, Kp: int, tol: float = 1e-12) -> np.ndarray:
    """For each token, the balanced selection with the largest total softmax mass; among selections
    within ``tol`` of the best, the one whose sorted expert tuple is lexicographically smallest
    (equal scores go to lower expert ids).  Returns sorted expert ids [T, M*Kp]."""
    T, N = lg.shape
    p = softmax64(lg)
    sels = list(balanced_selections(N, M, Kp))
    out = np.empty((T, M * Kp), dtype=np.int64)
    for t in range(T):
        masses = np.array([p[t, list(s)].sum() for s in sels])
        best = masses.max()
        cands = sorted(s for s, m in zip(sels, masses) if m >= best - tol)
        out[t] = cands[0]
    return out


def global_topk_argsort(lg: np.ndarray, K: int) -> np.ndarray:
    """Global top-K by a stable sort of the negated scores: equal scores keep ascending expert order."""
    return np.argsort(-lg.astype(np.float64), axis=1, kind="stable")[:, :K]
