"""Pins for the oracle's dispatch (counts, offsets, stable permutation) and imbalance score.

Fixed by library routines (NumPy bincount / cumsum / stable argsort) and closed forms, not by the oracle."""
import numpy as np
import pytest

import oracle


def _random_idx(rng, T, N, M, Kp):
    lg = (rng.standard_normal((T, N)) + rng.standard_normal(N) * 2).astype(np.float32)
    idx, _, _ = oracle.route(lg, M, Kp, "grouped")
    return idx


@pytest.mark.parametrize("T,N,M,Kp", [(64, 8, 4, 1), (257, 64, 8, 2), (1000, 256, 8, 1), (1, 8, 4, 2)])
def test_dispatch_matches_stable_argsort(T, N, M, Kp):
    rng = np.random.default_rng(T + N)
    idx = _random_idx(rng, T, N, M, Kp)
    counts, offsets, inv, perm = oracle.dispatch(idx, N)
    flat = idx.ravel()
    assert (counts == np.bincount(flat, minlength=N)).all()
    assert (offsets == np.concatenate([[0], np.cumsum(counts)])).all()
    order = np.argsort(flat, kind="stable")            # global row r holds flat entry order[r]
    K = idx.shape[1]
    assert (perm == order // K).all()
    rows = np.empty_like(order)
    rows[order] = np.arange(order.size)
    assert (inv.ravel() == rows).all()


@pytest.mark.parametrize("e_lo,e_hi", [(0, 8), (8, 16), (5, 13), (63, 64), (0, 64)])
def test_dispatch_expert_range(e_lo, e_hi):
    rng = np.random.default_rng(7)
    idx = _random_idx(rng, 300, 64, 8, 1)
    counts, offsets, inv, perm = oracle.dispatch(idx, 64, e_lo, e_hi)
    full_c, full_o, full_inv, full_perm = oracle.dispatch(idx, 64)
    assert (counts == full_c).all() and (offsets == full_o).all()
    inr = (idx >= e_lo) & (idx < e_hi)
    assert (inv[~inr] == -1).all()
    assert (inv[inr] == full_inv[inr] - full_o[e_lo]).all()
    assert (perm == full_perm[full_o[e_lo]:full_o[e_hi]]).all()
    assert perm.size == inr.sum()


def test_group_range_load_is_exact_under_skew():
    # one device's share: group 0's rows are exactly T*K' whatever the skew
    rng = np.random.default_rng(3)
    T, N, M, Kp = 4096, 64, 8, 1
    lg = (rng.standard_normal((T, N)) + np.where(np.arange(N) < 8, -6.0, 3.0)).astype(np.float32)
    idx, _, _ = oracle.route(lg, M, Kp, "grouped")
    counts, offsets, inv, perm = oracle.dispatch(idx, N, 0, 8)
    assert perm.size == T * Kp
    assert (np.sort(perm) == np.arange(T)).all()


def test_imbalance_closed_form():
    counts = np.array([5, 0, 3, 3, 10, 1, 0, 0], dtype=np.int32)
    gl, isr = oracle.imbalance(counts, 4)
    assert gl.tolist() == [5, 6, 11, 0] and isr == 11
    gl, isr = oracle.imbalance(counts, 1)
    assert gl.tolist() == [22] and isr == 0
