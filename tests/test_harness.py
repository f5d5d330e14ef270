"""Host logic of the GPU tests' routing comparison (no GPU)."""
import numpy as np

from synth import workloads as W
from tests import moge_harness as H


def _w(N, M, Kp):
    return W.variant(W.decode(), T=2, N=N, M=M, Kp=Kp)


def test_order_gap_against_a_direct_sort():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((5, 12)).astype(np.float32)
    got = H.order_gap(lg, 3, 2)
    for t in range(5):
        p = np.exp(lg[t].astype(np.float64) - lg[t].max())
        p /= p.sum()
        gaps = []
        for g in range(3):
            q = sorted(p[4 * g:4 * g + 4], reverse=True)[:3]
            gaps += [q[0] - q[1], q[1] - q[2]]
        assert abs(got[t] - min(gaps)) <= 1e-15
    # global mode: one group of all experts, K = M K' = 6 ranks and the 7th
    glob = H.order_gap(lg, 3, 2, "global")
    p = np.exp(lg[0].astype(np.float64) - lg[0].max())
    q = np.sort(p / p.sum())[::-1][:7]
    assert abs(glob[0] - (q[:-1] - q[1:]).min()) <= 1e-15
    assert np.isinf(H.order_gap(lg[:, :3], 3, 1)).all()   # one expert per group: no order to get wrong


def test_compare_routing_order_swaps():
    w = _w(8, 2, 2)
    ref = np.array([[1, 0, 5, 6], [2, 3, 4, 7]], dtype=np.int32)
    big = np.array([1.0, 1.0])
    swap = np.array([[0, 1, 5, 6], [2, 3, 4, 7]], dtype=np.int32)      # same experts, other order
    other = np.array([[1, 2, 5, 6], [2, 3, 4, 7]], dtype=np.int32)     # another expert chosen
    # an order swap is accepted only on an order near-tie, a different expert only on a boundary near-tie
    assert H.compare_routing(w, swap, ref, big)[2].tolist() == [0]
    assert H.compare_routing(w, swap, ref, big, np.array([1e-9, 1.0]))[1].tolist() == [0]
    assert H.compare_routing(w, swap, ref, big, np.array([1e-3, 1.0]))[2].tolist() == [0]
    assert H.compare_routing(w, other, ref, big, np.array([1e-9, 1.0]))[2].tolist() == [0]
    assert H.compare_routing(w, other, ref, np.array([1e-9, 1.0]), np.array([1.0, 1.0]))[1].tolist() == [0]
