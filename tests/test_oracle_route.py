"""Pins for the oracle's router: scores -> global softmax -> top-K' per group (and the global top-K comparator).

What fixes the answer here is not the oracle itself:
* hand-derived cases (tests/golden/route_hand_example.json, cited there);
* closed forms (equal scores; scores ln(k) give probabilities k / sum k);
* library routines (SciPy softmax; NumPy stable argsort for the M=1 case, where MoGE is global top-K);
* brute-force enumeration of every balanced selection (oracle/bruteforce.py) on tiny inputs;
* invariants the pages state: K' experts in every group, imbalance 0 for MoGE, global top-K imbalance
  usually positive on skewed scores, no two experts of one group co-activated when K' = 1.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import bruteforce
import synth
from synth import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden", "route_hand_example.json")


def _load_cases():
    with open(GOLD) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _load_cases(), ids=lambda c: c["name"])
def test_hand_examples(case):
    M, Kp = case["M"], case["Kp"]
    if "equal_T" in case:
        lg = np.zeros((case["equal_T"], case["N"]), dtype=np.float32)
        moge_idx = np.tile(case["moge_idx_row"], (case["equal_T"], 1))
        glob_idx = np.tile(case["global_idx_row"], (case["equal_T"], 1))
    else:
        lg = np.array(case["logits"], dtype=np.float32)
        moge_idx = np.array(case["moge_idx"])
        glob_idx = np.array(case["global_idx"])
    N = lg.shape[1]
    idx, gate, _ = oracle.route(lg, M, Kp, "grouped")
    assert (idx == moge_idx).all()
    gidx, ggate, _ = oracle.route(lg, M, Kp, "global")
    assert (gidx == glob_idx).all()
    counts = np.bincount(idx.ravel(), minlength=N)
    gl, isr = oracle.imbalance(counts, M)
    assert gl.tolist() == case["moge_group_load"] and isr == case["moge_is_raw"]
    gcounts = np.bincount(gidx.ravel(), minlength=N)
    gl, isr = oracle.imbalance(gcounts, M)
    assert gl.tolist() == case["global_group_load"] and isr == case["global_is_raw"]
    if "gate_each" in case:
        assert np.all(gate == case["gate_each"]) and np.all(ggate == case["gate_each"])


def test_softmax_closed_form_rational():
    # scores ln(k): the global softmax is k / sum(k) (to binary32 rounding of ln k)
    k = np.arange(1, 9, dtype=np.float64)
    lg = np.log(k).astype(np.float32)[None, :]
    idx, gate, _ = oracle.route(lg, 4, 2, "grouped")      # K' = group size: every expert chosen
    p = np.zeros(8)
    p[idx[0]] = gate[0]
    assert np.allclose(p, k / k.sum(), rtol=2e-7, atol=0)
    assert abs(gate.sum() - 1.0) < 1e-15


def test_gates_are_global_softmax_scipy():
    rng = np.random.default_rng(1)
    lg = (rng.standard_normal((200, 64)) * 3).astype(np.float32)
    idx, gate, _ = oracle.route(lg, 8, 1, "grouped")
    ref = scipy.special.softmax(lg.astype(np.float64), axis=1)
    assert np.allclose(gate, np.take_along_axis(ref, idx, 1), rtol=1e-14, atol=0)
    # not renormalised over the chosen experts
    assert (gate.sum(1) < 1.0).all()


@pytest.mark.parametrize("N,K", [(8, 4), (64, 8), (16, 3)])
def test_single_group_is_stable_argsort(N, K):
    rng = np.random.default_rng(N * 10 + K)
    lg = rng.integers(-3, 4, size=(300, N)).astype(np.float32)   # many planted ties
    for mode, M, Kp in (("grouped", 1, K), ("global", 1, K)):
        idx, _, _ = oracle.route(lg, M, Kp, mode)
        assert (idx == bruteforce.global_topk_argsort(lg, K)).all()


@pytest.mark.parametrize("N,M,Kp", [(8, 4, 1), (8, 4, 2), (8, 2, 2), (12, 3, 2), (6, 2, 1)])
def test_bruteforce_balanced_selection(N, M, Kp):
    rng = np.random.default_rng(N + 100 * M + 1000 * Kp)
    lg = rng.standard_normal((64, N)).astype(np.float32)
    lg[::7] = np.round(lg[::7])                             # plant ties on some tokens
    idx, _, _ = oracle.route(lg, M, Kp, "grouped")
    assert (np.sort(idx, 1) == bruteforce.route_bruteforce(lg, M, Kp)).all()


def test_slot_order_group_major_then_rank():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((100, 16)).astype(np.float32)
    idx, gate, _ = oracle.route(lg, 4, 2, "grouped")
    G = 4
    for t in range(100):
        for g in range(4):
            a, b = idx[t, 2 * g], idx[t, 2 * g + 1]
            assert a // G == g and b // G == g
            assert lg[t, a] > lg[t, b] or (lg[t, a] == lg[t, b] and a < b)
            assert gate[t, 2 * g] >= gate[t, 2 * g + 1]


def _tiny_logits():
    w = W.tiny()
    x = synth.normal_host(w.seed, W.TID_X, w.T * w.d, w.std_x, bf16=False).reshape(w.T, w.d)
    wr = synth.normal_host(w.seed, W.TID_WROUTER, w.N * w.d, w.std_router, bf16=False).reshape(w.N, w.d)
    return w, oracle.logits(x, wr)


def test_tiny_config_imbalance():
    # MoGE: imbalance exactly 0; the global top-4 baseline on the same scores: > 0 (seed 0)
    w, lg = _tiny_logits()
    idx, _, _ = oracle.route(lg, w.M, w.Kp, "grouped")
    gidx, _, _ = oracle.route(lg, w.M, w.Kp, "global")
    gl, isr = oracle.imbalance(np.bincount(idx.ravel(), minlength=w.N), w.M)
    assert isr == 0 and (gl == w.T * w.Kp).all()
    _, gisr = oracle.imbalance(np.bincount(gidx.ravel(), minlength=w.N), w.M)
    assert gisr > 0


def test_invariants_and_mass_order_random():
    rng = np.random.default_rng(11)
    for (N, M, Kp) in ((64, 8, 1), (64, 8, 2), (256, 8, 1), (32, 4, 3)):
        lg = (rng.standard_normal((500, N)) + rng.standard_normal(N) * 2).astype(np.float32)
        idx, gate, _ = oracle.route(lg, M, Kp, "grouped")
        gidx, ggate, _ = oracle.route(lg, M, Kp, "global")
        G = N // M
        grp = idx // G
        for g in range(M):
            assert ((grp == g).sum(1) == Kp).all()          # exactly K' per group
        assert all(len(set(r)) == M * Kp for r in idx)      # no expert twice
        if Kp == 1:                                          # no co-activation inside a group
            assert (np.sort(grp, 1) == np.arange(M)).all()
        # global top-K maximises selected mass over all K-subsets, MoGE over balanced ones
        assert (gate.sum(1) <= ggate.sum(1) + 1e-12).all()
        _, isr = oracle.imbalance(np.bincount(idx.ravel(), minlength=N), M)
        assert isr == 0


def test_routing_workload_sample_global_baseline_positive():
    # skewed scores (bias ~ N(0,2)) on a sample of the 65536-token routing workload
    w = W.routing()
    Ts = 512
    x = synth.normal_host(w.seed, W.TID_X, Ts * w.d, w.std_x, bf16=True).reshape(Ts, w.d)
    wr = synth.normal_host(w.seed, W.TID_WROUTER, w.N * w.d, w.std_router, bf16=True).reshape(w.N, w.d)
    b = synth.normal_host(w.seed, W.TID_BIAS, w.N, w.std_bias, bf16=False)
    lg = oracle.logits(x, wr, b)
    idx, _, _ = oracle.route(lg, w.M, w.Kp, "grouped")
    gidx, _, _ = oracle.route(lg, w.M, w.Kp, "global")
    _, isr = oracle.imbalance(np.bincount(idx.ravel(), minlength=w.N), w.M)
    _, gisr = oracle.imbalance(np.bincount(gidx.ravel(), minlength=w.N), w.M)
    assert isr == 0 and gisr > 0


def test_near_tie_gap():
    # group 0: probabilities of rank 0 and rank 1 differ by exactly what we plant
    lg = np.array([[1.0, 1.0, 0.0, -1.0], [2.0, 0.0, 0.5, -0.5]], dtype=np.float32)
    _, _, gap = oracle.route(lg, 2, 1, "grouped")
    assert gap[0] == 0.0                                    # exact tie in group 0
    p = scipy.special.softmax(lg[1].astype(np.float64))
    assert math.isclose(gap[1], min(p[0] - p[1], p[2] - p[3]), rel_tol=1e-12, abs_tol=1e-15)
    _, _, gap_full = oracle.route(lg, 2, 2, "grouped")       # K' = group size: no runner-up
    assert np.isinf(gap_full).all()
