"""GPU parity: moge_route (and dispatch's counts/offsets) through the C ABI against the oracle.

Bar: on oracle-supplied binary32 scores the chosen experts, per-expert counts and offsets are
bit-exact (ties -> lower expert id) and gates match the oracle's binary64 softmax to
|d| <= 1e-5 * gate + 1e-8.  From x, routing may differ only on near-tie tokens."""
import dataclasses

import numpy as np
import pytest
import torch

import mixture_grouped_experts_amd as moge
import oracle
import synth
from synth import workloads as W
from tests import moge_harness as H

pytestmark = pytest.mark.gpu


def _route_dev(w, lg_np=None, x=None, wr=None, bias=None, mode=moge.ROUTE_GROUPED, store_logits=False):
    s = moge.Shape(w.T, w.d, w.N, w.M, w.Kp, w.F, moge.BF16 if w.dtype == "bf16" else moge.F32)
    K = w.K
    idx = torch.full((w.T, K), -7, dtype=torch.int32, device="cuda")
    gate = torch.full((w.T, K), -1.0, dtype=torch.float32, device="cuda")
    if lg_np is not None:
        lg = torch.from_numpy(lg_np).cuda()
        moge.route(s, mode, None, None, None, lg, idx, gate)
    else:
        lg = torch.empty(w.T, w.N, dtype=torch.float32, device="cuda") if store_logits else None
        moge.route(s, mode, x, wr, bias, lg, idx, gate)
    torch.cuda.synchronize()
    return s, idx.cpu().numpy(), gate.cpu().numpy(), (lg.cpu().numpy() if lg is not None else None)


def _counts_dev(s, idx_np, mode):
    idx = torch.from_numpy(idx_np).cuda()
    counts = torch.full((s.N,), -1, dtype=torch.int32, device="cuda")
    offsets = torch.full((s.N + 1,), -1, dtype=torch.int32, device="cuda")
    ws = torch.empty(moge.workspace_size(s), dtype=torch.uint8, device="cuda")
    moge.dispatch(s, mode, idx, None, 0, s.N, 0, counts, offsets, None, None, None, ws)
    torch.cuda.synchronize()
    return counts.cpu().numpy(), offsets.cpu().numpy()


def test_synth_device_matches_host(gpu):
    for bf16, n, start, std in ((True, 100003, 0, 0.02), (False, 4099, 12345678, 2.0)):
        t = torch.empty(n, dtype=torch.bfloat16 if bf16 else torch.float32, device="cuda")
        synth.fill_device(t, 0, 5, std, start)
        host = synth.normal_host(0, 5, n, std, bf16, start)
        dev = t.view(torch.int16).cpu().numpy().view(np.uint16) if bf16 else t.cpu().numpy()
        assert (dev.view(np.uint8) == host.view(np.uint8)).all()


WORKLOADS = [W.tiny(), W.routing(), W.decode(), W.ultra()]


@pytest.mark.parametrize("w", WORKLOADS, ids=lambda w: w.name)
def test_route_on_oracle_scores_bitexact(gpu, w):
    print(f"[route logits-in] {w.name}", flush=True)
    h = H.HostInputs(w)
    lg = H.oracle_logits_all(h)
    for mode, omode in ((moge.ROUTE_GROUPED, "grouped"), (moge.ROUTE_GLOBAL, "global")):
        s, idx, gate, _ = _route_dev(w, lg_np=lg, mode=mode)
        ridx, rgate, _ = oracle.route(lg, w.M, w.Kp, omode)
        assert (idx == ridx).all(), f"{omode}: {(idx != ridx).any(1).sum()} tokens differ"
        assert (np.abs(gate - rgate) <= 1e-5 * rgate + 1e-8).all()
        counts, offsets = _counts_dev(s, idx, mode)
        rc, ro, _, _ = oracle.dispatch(ridx, w.N)
        assert (counts == rc).all() and (offsets == ro).all()
        gl, isr = oracle.imbalance(rc, w.M)
        if omode == "grouped":
            assert isr == 0 and (gl == w.T * w.Kp).all()


@pytest.mark.parametrize("w", WORKLOADS, ids=lambda w: w.name)
def test_route_from_x(gpu, w):
    print(f"[route from x] {w.name}", flush=True)
    h = H.HostInputs(w)
    lg_ref = H.oracle_logits_all(h)
    d = H.device_inputs(w)
    _, idx, gate, lg = _route_dev(w, x=d.x, wr=d.w_router, bias=d.bias, store_logits=True)
    # scores: float32 accumulation vs the oracle's binary64 sum rounded once
    scale = 1.0 + np.abs(lg_ref).max()
    assert np.abs(lg - lg_ref).max() <= 1e-4 * scale
    ridx, rgate, rgap = oracle.route(lg_ref, w.M, w.Kp, "grouped")
    n_near, flipped, hard = H.compare_routing(w, idx, ridx, rgap)
    print(f"  near-tie tokens {n_near}, flipped {len(flipped)}", flush=True)
    assert hard.size == 0, f"{hard.size} non-near-tie tokens routed differently"
    same = np.all(idx == ridx, axis=1)
    assert (np.abs(gate[same] - rgate[same]) <= 1e-4 * rgate[same] + 1e-7).all()


def test_route_ties_and_edge_shapes(gpu):
    rng = np.random.default_rng(0)
    cases = [(1, 8, 4, 1), (33, 64, 8, 2), (100, 16, 1, 5), (70, 12, 3, 4), (129, 256, 8, 1), (64, 256, 4, 8),
             (65, 128, 2, 3), (77, 15, 5, 2), (40, 6, 3, 1), (200, 250, 5, 7)]    # (N not a multiple of 4)
    for T, N, M, Kp in cases:
        w = W.variant(W.routing(), T=T, N=N, M=M, Kp=Kp)
        lg = rng.integers(-2, 3, size=(T, N)).astype(np.float32)        # heavy ties
        lg[::3] = (rng.standard_normal((len(lg[::3]), N)) * 2).astype(np.float32)
        lg[1::5] = 0.0
        lg[2::7] *= -0.0                                                # -0 and +0 compare equal
        for mode, omode in ((moge.ROUTE_GROUPED, "grouped"), (moge.ROUTE_GLOBAL, "global")):
            _, idx, gate, _ = _route_dev(w, lg_np=lg, mode=mode)
            ridx, rgate, _ = oracle.route(lg, M, Kp, omode)
            assert (idx == ridx).all(), (T, N, M, Kp, omode)
            assert (np.abs(gate - rgate) <= 1e-5 * rgate + 1e-8).all()


@pytest.mark.parametrize("N,M,Kp,d,store", [(64, 8, 1, 4096, True), (128, 4, 2, 1024, True), (256, 8, 1, 7680, True),
                                            (64, 8, 8, 520, True), (256, 8, 1, 7680, False), (192, 8, 2, 200, True),
                                            (256, 4, 1, 264, False)])
def test_route_from_x_shapes(gpu, N, M, Kp, d, store):
    # other expert counts (one, two and four 64-expert column groups; above 128 the stored-scores path
    # splits the experts in halves over the XCDs and chooses in a second pass, the other path keeps the
    # whole score row in one workgroup), ragged hidden sizes
    w = W.variant(W.decode(), T=300, d=d, N=N, M=M, Kp=Kp, std_bias=1.0)
    h = H.HostInputs(w)
    lg_ref = H.oracle_logits_all(h)
    dv = H.device_inputs(w)
    _, idx, gate, lg = _route_dev(w, x=dv.x, wr=dv.w_router, bias=dv.bias, store_logits=store)
    if store:
        assert np.abs(lg - lg_ref).max() <= 1e-4 * (1.0 + np.abs(lg_ref).max())
    ridx, _, rgap = oracle.route(lg_ref, M, Kp, "grouped")
    _, _, hard = H.compare_routing(w, idx, ridx, rgap)
    assert hard.size == 0
