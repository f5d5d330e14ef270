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
    nws = moge.workspace_size(s, moge.STAGE_ROUTE)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
    if lg_np is not None:
        lg = torch.from_numpy(lg_np).cuda()
        moge.route(s, mode, None, None, None, lg, idx, gate)
    else:
        lg = torch.empty(w.T, w.N, dtype=torch.float32, device="cuda") if store_logits else None
        moge.route(s, mode, x, wr, bias, lg, idx, gate, ws)
    torch.cuda.synchronize()
    return s, idx.cpu().numpy(), gate.cpu().numpy(), (lg.cpu().numpy() if lg is not None else None)


def _route_pair_dev(w, lg_np=None, x=None, wr=None, bias=None):
    """moge_route_pair: both routers from one pass; returns (idx, gate, gidx, ggate)."""
    s = moge.Shape(w.T, w.d, w.N, w.M, w.Kp, w.F, moge.BF16 if w.dtype == "bf16" else moge.F32)
    K = w.K
    outs = [torch.full((w.T, K), -7, dtype=torch.int32, device="cuda"),
            torch.full((w.T, K), -1.0, dtype=torch.float32, device="cuda"),
            torch.full((w.T, K), -7, dtype=torch.int32, device="cuda"),
            torch.full((w.T, K), -1.0, dtype=torch.float32, device="cuda")]
    nws = moge.workspace_size(s, moge.STAGE_ROUTE)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
    if lg_np is not None:
        moge.route_pair(s, None, None, None, torch.from_numpy(lg_np).cuda(), *outs)
    else:
        moge.route_pair(s, x, wr, bias, None, *outs, ws)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


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
    pair = _route_pair_dev(w, lg_np=lg)
    for mode, omode in ((moge.ROUTE_GROUPED, "grouped"), (moge.ROUTE_GLOBAL, "global")):
        s, idx, gate, _ = _route_dev(w, lg_np=lg, mode=mode)
        ridx, rgate, _ = oracle.route(lg, w.M, w.Kp, omode)
        pi, pg = pair[0:2] if omode == "grouped" else pair[2:4]
        assert (pi == ridx).all() and (np.abs(pg - rgate) <= 1e-5 * rgate + 1e-8).all()
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
    # both routers from one pass give exactly the grouped router's choice and, on the global
    # side, the choice the global router makes on the same stored scores
    pidx, pgate, pgidx, pggate = _route_pair_dev(w, x=d.x, wr=d.w_router, bias=d.bias)
    _, gidx, ggate, _ = _route_dev(w, lg_np=lg, mode=moge.ROUTE_GLOBAL)
    def _same(a, b, ga, gb, what):
        bad = np.nonzero((a != b).any(1) | (ga != gb).any(1))[0]
        assert bad.size == 0, (f"{what}: {bad.size} tokens differ, e.g. token {bad[0]}: {a[bad[0]]} {b[bad[0]]} "
                               f"{ga[bad[0]]} {gb[bad[0]]}")
    _same(pidx, idx, pgate, gate, "pair vs grouped")
    _same(pgidx, gidx, pggate, ggate, "pair vs global")
    # scores: float32 accumulation vs the oracle's binary64 sum rounded once
    scale = 1.0 + np.abs(lg_ref).max()
    assert np.abs(lg - lg_ref).max() <= 1e-4 * scale
    ridx, rgate, rgap = oracle.route(lg_ref, w.M, w.Kp, "grouped")
    n_near, flipped, hard = H.compare_routing(w, idx, ridx, rgap, H.order_gap(lg_ref, w.M, w.Kp))
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
    # other expert counts (one, two and four 64-expert column groups; 300 tokens take the router split
    # over slices of d, whose partial sums are added in a second pass that also makes the choice),
    # ragged hidden sizes
    w = W.variant(W.decode(), T=300, d=d, N=N, M=M, Kp=Kp, std_bias=1.0)
    h = H.HostInputs(w)
    lg_ref = H.oracle_logits_all(h)
    dv = H.device_inputs(w)
    _, idx, gate, lg = _route_dev(w, x=dv.x, wr=dv.w_router, bias=dv.bias, store_logits=store)
    if store:
        assert np.abs(lg - lg_ref).max() <= 1e-4 * (1.0 + np.abs(lg_ref).max())
    ridx, _, rgap = oracle.route(lg_ref, M, Kp, "grouped")
    _, _, hard = H.compare_routing(w, idx, ridx, rgap, H.order_gap(lg_ref, M, Kp))
    assert hard.size == 0


def _int_operands(T, d, N, seed, f32=False, zero_rows=()):
    """x in {-2..2}, router rows in {-1, 0, 1}, an integer bias with -0 and +0: every score is an
    exact integer (|score| <= 2 d + 3) whatever the order of the float32 sums, so experts tie
    exactly and often.  Returns device tensors and the oracle's host copies (same values)."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randint(-2, 3, (T, d), generator=g).float()
    x[list(zero_rows)] = 0.0                                    # these tokens score the bias alone
    wr = torch.randint(-1, 2, (N, d), generator=g).float()
    bias = torch.randint(-3, 4, (N,), generator=g).float()
    bias[(bias == 0) & (torch.arange(N) % 2 == 1)] = -0.0      # half the zero biases are -0
    dt = torch.float32 if f32 else torch.bfloat16
    xd, wd = x.to(dt).cuda(), wr.to(dt).cuda()

    def host(t):
        return t.numpy() if f32 else t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return xd, wd, bias.cuda(), host(x), host(wr), bias.numpy()


# (T, d, N, M, Kp, dtype, store): every router path -- the one-pass kernel whole (token tiles
# that fill the CUs, or d < 128) and in slices of d (2, 8 and 16 slices, with ragged tails of d
# in the last slice) with the reduction that makes the choice (rank count at
# N <= 64, the lists above), the 256-expert split kernel, the float32 kernel -- with the
# sorting-network choice (groups of 8), the list choice (other groups: 8, 16, 32 experts at
# N = 128 and 256), both routers
TIE_CASES = [(300, 128, 64, 8, 1, "bf16", True), (300, 128, 64, 8, 2, "bf16", False),
             (32832, 128, 64, 8, 1, "bf16", True), (32832, 64, 64, 8, 2, "bf16", False),
             (300, 128, 128, 4, 2, "bf16", True), (32832, 64, 128, 4, 2, "bf16", False),
             (520, 128, 256, 8, 1, "bf16", True), (520, 128, 256, 8, 1, "bf16", False),
             (300, 96, 16, 4, 1, "bf16", True), (64, 128, 8, 4, 1, "f32", True),
             (5000, 64, 64, 8, 1, "bf16", False), (5000, 64, 128, 4, 2, "bf16", True),
             (32832, 64, 16, 4, 1, "bf16", True), (32832, 96, 40, 5, 2, "bf16", False),   # N < 64, one pass
             (1000, 1000, 64, 8, 2, "bf16", True), (2000, 2056, 128, 4, 1, "bf16", False),
             (300, 128, 128, 16, 1, "bf16", True), (300, 128, 256, 16, 2, "bf16", False),  # groups of 8, 16
             # ragged tails of 16 to 56 columns past the last 64-column step: one pass (N = 64 and
             # 128), its slice mode, and the 256-expert split with one or several steps per slice
             (32832, 120, 64, 8, 1, "bf16", True), (5000, 1048, 128, 4, 2, "bf16", True),
             (2000, 4112, 64, 8, 1, "bf16", True), (520, 184, 256, 8, 1, "bf16", True),
             (300, 7720, 256, 8, 1, "bf16", True),
             (300, 40, 64, 8, 1, "bf16", True), (300, 56, 256, 8, 1, "bf16", False)]  # d below one step


@pytest.mark.parametrize("T,d,N,M,Kp,dtype,store", TIE_CASES)
def test_route_from_x_exact_ties(gpu, T, d, N, M, Kp, dtype, store):
    # integer scores are computed exactly on both sides, so the choice -- including every tie,
    # broken by the lower expert id, and -0 == +0 -- must match the oracle bit for bit, for each
    # router alone and for both from one pass
    print(f"[route ties from x] T={T} d={d} N={N} M={M} K'={Kp} {dtype} store={store}", flush=True)
    xd, wd, bd, xh, wh, bh = _int_operands(T, d, N, seed=T + N + Kp, f32=dtype == "f32", zero_rows=(0, 1, T - 1))
    w = W.variant(W.routing(), T=T, d=d, N=N, M=M, Kp=Kp, dtype=dtype)
    lg_ref = oracle.logits(xh, wh, bh)
    ref = {}
    for mode, omode in ((moge.ROUTE_GROUPED, "grouped"), (moge.ROUTE_GLOBAL, "global")):
        _, idx, gate, lg = _route_dev(w, x=xd, wr=wd, bias=bd, mode=mode, store_logits=store)
        if store:
            assert np.array_equal(lg, lg_ref)
        ridx, rgate, _ = oracle.route(lg_ref, M, Kp, omode)
        ref[omode] = (ridx, rgate)
        assert (idx == ridx).all(), f"{omode}: {(idx != ridx).any(1).sum()} tokens differ"
        assert (np.abs(gate - rgate) <= 1e-5 * rgate + 1e-8).all()
    idx, gate, gidx, ggate = _route_pair_dev(w, x=xd, wr=wd, bias=bd)
    for (i, g), omode in (((idx, gate), "grouped"), ((gidx, ggate), "global")):
        ridx, rgate = ref[omode]
        assert (i == ridx).all(), f"pair {omode}: {(i != ridx).any(1).sum()} tokens differ"
        assert (np.abs(g - rgate) <= 1e-5 * rgate + 1e-8).all()


NAN_CASES = [(200, 64, 8, 1, moge.ROUTE_GROUPED), (200, 64, 8, 2, moge.ROUTE_GLOBAL),
             (130, 256, 8, 8, moge.ROUTE_GLOBAL), (100, 16, 4, 2, moge.ROUTE_GROUPED)]


@pytest.mark.parametrize("T,N,M,Kp,mode", NAN_CASES)
def test_route_nan_scores_keep_the_groups_full(gpu, T, N, M, Kp, mode):
    # NaN is outside the method; the library ranks it as -inf, so every group still gets exactly K'
    # distinct experts of its own, the same ones the oracle picks with NaN read as -inf
    rng = np.random.default_rng(T + N)
    lg = rng.standard_normal((T, N)).astype(np.float32)
    lg[rng.random((T, N)) < 0.1] = np.nan
    lg[3] = np.nan                                              # a token with no number at all
    lg[5, :N // 2] = -np.inf
    w = W.variant(W.routing(), T=T, N=N, M=M, Kp=Kp)
    _, idx, _, _ = _route_dev(w, lg_np=lg, mode=mode)
    omode = "grouped" if mode == moge.ROUTE_GROUPED else "global"
    ridx, _, _ = oracle.route(np.where(np.isnan(lg), -np.inf, lg).astype(np.float32), M, Kp, omode)
    assert (idx == ridx).all()
    k, G, ng = (Kp, N // M, M) if mode == moge.ROUTE_GROUPED else (M * Kp, N, 1)
    for g in range(ng):                         # exactly k distinct experts of group g in its slots
        sl = idx[:, g * k:(g + 1) * k]
        assert ((sl >= g * G) & (sl < (g + 1) * G)).all()
        assert all(len(set(r)) == k for r in sl.tolist())


def test_route_nan_token_from_x(gpu):
    # a NaN in a token's row makes all its scores NaN inside the fused epilogue: it still takes
    # the first K' experts of every group (ties by the lower id); the other tokens are unaffected
    T, d, N, M, Kp = 300, 128, 64, 8, 2
    xd, wd, bd, xh, wh, bh = _int_operands(T, d, N, seed=11)
    xd[7, 3] = float("nan")
    w = W.variant(W.routing(), T=T, d=d, N=N, M=M, Kp=Kp)
    _, idx, _, _ = _route_dev(w, x=xd, wr=wd, bias=bd)
    ridx, _, _ = oracle.route(oracle.logits(xh, wh, bh), M, Kp, "grouped")
    keep = np.arange(T) != 7
    assert (idx[keep] == ridx[keep]).all()
    assert (idx[7] == np.repeat(np.arange(M) * (N // M), Kp) + np.tile(np.arange(Kp), M)).all()


def test_check_finite(gpu):
    ws = torch.empty(moge.workspace_size(moge.Shape(1, 8, 1, 1, 1, 0, moge.F32), moge.STAGE_CHECK),
                     dtype=torch.uint8, device="cuda")
    a = torch.randn(1_000_003, device="cuda")
    moge.check_finite(a, ws)
    for bad, where in ((float("nan"), 999_999), (float("inf"), 5), (float("-inf"), 1_000_002)):
        b = a.clone()
        b[where] = bad
        b[where + 1 if where + 1 < b.numel() else 0] = bad
        with pytest.raises(moge.MogeError, match="NONFINITE") as ei:
            moge.check_finite(b, ws)
        first = min(where, where + 1 if where + 1 < b.numel() else 0)
        assert f"2 of {b.numel()} values" in str(ei.value) and f"index {first}" in str(ei.value)
    h = torch.randn(4099, device="cuda").to(torch.bfloat16)
    moge.check_finite(h, ws)
    h[4098] = float("inf")
    with pytest.raises(moge.MogeError, match="NONFINITE"):
        moge.check_finite(h, ws)
    moge.check_finite(torch.empty(0, device="cuda"), ws)
