"""GPU parity: moge_grouped_ffn against the oracle's SwiGLU expert (binary64) and, for the bf16
path, against dense torch.matmul on the same bf16 operands (a library routine)."""
import dataclasses

import numpy as np
import pytest
import torch

import mixture_grouped_experts_amd as moge
import oracle
from synth import workloads as W
from tests import moge_harness as H

pytestmark = pytest.mark.gpu


def _pack(dtype_code, w):
    out = torch.empty(w.shape[0] * moge.packed_weight_elems(w.shape[1], w.shape[2]), dtype=w.dtype, device="cuda")
    moge.pack_weights(dtype_code, w, out)
    return out


def _dispatch_then_ffn(w, e_lo=None, e_hi=None):
    """Route with the oracle, dispatch and run the grouped FFN through the C ABI.  Returns the
    un-tiled x_perm and h (test-side restatement of the tiled layout) and the segment bases."""
    e_lo = w.e_lo if e_lo is None else e_lo
    e_hi = w.e_hi if e_hi is None else e_hi
    w = dataclasses.replace(w, e_lo=e_lo, e_hi=e_hi)
    dv = H.device_inputs(w)
    hi = H.HostInputs(w)
    lg = H.oracle_logits_all(hi)
    idx, _, _ = oracle.route(lg, w.M, w.Kp, "grouped")
    dc = moge.BF16 if w.dtype == "bf16" else moge.F32
    s = moge.Shape(w.T, w.d, w.N, w.M, w.Kp, w.F, dc)
    cap = moge.rows_bound(s, moge.ROUTE_GROUPED, e_lo, e_hi)
    dt = dv.x.dtype
    i32 = dict(dtype=torch.int32, device="cuda")
    counts, offsets = torch.empty(w.N, **i32), torch.empty(w.N + 1, **i32)
    inv, perm = torch.empty(w.T, w.K, **i32), torch.empty(cap, **i32)
    xp = torch.empty(moge.tiled_elems(cap, w.d), dtype=dt, device="cuda")
    ws = torch.empty(moge.workspace_size(s), dtype=torch.uint8, device="cuda")
    moge.dispatch(s, moge.ROUTE_GROUPED, torch.from_numpy(idx).cuda(), dv.x, e_lo, e_hi, cap, counts, offsets, inv,
                  perm, xp, ws)
    pg, pu, pd = _pack(dc, dv.w_gate), _pack(dc, dv.w_up), _pack(dc, dv.w_down)
    torch.cuda.synchronize()
    # packing against the test-side restatement of the layout
    assert torch.equal(pg, H.pack_ref(dv.w_gate)) and torch.equal(pd, H.pack_ref(dv.w_down))
    hbuf = torch.full((moge.tiled_elems(cap, w.F),), float("nan"), dtype=dt, device="cuda")
    out = torch.full((cap, w.d), float("nan"), dtype=dt, device="cuda")
    moge.grouped_ffn(s, xp, offsets, e_lo, e_hi, cap, pg, pu, pd, hbuf, out)
    torch.cuda.synchronize()
    counts = counts.cpu().numpy()
    P = H.segment_bases(counts, e_lo, e_hi)
    X = H.untile_rows(xp, cap, w.d)
    Hm = H.untile_rows(hbuf, cap, w.F, keep_pad_cols=True)
    return w, dv, hi, idx, counts, P, perm.cpu().numpy(), X, Hm, out


def _live_rows(w, counts, P):
    return np.concatenate([np.arange(P[k], P[k] + counts[w.e_lo + k]) for k in range(w.e_hi - w.e_lo)])


def _expert_of(w, P, rows):
    return np.searchsorted(P, rows, side="right") - 1 + w.e_lo


MID = W.variant(W.decode(), name="mid_T300_d256_N16_M4_K2_F200", T=300, d=256, N=16, M=4, Kp=2, F=200,
                          std_bias=1.0)


@pytest.mark.parametrize("w", [MID, W.variant(MID, name="mid_F1408_d520", d=520, F=1408, T=97),
                               W.decode()], ids=lambda w: w.name)
def test_grouped_ffn_vs_torch_matmul(gpu, w):
    print(f"[ffn vs torch] {w.name}", flush=True)
    w, dv, _, _, counts, P, perm, X, Hm, out = _dispatch_then_ffn(w)
    for ei in range(w.e_hi - w.e_lo):
        e = w.e_lo + ei
        r0, r1 = int(P[ei]), int(P[ei] + counts[e])
        if r1 == r0:
            continue
        xe = X[r0:r1].float()
        a = xe @ dv.w_gate[ei].float().t().contiguous()
        b = xe @ dv.w_up[ei].float().t().contiguous()
        href = (a * torch.sigmoid(a) * b)
        # h: float32 epilogue of float32 sums, rounded to bf16 -> within a couple of bf16 ulps
        hm = Hm[r0:r1, :w.F].float()
        assert torch.allclose(hm, href, rtol=1.6e-2, atol=1e-3 * href.abs().max().item() + 1e-6)
        assert (Hm[r0:r1, w.F:] == 0).all()  # padding columns of h are exact zeros
        oref = hm @ dv.w_down[ei].float().t().contiguous()
        assert torch.allclose(out[r0:r1].float(), oref, rtol=1.6e-2, atol=1e-3 * oref.abs().max().item() + 1e-6)
    live = torch.from_numpy(_live_rows(w, counts, P)).long().cuda()
    assert not torch.isnan(out[live].float()).any()


@pytest.mark.parametrize("w", [MID, W.decode(), W.tiny()], ids=lambda w: w.name)
def test_grouped_ffn_vs_oracle_rows(gpu, w):
    print(f"[ffn vs oracle] {w.name}", flush=True)
    w, dv, hi, idx, counts, P, perm, X, Hm, out = _dispatch_then_ffn(w)
    live = _live_rows(w, counts, P)
    rows = live[np.unique(np.linspace(0, live.size - 1, min(live.size, 48)).astype(int))]
    expert_of = _expert_of(w, P, rows)
    ref = np.stack([oracle.ffn_row(hi.x_rows([perm[r]])[0], *hi.expert(int(e))) for r, e in zip(rows, expert_of)])
    got = out[torch.from_numpy(rows).long().cuda()].float().cpu().numpy()
    ok, err, bound = H.tol_ok(got, ref)
    assert ok, (err, bound)


def test_grouped_ffn_expert_range_and_shared_form(gpu):
    # a device's share: experts [4, 8) only, weights of those experts only
    w, dv, hi, idx, counts, P, perm, X, Hm, out = _dispatch_then_ffn(MID, 4, 8)
    live = _live_rows(w, counts, P)
    rows = live[::max(1, live.size // 20)]
    expert_of = _expert_of(w, P, rows)
    ref = np.stack([oracle.ffn_row(hi.x_rows([perm[r]])[0], *hi.expert(int(e))) for r, e in zip(rows, expert_of)])
    ok, err, bound = H.tol_ok(out[torch.from_numpy(rows).long().cuda()].float().cpu().numpy(), ref)
    assert ok, (err, bound)
    # the shared-expert form: one expert, offsets {0, T}, x_perm = x in the tiled layout
    sw = W.variant(MID, F_shared=136, std_shared_down=0.02)
    dsh = H.device_inputs(sw).shared
    hsh = H.HostInputs(sw).shared()
    s1 = moge.Shape(sw.T, sw.d, 1, 1, 1, 136, moge.BF16)
    so = torch.tensor([0, sw.T], dtype=torch.int32, device="cuda")
    hb = torch.empty(moge.tiled_elems(sw.T, 136), dtype=torch.bfloat16, device="cuda")
    ob = torch.empty(sw.T, sw.d, dtype=torch.bfloat16, device="cuda")
    packed = [_pack(moge.BF16, m.unsqueeze(0)) for m in dsh]
    moge.grouped_ffn(s1, H.tile_rows(dv.x), so, 0, 1, sw.T, packed[0], packed[1], packed[2], hb, ob)
    torch.cuda.synchronize()
    toks = [0, 1, 150, sw.T - 1]
    ref = np.stack([oracle.ffn_row(hi.x_rows([t])[0], *hsh) for t in toks])
    ok, err, bound = H.tol_ok(ob[toks].float().cpu().numpy(), ref)
    assert ok, (err, bound)


@pytest.mark.parametrize("w", [
    W.variant(MID, name="fused_shared_d256", F_shared=136, std_shared_down=0.02, T=333),
    # d = 520: 17 reduction steps, so the gate/up GEMM's per-expert starting step is not 0 for the
    # shared expert's position in the list either (16 * 37 mod 17 = 14)
    W.variant(MID, name="fused_shared_d520", d=520, F_shared=136, std_shared_down=0.02, T=333),
], ids=lambda w: w.name)
def test_routed_and_shared_in_one_launch_bitexact(gpu, w):
    # the fused launches compute every element exactly as the separate calls do
    dv = H.device_inputs(w)
    hi = H.HostInputs(w)
    idx, _, _ = oracle.route(H.oracle_logits_all(hi), w.M, w.Kp, "grouped")
    s = moge.Shape(w.T, w.d, w.N, w.M, w.Kp, w.F, moge.BF16)
    cap = moge.rows_bound(s, moge.ROUTE_GROUPED, 0, w.N)
    i32 = dict(dtype=torch.int32, device="cuda")
    bf = dict(dtype=torch.bfloat16, device="cuda")
    counts, offsets = torch.empty(w.N, **i32), torch.empty(w.N + 1, **i32)
    inv, perm = torch.empty(w.T, w.K, **i32), torch.empty(cap, **i32)
    xp, xt = torch.empty(moge.tiled_elems(cap, w.d), **bf), torch.empty(moge.tiled_elems(w.T, w.d), **bf)
    ws = torch.empty(moge.workspace_size(s), dtype=torch.uint8, device="cuda")
    moge.dispatch(s, moge.ROUTE_GROUPED, torch.from_numpy(idx).cuda(), dv.x, 0, w.N, cap, counts, offsets, inv, perm,
                  xp, ws, x_tiled=xt)
    pg, pu, pd = _pack(moge.BF16, dv.w_gate), _pack(moge.BF16, dv.w_up), _pack(moge.BF16, dv.w_down)
    sg, su, sd = (_pack(moge.BF16, m.unsqueeze(0)) for m in dv.shared)
    Fs = w.F_shared

    def bufs():
        return (torch.zeros(moge.tiled_elems(cap, w.F), **bf), torch.zeros(cap, w.d, **bf),
                torch.zeros(moge.tiled_elems(w.T, Fs), **bf), torch.zeros(w.T, w.d, **bf))
    h1, o1, hs1, so1 = bufs()
    moge.expert_gate_up(s, xp, offsets, 0, w.N, cap, pg, pu, h1)
    moge.expert_down(s, h1, offsets, 0, w.N, cap, pd, o1)
    moge.grouped_ffn(moge.Shape(w.T, w.d, 1, 1, 1, Fs, moge.BF16), xt,
                     torch.tensor([0, w.T], **i32), 0, 1, w.T, sg, su, sd, hs1, so1)
    h2, o2, hs2, so2 = bufs()
    moge.expert_gate_up_with_shared(s, Fs, xp, offsets, 0, w.N, cap, pg, pu, h2, xt, sg, su, hs2)
    moge.expert_down_with_shared(s, Fs, h2, offsets, 0, w.N, cap, pd, o2, hs2, sd, so2)
    torch.cuda.synchronize()
    P = H.segment_bases(counts.cpu().numpy(), 0, w.N)
    live = torch.from_numpy(_live_rows(w, counts.cpu().numpy(), P)).long().cuda()
    assert torch.equal(H.untile_rows(h1, cap, w.F)[live], H.untile_rows(h2, cap, w.F)[live])
    assert torch.equal(o1[live], o2[live])
    assert torch.equal(hs1, hs2) and torch.equal(so1, so2)
    # an expert's outputs do not depend on the expert range of the call: experts [5, 13) alone
    lo, hi_ = 5, 13
    cap3 = moge.rows_bound(s, moge.ROUTE_GROUPED, lo, hi_)
    c3, of3 = torch.empty(w.N, **i32), torch.empty(w.N + 1, **i32)
    inv3, perm3, xp3 = torch.empty(w.T, w.K, **i32), torch.empty(cap3, **i32), torch.empty(moge.tiled_elems(cap3, w.d), **bf)
    moge.dispatch(s, moge.ROUTE_GROUPED, torch.from_numpy(idx).cuda(), dv.x, lo, hi_, cap3, c3, of3, inv3, perm3,
                  xp3, ws)
    h3 = torch.zeros(moge.tiled_elems(cap3, w.F), **bf)
    o3 = torch.zeros(cap3, w.d, **bf)
    sl = slice(lo * moge.packed_weight_elems(w.F, w.d), hi_ * moge.packed_weight_elems(w.F, w.d))
    sld = slice(lo * moge.packed_weight_elems(w.d, w.F), hi_ * moge.packed_weight_elems(w.d, w.F))
    moge.grouped_ffn(s, xp3, of3, lo, hi_, cap3, pg[sl], pu[sl], pd[sld], h3, o3)
    torch.cuda.synchronize()
    cn = counts.cpu().numpy()
    P3 = H.segment_bases(cn, lo, hi_)
    H1 = H.untile_rows(h1, cap, w.F)
    H3 = H.untile_rows(h3, cap3, w.F)
    for e in range(lo, hi_):
        n = int(cn[e])
        a0, b0 = int(P[e]), int(P3[e - lo])
        assert torch.equal(H1[a0:a0 + n], H3[b0:b0 + n]), e
        assert torch.equal(o1[a0:a0 + n], o3[b0:b0 + n]), e


@pytest.mark.parametrize("w", [
    W.variant(MID, name="gather_shared_T333", F_shared=136, std_shared_down=0.02, T=333),
    W.variant(MID, name="gather_range_3_11", e_lo=3, e_hi=11),
    W.variant(MID, name="gather_shared_T1", F_shared=64, std_shared_down=0.02, T=1),
    W.variant(MID, name="gather_T17_d512_N64_M8", T=17, d=512, N=64, M=8, Kp=1, F=1408, F_shared=256,
              std_shared_down=0.02),
], ids=lambda w: w.name)
def test_gathered_gate_up_bitexact(gpu, w):
    # reading the token rows from x through perm gives exactly the h of the tiled x_perm
    dv = H.device_inputs(w)
    hi = H.HostInputs(w)
    idx, _, _ = oracle.route(H.oracle_logits_all(hi), w.M, w.Kp, "grouped")
    s = moge.Shape(w.T, w.d, w.N, w.M, w.Kp, w.F, moge.BF16)
    cap = moge.rows_bound(s, moge.ROUTE_GROUPED, w.e_lo, w.e_hi)
    i32 = dict(dtype=torch.int32, device="cuda")
    bf = dict(dtype=torch.bfloat16, device="cuda")
    dix = torch.from_numpy(idx).cuda()
    ws = torch.empty(moge.workspace_size(s), dtype=torch.uint8, device="cuda")
    Fs = w.F_shared

    def disp(copy):
        counts, offsets = torch.empty(w.N, **i32), torch.empty(w.N + 1, **i32)
        inv, perm = torch.empty(w.T, w.K, **i32), torch.full((cap,), -7, **i32)
        xp = torch.empty(moge.tiled_elems(cap, w.d), **bf) if copy else None
        xt = torch.empty(moge.tiled_elems(w.T, w.d), **bf) if copy and Fs else None
        moge.dispatch(s, moge.ROUTE_GROUPED, dix, dv.x if copy else None, w.e_lo, w.e_hi, cap, counts, offsets, inv,
                      perm, xp, ws, x_tiled=xt)
        return counts, offsets, inv, perm, xp, xt
    c1, o1, inv1, p1, xp, xt = disp(True)
    c2, o2, inv2, p2, _, _ = disp(False)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(o1, o2) and torch.equal(inv1, inv2) and torch.equal(p1, p2)
    pg, pu = _pack(moge.BF16, dv.w_gate), _pack(moge.BF16, dv.w_up)   # experts e_lo .. e_hi-1
    sg, su = (_pack(moge.BF16, m.unsqueeze(0)) for m in dv.shared[:2]) if Fs else (None, None)
    h1 = torch.full((moge.tiled_elems(cap, w.F),), 3.0, **bf)
    h2 = torch.full((moge.tiled_elems(cap, w.F),), 5.0, **bf)
    hs1 = torch.full((moge.tiled_elems(w.T, Fs),), 3.0, **bf) if Fs else None
    hs2 = torch.full((moge.tiled_elems(w.T, Fs),), 5.0, **bf) if Fs else None
    if Fs:
        moge.expert_gate_up_with_shared(s, Fs, xp, o1, w.e_lo, w.e_hi, cap, pg, pu, h1, xt, sg, su, hs1)
    else:
        moge.expert_gate_up(s, xp, o1, w.e_lo, w.e_hi, cap, pg, pu, h1)
    moge.expert_gate_up_gather(s, dv.x, p2, o2, w.e_lo, w.e_hi, cap, pg, pu, h2, Fs, sg, su, hs2)
    torch.cuda.synchronize()
    counts = c1.cpu().numpy()
    P = H.segment_bases(counts, w.e_lo, w.e_hi)
    live = torch.from_numpy(_live_rows(w, counts, P)).long().cuda()
    if live.numel():
        assert torch.equal(H.untile_rows(h1, cap, w.F, keep_pad_cols=True)[live],
                          H.untile_rows(h2, cap, w.F, keep_pad_cols=True)[live])
    if Fs:   # rows T .. (rounded up to 16) of the tiled hs are never written
        assert torch.equal(H.untile_rows(hs1, w.T, Fs, keep_pad_cols=True),
                           H.untile_rows(hs2, w.T, Fs, keep_pad_cols=True))


def test_gathered_gate_up_clipped_capacity(gpu):
    # a capacity below the padded rows, not a multiple of 16: the last segments are cut at
    # rows_cap in both row sources alike, and perm holds exactly rows_cap entries
    w = W.variant(MID, name="gather_clipped")
    print(f"[gather clipped] {w.name}", flush=True)
    dv = H.device_inputs(w)
    idx, _, _ = oracle.route(H.oracle_logits_all(H.HostInputs(w)), w.M, w.Kp, "grouped")
    s = moge.Shape(w.T, w.d, w.N, w.M, w.Kp, w.F, moge.BF16)
    cap = moge.rows_bound(s, moge.ROUTE_GROUPED, 0, w.N)
    i32 = dict(dtype=torch.int32, device="cuda")
    bf = dict(dtype=torch.bfloat16, device="cuda")
    counts, offsets = torch.empty(w.N, **i32), torch.empty(w.N + 1, **i32)
    inv, perm = torch.empty(w.T, w.K, **i32), torch.empty(cap, **i32)
    xp = torch.empty(moge.tiled_elems(cap, w.d), **bf)
    ws = torch.empty(moge.workspace_size(s), dtype=torch.uint8, device="cuda")
    moge.dispatch(s, moge.ROUTE_GROUPED, torch.from_numpy(idx).cuda(), dv.x, 0, w.N, cap, counts, offsets, inv, perm,
                  xp, ws)
    torch.cuda.synchronize()
    cn = counts.cpu().numpy()
    P = H.segment_bases(cn, 0, w.N)
    padded = int(P[-1])                          # P has N + 1 entries: the last is the padded total
    cap2 = padded - 21
    assert cap2 % 16 and cap2 < P[-2] + cn[-1]   # the last expert is cut inside one of its 16-row bands
    perm2 = perm[:cap2].clone()
    pg, pu = _pack(moge.BF16, dv.w_gate), _pack(moge.BF16, dv.w_up)
    h1 = torch.full((moge.tiled_elems(cap2, w.F),), 3.0, **bf)
    h2 = torch.full((moge.tiled_elems(cap2, w.F),), 5.0, **bf)
    moge.expert_gate_up(s, xp, offsets, 0, w.N, cap2, pg, pu, h1)
    moge.expert_gate_up_gather(s, dv.x, perm2, offsets, 0, w.N, cap2, pg, pu, h2, 0, None, None, None)
    torch.cuda.synchronize()
    live = _live_rows(w, cn, P)
    live = torch.from_numpy(live[live < cap2]).long().cuda()
    a = H.untile_rows(h1, cap2, w.F, keep_pad_cols=True)[live]
    b = H.untile_rows(h2, cap2, w.F, keep_pad_cols=True)[live]
    assert torch.equal(a, b)
    # rows at and past rows_cap are never written
    tail = H.untile_rows(h2, (cap2 + 15) // 16 * 16, w.F, keep_pad_cols=True)[cap2:]
    assert bool((tail == 5.0).all())


@pytest.mark.parametrize("w", [
    W.variant(MID, name="fused_group1_T333", T=333, Kp=1, e_lo=4, e_hi=8),
    W.variant(MID, name="fused_group0_T2000_N64", T=2000, d=256, N=64, M=8, Kp=1, F=136, e_lo=0, e_hi=8,
              std_bias=2.0),
    W.variant(MID, name="fused_T1", T=1, Kp=1, e_lo=12, e_hi=16),
], ids=lambda w: w.name)
def test_down_combine_bitexact(gpu, w):
    # one whole group with K' = 1: GEMM 2 writing y itself equals GEMM 2 + the combine pass bit for bit
    dv = H.device_inputs(w)
    hi = H.HostInputs(w)
    idx, gate, _ = oracle.route(H.oracle_logits_all(hi), w.M, w.Kp, "grouped")
    s = moge.Shape(w.T, w.d, w.N, w.M, w.Kp, w.F, moge.BF16)
    cap = moge.rows_bound(s, moge.ROUTE_GROUPED, w.e_lo, w.e_hi)
    i32 = dict(dtype=torch.int32, device="cuda")
    bf = dict(dtype=torch.bfloat16, device="cuda")
    counts, offsets = torch.empty(w.N, **i32), torch.empty(w.N + 1, **i32)
    inv, perm = torch.empty(w.T, w.K, **i32), torch.empty(cap, **i32)
    ws = torch.empty(moge.workspace_size(s), dtype=torch.uint8, device="cuda")
    moge.dispatch(s, moge.ROUTE_GROUPED, torch.from_numpy(idx).cuda(), None, w.e_lo, w.e_hi, cap, counts, offsets,
                  inv, perm, None, ws)
    pg, pu, pd = _pack(moge.BF16, dv.w_gate), _pack(moge.BF16, dv.w_up), _pack(moge.BF16, dv.w_down)
    h = torch.empty(moge.tiled_elems(cap, w.F), **bf)
    moge.expert_gate_up_gather(s, dv.x, perm, offsets, w.e_lo, w.e_hi, cap, pg, pu, h)
    g = torch.from_numpy(gate.astype(np.float32)).cuda()
    o = torch.empty(cap, w.d, **bf)
    y1 = torch.full((w.T, w.d), float("nan"), dtype=torch.float32, device="cuda")
    y2 = torch.full((w.T, w.d), float("nan"), dtype=torch.float32, device="cuda")
    moge.expert_down(s, h, offsets, w.e_lo, w.e_hi, cap, pd, o)
    moge.combine(s, o, inv, g, cap, None, y1)
    moge.expert_down_combine(s, h, offsets, w.e_lo, w.e_hi, cap, pd, perm, g, y2)
    torch.cuda.synchronize()
    assert torch.isfinite(y2).all()                       # every token's row written
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


@pytest.mark.parametrize("w", [
    W.decode(),                                                                          # 64 rows per expert
    W.variant(MID, name="tiles_shared_T333", F_shared=136, std_shared_down=0.02, T=333),
    W.variant(MID, name="tiles_range_T700", T=700, e_lo=3, e_hi=11, F=1408),
    W.variant(MID, name="tiles_group_fused", T=333, Kp=1, e_lo=4, e_hi=8),
    # split columns with a ragged width (1400 = 43.75 units) and the shared expert in the same launch
    W.variant(MID, name="tiles_split_ragged_shared", T=400, F=1400, F_shared=136, std_shared_down=0.02),
], ids=lambda w: w.name)
def test_tile_shapes_bitexact(gpu, w):
    # the 320 x 256 tiles, the 96 x 512 tiles and the tall tiles with gate/up's columns split
    # into 128- and 96-column tiles compute every output element identically
    dv = H.device_inputs(w)
    hi = H.HostInputs(w)
    idx, gate, _ = oracle.route(H.oracle_logits_all(hi), w.M, w.Kp, "grouped")
    s = moge.Shape(w.T, w.d, w.N, w.M, w.Kp, w.F, moge.BF16)
    cap = moge.rows_bound(s, moge.ROUTE_GROUPED, w.e_lo, w.e_hi)
    i32 = dict(dtype=torch.int32, device="cuda")
    bf = dict(dtype=torch.bfloat16, device="cuda")
    counts, offsets = torch.empty(w.N, **i32), torch.empty(w.N + 1, **i32)
    inv, perm = torch.empty(w.T, w.K, **i32), torch.empty(cap, **i32)
    ws = torch.empty(moge.workspace_size(s), dtype=torch.uint8, device="cuda")
    moge.dispatch(s, moge.ROUTE_GROUPED, torch.from_numpy(idx).cuda(), None, w.e_lo, w.e_hi, cap, counts, offsets,
                  inv, perm, None, ws)
    pg, pu, pd = _pack(moge.BF16, dv.w_gate), _pack(moge.BF16, dv.w_up), _pack(moge.BF16, dv.w_down)
    Fs = w.F_shared
    sg, su, sd = (_pack(moge.BF16, m.unsqueeze(0)) for m in dv.shared) if Fs else (None, None, None)
    g = torch.from_numpy(gate.astype(np.float32)).cuda()
    fused = w.Kp == 1 and not Fs and w.e_hi - w.e_lo == w.N // w.M and w.e_lo % (w.N // w.M) == 0
    outs = []
    for tiles in (moge.TILES_TALL, moge.TILES_WIDE, moge.TILES_BALANCED):
        s.tiles = tiles
        if True:
            h = torch.zeros(moge.tiled_elems(cap, w.F), **bf)
            hs = torch.zeros(moge.tiled_elems(w.T, Fs), **bf) if Fs else None
            o = torch.zeros(cap, w.d, **bf)
            so = torch.zeros(w.T, w.d, **bf) if Fs else None
            y = torch.zeros(w.T, w.d, dtype=torch.float32, device="cuda")
            moge.expert_gate_up_gather(s, dv.x, perm, offsets, w.e_lo, w.e_hi, cap, pg, pu, h, Fs, sg, su, hs)
            if Fs:
                moge.expert_down_with_shared(s, Fs, h, offsets, w.e_lo, w.e_hi, cap, pd, o, hs, sd, so)
            else:
                moge.expert_down(s, h, offsets, w.e_lo, w.e_hi, cap, pd, o)
            if fused:
                moge.expert_down_combine(s, h, offsets, w.e_lo, w.e_hi, cap, pd, perm, g, y)
            torch.cuda.synchronize()
            outs.append((h, o, hs, so, y))
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            if a is not None:
                assert H.same_bits(a, b)
