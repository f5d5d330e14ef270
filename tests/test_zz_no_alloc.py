"""moge_dispatch_noalloc (the dispatch for callers that cannot allocate device memory) against
moge_dispatch with a caller workspace: identical counts, offsets, inv, perm and row copies, on two
calls in a row, the second with a smaller input (the fixed scratch array keeps the first call's
contents, which the second must not depend on)."""
import numpy as np
import pytest
import torch

import mixture_grouped_experts_amd as moge
import oracle

pytestmark = pytest.mark.gpu


def _idx(T, N, M, Kp, seed):
    rng = np.random.default_rng(seed)
    lg = (rng.standard_normal((T, N)) + rng.standard_normal(N) * 2.0).astype(np.float32)
    return oracle.route(lg, M, Kp, "grouped")[0]


def _dispatch(noalloc, s, idx, x, e_lo, e_hi, cap):
    T, N, K, d = s.T, s.N, s.K, s.d
    dev = dict(dtype=torch.int32, device="cuda")
    counts, offsets = torch.full((N,), -1, **dev), torch.full((N + 1,), -1, **dev)
    inv, perm = torch.full((T, K), -9, **dev), torch.full((cap,), -9, **dev)
    xp = torch.full((moge.tiled_elems(cap, d),), 7.0, dtype=x.dtype, device="cuda")
    di = torch.from_numpy(idx).cuda()
    if noalloc:
        moge.dispatch_noalloc(s, moge.ROUTE_GROUPED, di, x, e_lo, e_hi, cap, counts, offsets, inv, perm, xp)
    else:
        ws = torch.empty(moge.workspace_size(s), dtype=torch.uint8, device="cuda")
        moge.dispatch(s, moge.ROUTE_GROUPED, di, x, e_lo, e_hi, cap, counts, offsets, inv, perm, xp, ws)
    torch.cuda.synchronize()
    return counts, offsets, inv, perm, xp


def test_noalloc_dispatch_matches_workspace_dispatch(gpu):
    # first call large (several 64-token blocks: the scratch holds the block counts), second smaller
    for T, N, M, Kp, d, e_lo, e_hi in ((20000, 64, 8, 1, 128, 0, 64), (9000, 256, 8, 1, 64, 32, 96)):
        print(f"[noalloc dispatch] T={T} N={N} M={M} K'={Kp} range [{e_lo}, {e_hi})", flush=True)
        s = moge.Shape(T, d, N, M, Kp, 8, moge.BF16)
        cap = moge.rows_bound(s, moge.ROUTE_GROUPED, e_lo, e_hi)
        idx = _idx(T, N, M, Kp, seed=T)
        x = torch.randn(T, d, device="cuda").to(torch.bfloat16)
        ref = _dispatch(False, s, idx, x, e_lo, e_hi, cap)
        got = _dispatch(True, s, idx, x, e_lo, e_hi, cap)
        for a, b in zip(ref, got):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.uint8) if b.dtype == torch.bfloat16 else b)
        rc, ro, _, _ = oracle.dispatch(idx, N, e_lo, e_hi)
        assert (got[0].cpu().numpy() == rc).all() and (got[1].cpu().numpy() == ro).all()


def test_noalloc_dispatch_rejects_shapes_past_its_scratch(gpu):
    s = moge.Shape(131073, 64, 256, 8, 1, 8, moge.BF16)       # 256 * 2049 blocks * 8 bytes > 4 MiB
    dev = dict(dtype=torch.int32, device="cuda")
    with pytest.raises(moge.MogeError, match="WORKSPACE"):
        moge.dispatch_noalloc(s, moge.ROUTE_GROUPED, torch.zeros(1, s.K, **dev).expand(s.T, s.K).contiguous(),
                              None, 0, 256, 0, torch.empty(256, **dev), torch.empty(257, **dev), None, None, None)
