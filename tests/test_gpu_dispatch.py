"""GPU parity: moge_dispatch against the oracle (bit-exact counts, offsets, inv, perm, x_perm)."""
import numpy as np
import pytest
import torch

import mixture_grouped_experts_amd as moge
import oracle
import synth
from tests import moge_harness as H

pytestmark = pytest.mark.gpu


def _idx(T, N, M, Kp, seed, skew=2.0, mode="grouped"):
    rng = np.random.default_rng(seed)
    lg = (rng.standard_normal((T, N)) + rng.standard_normal(N) * skew).astype(np.float32)
    return oracle.route(lg, M, Kp, mode)[0]


def _run(T, d, N, M, Kp, idx, e_lo, e_hi, bf16=True, mode=moge.ROUTE_GROUPED, extra_cap=0):
    s = moge.Shape(T, d, N, M, Kp, 8, moge.BF16 if bf16 else moge.F32)
    cap = moge.rows_bound(s, mode, e_lo, e_hi) + extra_cap
    K = M * Kp
    x = torch.empty(T, d, dtype=torch.bfloat16 if bf16 else torch.float32, device="cuda")
    synth.fill_device(x, 3, 1, 1.0)
    dev = dict(dtype=torch.int32, device="cuda")
    counts = torch.full((N,), -1, **dev)
    offsets = torch.full((N + 1,), -1, **dev)
    inv = torch.full((T, K), -9, **dev)
    perm = torch.full((cap,), -9, **dev)
    xp = torch.full((moge.tiled_elems(cap, d),), 7.0, dtype=x.dtype, device="cuda")   # padding columns must become 0
    xt = torch.full((moge.tiled_elems(T, d),), 7.0, dtype=x.dtype, device="cuda")
    ws = torch.empty(moge.workspace_size(s), dtype=torch.uint8, device="cuda")
    moge.dispatch(s, mode, torch.from_numpy(idx).cuda(), x, e_lo, e_hi, cap, counts, offsets, inv, perm, xp, ws,
                  x_tiled=xt)
    torch.cuda.synchronize()
    # the token-order tiled copy is x itself, padding columns zero
    assert torch.equal(H.untile_rows(xt, T, d), x)
    assert (H.untile_rows(xt, T, d, keep_pad_cols=True)[:, d:] == 0).all()
    return x, counts.cpu().numpy(), offsets.cpu().numpy(), inv.cpu().numpy(), perm.cpu().numpy(), xp


def _check_rows(idx, x, counts, offsets, inv, perm, xp, e_lo, e_hi):
    """counts/offsets bit-exact; inv/perm equal to the oracle's rows in the padded numbering; live rows
    of x_perm are the tokens' rows (padding columns zero); rows past the last segment untouched."""
    N = counts.size
    rc, ro, rinv, rperm = oracle.dispatch(idx, N, e_lo, e_hi)
    assert (counts == rc).all() and (offsets == ro).all()
    pinv, pperm = H.padded_rows(idx, rinv, rperm, rc, ro, e_lo, e_hi)
    assert (inv == pinv).all()
    end = pperm.size
    assert (perm[:end] == pperm).all() and (perm[end:] == -9).all()
    d = x.shape[1]
    live = np.nonzero(pperm >= 0)[0]
    rows = H.untile_rows(xp, end, d, keep_pad_cols=True) if end else None
    if live.size:
        assert torch.equal(rows[torch.from_numpy(live).cuda(), :d], x[torch.from_numpy(pperm[live]).long().cuda()])
        assert (rows[torch.from_numpy(live).cuda(), d:] == 0).all()


CASES = [
    # T, d, N, M, Kp, e_lo, e_hi
    (64, 128, 8, 4, 1, 0, 8),
    (1, 64, 8, 4, 2, 0, 8),
    (257, 256, 64, 8, 2, 0, 64),
    (1000, 520, 64, 8, 1, 0, 8),
    (3000, 128, 256, 8, 1, 0, 256),
    (777, 64, 64, 8, 1, 13, 45),
    (513, 64, 16, 1, 4, 0, 16),
    (300, 64, 64, 8, 8, 0, 64),
]


@pytest.mark.parametrize("T,d,N,M,Kp,e_lo,e_hi", CASES)
def test_dispatch_bitexact(gpu, T, d, N, M, Kp, e_lo, e_hi):
    idx = _idx(T, N, M, Kp, seed=T + N)
    x, counts, offsets, inv, perm, xp = _run(T, d, N, M, Kp, idx, e_lo, e_hi)
    _check_rows(idx, x, counts, offsets, inv, perm, xp, e_lo, e_hi)


def test_dispatch_skewed_and_empty_experts(gpu):
    T, d, N, M, Kp = 2048, 64, 64, 8, 1
    idx = np.empty((T, M * Kp), dtype=np.int32)
    idx[:] = np.arange(M) * (N // M)           # every token picks the first expert of every group
    idx[::5] += 1                              # a few pick the second; experts 2..7 of each group stay empty
    x, counts, offsets, inv, perm, xp = _run(T, d, N, M, Kp, idx, 0, N)
    _check_rows(idx, x, counts, offsets, inv, perm, xp, 0, N)
    assert (counts[2:8] == 0).all()


def test_dispatch_float32_and_global_mode(gpu):
    T, d, N, M, Kp = 333, 64, 16, 4, 1
    idx = _idx(T, N, M, Kp, seed=1, mode="global")
    x, counts, offsets, inv, perm, xp = _run(T, 72, N, M, Kp, idx, 4, 12, bf16=False, mode=moge.ROUTE_GLOBAL)
    _check_rows(idx, x, counts, offsets, inv, perm, xp, 4, 12)


def test_dispatch_rejects_small_capacity(gpu):
    s = moge.Shape(100, 64, 8, 4, 1, 8, moge.BF16)
    cap = moge.rows_bound(s, moge.ROUTE_GROUPED, 0, 8)
    dev = dict(dtype=torch.int32, device="cuda")
    with pytest.raises(moge.MogeError, match="CAPACITY"):
        moge.dispatch(s, moge.ROUTE_GROUPED, torch.zeros(100, 4, **dev), torch.zeros(100, 64, dtype=torch.bfloat16,
                      device="cuda"), 0, 8, cap - 1, torch.zeros(8, **dev), torch.zeros(9, **dev),
                      torch.zeros(100, 4, **dev), torch.zeros(cap, **dev),
                      torch.zeros(moge.tiled_elems(cap, 64), dtype=torch.bfloat16, device="cuda"),
                      torch.empty(moge.workspace_size(s), dtype=torch.uint8, device="cuda"))


@pytest.mark.parametrize("T,d,N,M,Kp", [
    (8192, 64, 256, 1, 1),    # M = 1 (MoGE is the global top-K), one workgroup: 70.6 KiB of LDS
    (8192, 64, 1, 1, 1),      # one expert takes every token
    (32, 64, 256, 8, 32),     # K' = N/M: every expert chosen, K = 256, one workgroup
    (40, 64, 256, 8, 32),     # K = 256 over several 64-token blocks
    (20, 64, 256, 1, 256),    # one group of all 256 experts, every one chosen
])
def test_dispatch_edge_slot_counts(gpu, T, d, N, M, Kp):
    idx = _idx(T, N, M, Kp, seed=T * 7 + Kp)
    x, counts, offsets, inv, perm, xp = _run(T, d, N, M, Kp, idx, 0, N)
    _check_rows(idx, x, counts, offsets, inv, perm, xp, 0, N)
