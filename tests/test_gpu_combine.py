"""GPU parity: moge_combine on its own, against the weighted sum it is defined as.

y[t] = sum over the token's slots s, in slot order, of gate[t,s] * o[inv[t,s]] (slots with inv = -1 are
skipped), plus the shared expert's output row when one is given.  The reference is that sum in float64;
the kernel accumulates in float32, so the bound is a few float32 roundings of the sum of magnitudes.
"""
import numpy as np
import pytest
import torch

import mixture_grouped_experts_amd as moge

pytestmark = pytest.mark.gpu


def _case(T, d, N, M, Kp, rows_cap, bf16, shared, drop, seed):
    rng = np.random.default_rng(seed)
    K = M * Kp
    tdt = torch.bfloat16 if bf16 else torch.float32
    o = torch.from_numpy(rng.standard_normal((rows_cap, d)).astype(np.float32)).to(tdt)
    inv = rng.integers(0, rows_cap, size=(T, K)).astype(np.int32)
    inv[rng.random((T, K)) < drop] = -1          # slots of experts outside the computed range
    gate = rng.random((T, K)).astype(np.float32)
    sh = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(tdt) if shared else None
    s = moge.Shape(T, d, N, M, Kp, 8, moge.BF16 if bf16 else moge.F32)
    y = torch.full((T, d), np.nan, dtype=torch.float32, device="cuda")
    moge.combine(s, o.cuda(), torch.from_numpy(inv).cuda(), torch.from_numpy(gate).cuda(), rows_cap,
                 sh.cuda() if shared else None, y)
    torch.cuda.synchronize()
    o64 = o.double().numpy()
    ref = np.zeros((T, d))
    mag = np.zeros((T, d))
    for k in range(K):
        live = inv[:, k] >= 0
        term = gate[:, k, None].astype(np.float64) * o64[np.where(live, inv[:, k], 0)]
        ref += np.where(live[:, None], term, 0.0)
        mag += np.where(live[:, None], np.abs(term), 0.0)
    if shared:
        ref += sh.double().numpy()
        mag += np.abs(sh.double().numpy())
    got = y.cpu().double().numpy()
    bound = (K + 2) * 2.0 ** -23 * mag + 1e-30
    assert np.isfinite(got).all()
    assert (np.abs(got - ref) <= bound).all(), float(np.max(np.abs(got - ref) - bound))


@pytest.mark.parametrize("T,d,N,M,Kp,rows_cap,bf16,shared,drop", [
    (1, 64, 8, 4, 1, 5, True, False, 0.0),
    (3, 520, 64, 8, 2, 40, True, True, 0.0),       # ragged hidden size: a 512-column block plus 8 columns
    (257, 1024, 64, 8, 1, 3000, True, False, 0.3),
    (100, 72, 16, 4, 1, 400, False, True, 0.5),
    (37, 256, 128, 8, 9, 3000, True, True, 0.2),   # K = 72: more than one 64-slot batch
    (64, 128, 16, 1, 3, 200, False, False, 0.0),   # K = 3: a partial 8-slot batch
    (50, 96, 8, 8, 1, 60, True, False, 1.0),       # every slot outside the range: y is the zero vector
])
def test_combine_matches_weighted_sum(gpu, T, d, N, M, Kp, rows_cap, bf16, shared, drop):
    _case(T, d, N, M, Kp, rows_cap, bf16, shared, drop, seed=T * 7 + d)
