"""GPU parity of the Monte-Carlo imbalance study (moge_route on given scores + moge_imbalance_batches)
against the oracle: every batch's group loads and imbalance score, both routers, bit-exact."""
import numpy as np
import pytest
import torch

import mixture_grouped_experts_amd as moge
from mixture_grouped_experts_amd import imbalance_study as S
import oracle

pytestmark = pytest.mark.gpu


def _oracle_batches(lg, cfg, mode):
    loads, isr = [], []
    for b in range(cfg.batches):
        part = lg[b * cfg.tokens:(b + 1) * cfg.tokens]
        idx, _, _ = oracle.route(part, cfg.M, cfg.Kp, mode)
        gl, ir = oracle.imbalance(np.bincount(idx.ravel(), minlength=cfg.N), cfg.M)
        loads.append(gl)
        isr.append(ir)
    return np.array(loads), np.array(isr)


@pytest.mark.parametrize("cfg", [S.StudyConfig(64, 8, 1, 64, 2.0, 40), S.StudyConfig(16, 4, 2, 33, 0.5, 25),
                                 S.StudyConfig(256, 8, 1, 16, 0.0, 30)], ids=str)
def test_study_matches_oracle_per_batch(gpu, cfg):
    lg = S.scores(cfg, seed=3)
    lg_host = lg.cpu().numpy()
    for mode, omode in ((moge.ROUTE_GROUPED, "grouped"), (moge.ROUTE_GLOBAL, "global")):
        _, is_raw, loads = S.route_and_score(cfg, lg, mode)
        torch.cuda.synchronize()
        rl, ri = _oracle_batches(lg_host, cfg, omode)
        assert (loads.cpu().numpy() == rl).all(), omode
        assert (is_raw.cpu().numpy() == ri).all(), omode
        if omode == "grouped":
            assert (ri == 0).all() and (rl == cfg.tokens * cfg.Kp).all()


def test_study_summary_shows_the_pages_claim(gpu):
    # with popular experts, global top-K almost always leaves the devices unbalanced; MoGE never does
    r = S.study(S.StudyConfig(64, 8, 1, 256, 2.0, 200), seed=1)
    assert r["moge"]["max_is_raw"] == 0 and r["moge"]["p_positive"] == 0.0
    assert r["global_topk"]["p_positive"] > 0.95
