"""Monte-Carlo imbalance study: the conventional global top-K router against MoGE's grouped top-K'.

Pangu Pro MoE, lsdiaocha.cn summary, section 1: the imbalance score of a batch is the workload gap
between its busiest and its idlest device; simulating routing shows that the conventional top-K
router's score is almost always above zero, while MoGE, which takes K' experts from every group
(one group per device), keeps it at exactly zero.

Each batch here is `tokens` tokens whose router scores are independent N(0, 1) draws plus one
expert-popularity offset per (batch, expert) drawn from N(0, skew) -- skew 0 means no expert is
favoured, larger skew makes a few experts popular, the situation that unbalances global top-K.
Scores come from the seeded counter-based generator of ``synth``; routing and the per-batch score
run through the libmoge C ABI (moge_route on given scores, then moge_imbalance_batches), so every
batch of the study is routed by the same kernels as the layer.

    python -m mixture_grouped_experts_amd.imbalance_study [--batches B] [--seed S]

prints one JSON line per configuration and a summary line with the routing throughput.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import time

import torch

import synth

from . import _lib as L

TID_SCORES = 20   # generator streams of the study (distinct from the layer's tensors)
TID_BIAS = 21


@dataclasses.dataclass(frozen=True)
class StudyConfig:
    N: int          # routed experts
    M: int          # groups (devices)
    Kp: int         # experts per group (MoGE); the global router takes K = M * Kp
    tokens: int     # tokens per batch
    skew: float     # std of the per-(batch, expert) popularity offset
    batches: int    # Monte-Carlo batches


def scores(cfg: StudyConfig, seed: int, device="cuda") -> torch.Tensor:
    """[batches * tokens][N] float32 router scores of the study (deterministic in seed and cfg)."""
    T = cfg.batches * cfg.tokens
    lg = torch.empty(T, cfg.N, dtype=torch.float32, device=device)
    synth.fill_device(lg, seed, TID_SCORES, 1.0)
    if cfg.skew > 0:
        bias = torch.empty(cfg.batches, cfg.N, dtype=torch.float32, device=device)
        synth.fill_device(bias, seed, TID_BIAS, cfg.skew)
        lg.view(cfg.batches, cfg.tokens, cfg.N).add_(bias[:, None, :])
    return lg


def route_and_score(cfg: StudyConfig, lg: torch.Tensor, mode: int, stream=None):
    """Routes every batch with `mode` and returns (idx [T][K], per-batch is_raw [B], group_load [B][M])."""
    T = cfg.batches * cfg.tokens
    shape = L.Shape(T, 8, cfg.N, cfg.M, cfg.Kp, 0, L.F32)
    K = cfg.M * cfg.Kp
    dev = lg.device
    idx = torch.empty(T, K, dtype=torch.int32, device=dev)
    gate = torch.empty(T, K, dtype=torch.float32, device=dev)
    group_load = torch.empty(cfg.batches, cfg.M, dtype=torch.int32, device=dev)
    is_raw = torch.empty(cfg.batches, dtype=torch.int32, device=dev)
    L.route(shape, mode, None, None, None, lg, idx, gate, None, stream)
    L.imbalance_batches(shape, idx, cfg.tokens, group_load, is_raw, stream)
    return idx, is_raw, group_load


def study(cfg: StudyConfig, seed: int = 0, device="cuda") -> dict:
    lg = scores(cfg, seed, device)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _, is_moge, _ = route_and_score(cfg, lg, L.ROUTE_GROUPED)
    _, is_glob, _ = route_and_score(cfg, lg, L.ROUTE_GLOBAL)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    g = is_glob.double()
    m = is_moge.double()
    return {
        "N": cfg.N, "M": cfg.M, "k_per_group": cfg.Kp, "K": cfg.M * cfg.Kp, "tokens_per_batch": cfg.tokens,
        "skew": cfg.skew, "batches": cfg.batches,
        "global_topk": {"p_positive": float((g > 0).double().mean()), "mean_is_raw": float(g.mean()),
                        "mean_is_norm": float(g.mean() / cfg.tokens), "max_is_raw": int(g.max())},
        "moge": {"p_positive": float((m > 0).double().mean()), "max_is_raw": int(m.max())},
        "seconds": dt, "tokens_routed_per_s": 2 * cfg.batches * cfg.tokens / dt,
    }


DEFAULT_GRID = [StudyConfig(N, M, 1, t, s, 0) for (N, M) in ((64, 8), (256, 8))
                for t in (16, 64, 256, 1024, 4096) for s in (0.0, 0.5, 2.0)]


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--batches", type=int, default=1000)
    p.add_argument("--seed", type=int, default=0)
    args = p.parse_args()
    total_tokens, total_s = 0, 0.0
    for c in DEFAULT_GRID:
        cfg = dataclasses.replace(c, batches=args.batches)
        r = study(cfg, args.seed)
        total_tokens += 2 * cfg.batches * cfg.tokens
        total_s += r["seconds"]
        print(json.dumps(r), flush=True)
    print(json.dumps({"summary": "imbalance study", "configurations": len(DEFAULT_GRID), "batches": args.batches,
                      "tokens_routed": total_tokens, "seconds": total_s,
                      "tokens_routed_per_s": total_tokens / total_s}), flush=True)


if __name__ == "__main__":
    main()
