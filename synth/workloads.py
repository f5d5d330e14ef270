"""The seeded synthetic MoGE workloads (shapes and value distributions only).

Shapes follow the pages' workloads: a tiny layer with 8 experts in 4 groups of 2
(the restaurant picture of 8 waiters in 4 zones, Pangu Pro MoE summary, section 1);
Pangu Pro's 64 experts in 8 groups with top-1 per group; the Pangu Ultra MoE shape
(hidden 7680, 256 routed experts, 1 shared expert, expert width 2048, 8 active);
one device's share of a 32 x 2048-token batch under 8-way expert grouping; and the
Pangu Pro layer (hidden 5120, 64 experts, 4 shared experts; expert width chosen).

``N(0, s)`` names the standard deviation ``s``.  Values come from the counter-based
generator in ``synth_def.h``; each tensor has its own stream id below.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

# stream ids (one independent stream per tensor)
TID_X = 1
TID_WROUTER = 2
TID_BIAS = 3
TID_WGATE = 4
TID_WUP = 5
TID_WDOWN = 6
TID_SGATE = 7
TID_SUP = 8
TID_SDOWN = 9


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    N: int
    M: int
    Kp: int
    F: int                      # expert FFN width (0: routing only)
    F_shared: int               # shared-expert width (0: none)
    dtype: str                  # "bf16" or "f32"
    std_x: float
    std_router: float
    std_gate: float
    std_up: float
    std_down: float
    std_shared_down: float
    std_bias: Optional[float]   # None: no router bias
    e_lo: int                   # routed experts computed: [e_lo, e_hi)
    e_hi: int
    seed: int = 0

    @property
    def G(self) -> int:
        return self.N // self.M

    @property
    def K(self) -> int:
        return self.M * self.Kp

    @property
    def routing_only(self) -> bool:
        return self.F == 0

    def rows_cap(self) -> int:
        """Rows of the expert range under grouped routing: each token puts
        min(K', |range & group|) rows into every group the range touches."""
        rows = 0
        for g in range(self.M):
            lo, hi = max(self.e_lo, g * self.G), min(self.e_hi, (g + 1) * self.G)
            if hi > lo:
                rows += min(self.Kp, hi - lo)
        return self.T * rows


def tiny() -> Workload:
    s_in = float(1.0 / math.sqrt(128))
    return Workload("tiny_fp32_T64_d128_N8_M4", 64, 128, 8, 4, 1, 64, 0, "f32", 1.0, s_in, s_in, s_in,
                    float(1.0 / math.sqrt(64)), 0.0, None, 0, 8)


def routing() -> Workload:
    return Workload("route_T65536_d4096_N64_M8", 65536, 4096, 64, 8, 1, 0, 0, "bf16", 1.0, 0.02, 0.0, 0.0, 0.0,
                    0.0, 2.0, 0, 64)


def decode() -> Workload:
    return Workload("decode_T256_d4096_N64_M8_K2_F1408", 256, 4096, 64, 8, 2, 1408, 0, "bf16", 1.0, 0.02, 0.02,
                    0.02, 0.02, 0.0, None, 0, 64)


def ultra() -> Workload:
    return Workload("ultra_T8192_d7680_N256_M8_F2048_shared1", 8192, 7680, 256, 8, 1, 2048, 2048, "bf16", 1.0,
                    0.02, 0.02, 0.02, 0.02, 0.02, None, 0, 256)


def group0() -> Workload:
    return Workload("group0_T65536_d4096_N64_M8_F1408", 65536, 4096, 64, 8, 1, 1408, 0, "bf16", 1.0, 0.02, 0.02,
                    0.02, 0.02, 0.0, 2.0, 0, 8)


def pro() -> Workload:
    """Pangu Pro layer shape (lsdiaocha.cn summary, section 2: hidden 5120, 64 routed experts in
    8 groups with top-1 per group, 4 shared experts).  The expert width is not on the pages: 1408
    is chosen (the width of the other 64-expert workloads); the 4 shared SwiGLU experts are one
    shared expert of width 4 x 1408 = 5632, which computes exactly their sum."""
    return Workload("pro_T8192_d5120_N64_M8_F1408_shared4", 8192, 5120, 64, 8, 1, 1408, 4 * 1408, "bf16", 1.0,
                    0.02, 0.02, 0.02, 0.02, 0.02, None, 0, 64)


def variant(base: Workload, **kw) -> Workload:
    """A workload derived from `base`; the expert range defaults to all N experts."""
    if "e_hi" not in kw:
        kw["e_hi"] = kw.get("N", base.N)
        kw.setdefault("e_lo", 0)
    return dataclasses.replace(base, **kw)


ALL = {w.name: w for w in (tiny(), routing(), decode(), ultra(), group0(), pro())}
