"""The seeded inputs of a workload, on the device (for the library) and on the host (for the
oracle), generated from the same streams so both sides see identical bytes.

Generation only: nothing here computes any part of the MoGE layer.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import fill_device, normal_host
from . import workloads as W


@dataclasses.dataclass
class DeviceInputs:
    x: "object"
    w_router: "object"
    bias: "object | None"
    w_gate: "object | None"
    w_up: "object | None"
    w_down: "object | None"
    shared: "tuple | None"


def device_inputs(w: W.Workload, device="cuda") -> DeviceInputs:
    """Every input tensor of `w` on the device, filled by the generator's HIP kernel.  Expert
    weights are row-major ([E][F][d], [E][F][d], [E][d][F]) for experts [e_lo, e_hi): expert e's
    weights are the elements from e*F*d on of their tensor's stream."""
    import torch

    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    E = w.e_hi - w.e_lo

    def filled(shape, tid, std, start=0, dtype=dt):
        t = torch.empty(shape, dtype=dtype, device=device)
        fill_device(t, w.seed, tid, std, start)
        return t

    x = filled((w.T, w.d), W.TID_X, w.std_x)
    wr = filled((w.N, w.d), W.TID_WROUTER, w.std_router)
    bias = filled((w.N,), W.TID_BIAS, w.std_bias, dtype=torch.float32) if w.std_bias else None
    wg = wu = wd = shared = None
    if w.F:
        wg = filled((E, w.F, w.d), W.TID_WGATE, w.std_gate, w.e_lo * w.F * w.d)
        wu = filled((E, w.F, w.d), W.TID_WUP, w.std_up, w.e_lo * w.F * w.d)
        wd = filled((E, w.d, w.F), W.TID_WDOWN, w.std_down, w.e_lo * w.d * w.F)
    if w.F_shared:
        shared = (filled((w.F_shared, w.d), W.TID_SGATE, w.std_gate), filled((w.F_shared, w.d), W.TID_SUP, w.std_up),
                  filled((w.d, w.F_shared), W.TID_SDOWN, w.std_shared_down))
    return DeviceInputs(x, wr, bias, wg, wu, wd, shared)


class HostInputs:
    """Host-side view of the same inputs, generated lazily and in pieces (uint16 bf16 bit patterns
    or float32 values)."""

    def __init__(self, w: W.Workload):
        self.w = w
        self.bf16 = w.dtype == "bf16"
        self._experts = {}

    def _gen(self, tid, n, std, start=0):
        return normal_host(self.w.seed, tid, n, std, self.bf16, start)

    def x_rows(self, tokens) -> np.ndarray:
        w = self.w
        return np.stack([self._gen(W.TID_X, w.d, w.std_x, int(t) * w.d) for t in tokens])

    def x_all(self) -> np.ndarray:
        w = self.w
        return self._gen(W.TID_X, w.T * w.d, w.std_x).reshape(w.T, w.d)

    def w_router(self) -> np.ndarray:
        w = self.w
        return self._gen(W.TID_WROUTER, w.N * w.d, w.std_router).reshape(w.N, w.d)

    def bias(self):
        w = self.w
        return normal_host(w.seed, W.TID_BIAS, w.N, w.std_bias, False) if w.std_bias else None

    def expert(self, e: int):
        if e not in self._experts:
            w = self.w
            fd = w.F * w.d
            self._experts[e] = (self._gen(W.TID_WGATE, fd, w.std_gate, e * fd).reshape(w.F, w.d),
                                self._gen(W.TID_WUP, fd, w.std_up, e * fd).reshape(w.F, w.d),
                                self._gen(W.TID_WDOWN, fd, w.std_down, e * fd).reshape(w.d, w.F))
        return self._experts[e]

    def shared(self):
        w = self.w
        if not w.F_shared:
            return None
        fd = w.F_shared * w.d
        return (self._gen(W.TID_SGATE, fd, w.std_gate).reshape(w.F_shared, w.d),
                self._gen(W.TID_SUP, fd, w.std_up).reshape(w.F_shared, w.d),
                self._gen(W.TID_SDOWN, fd, w.std_shared_down).reshape(w.d, w.F_shared))


def sample_tokens(T: int, n: int, seed: int = 123) -> np.ndarray:
    """A seeded sample of about n token ids out of T (always including the first and the last)."""
    rng = np.random.default_rng(seed)
    pick = set([0, T - 1]) | set(rng.choice(T, size=min(n, T), replace=False).tolist())
    return np.array(sorted(pick)[:max(n, 2)], dtype=np.int64)
