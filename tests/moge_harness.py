"""Shared helpers for the GPU parity tests and the smoke check.

Inputs come from the ``synth`` generator on both sides (device buffers filled by its HIP
kernel, host arrays for the oracle by its C filler: identical bytes).  The GPU side runs
only through the libmoge C ABI (``mixture_grouped_experts_amd``); the expected values
come only from ``oracle``.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import oracle
import synth
from synth import workloads as W

NEAR_TIE = 1e-5  # p(K'-th) - p((K'+1)-th) below this: a token whose choice may legitimately flip


def tol_ok(gpu: np.ndarray, ref: np.ndarray):
    """End-to-end bar: max|gpu - ref| <= 1e-2 * max|ref| + 1e-3."""
    err = float(np.max(np.abs(gpu.astype(np.float64) - ref))) if ref.size else 0.0
    bound = 1e-2 * float(np.max(np.abs(ref))) + 1e-3 if ref.size else 1e-3
    return err <= bound, err, bound


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Run-to-run equality of whole buffers, padding included: compared as raw bytes, since rows
    that no kernel writes keep whatever the allocator handed out, NaN patterns among them, and
    NaN never compares equal as a number."""
    if a.shape != b.shape or a.dtype != b.dtype:
        return False
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


# ---- the tiled operand layout and padded row numbering of include/moge.h, restated here
# from that header's definition (test side; the library is not consulted)

def _up(v: int, a: int) -> int:
    return -(-v // a) * a


def tile_rows(a: torch.Tensor, row_align: int = 16) -> torch.Tensor:
    """[R][C] row-major -> flat tiled layout: 16 x 32 tiles, rows padded to row_align, cols to 32 (zeros)."""
    R, C = a.shape
    Rp, Cp = _up(R, row_align), _up(C, 32)
    p = torch.zeros(Rp, Cp, dtype=a.dtype, device=a.device)
    p[:R, :C] = a
    return p.reshape(Rp // 16, 16, Cp // 32, 32).permute(0, 2, 1, 3).contiguous().reshape(-1)


def untile_rows(flat: torch.Tensor, R: int, C: int, keep_pad_cols: bool = False) -> torch.Tensor:
    """Inverse of tile_rows for the first R rows (all Cp columns if keep_pad_cols)."""
    Rp, Cp = _up(R, 16), _up(C, 32)
    a = flat[:Rp * Cp].reshape(Rp // 16, Cp // 32, 16, 32).permute(0, 2, 1, 3).reshape(Rp, Cp)
    return a[:R] if keep_pad_cols else a[:R, :C]


def pack_ref(w: torch.Tensor) -> torch.Tensor:
    """Packed expert weights [E][rows][cols] -> E tiled matrices, rows and cols padded to 32."""
    return torch.cat([tile_rows(w[e], 32) for e in range(w.shape[0])])


def segment_bases(counts: np.ndarray, e_lo: int, e_hi: int) -> np.ndarray:
    """P(e) for e in [e_lo, e_hi] (index e - e_lo): segments rounded up to 16 rows."""
    c = np.asarray(counts, dtype=np.int64)[e_lo:e_hi]
    return np.concatenate([[0], np.cumsum(-(-c // 16) * 16)])


def padded_rows(idx: np.ndarray, rinv: np.ndarray, rperm: np.ndarray, counts: np.ndarray, offsets: np.ndarray,
                e_lo: int, e_hi: int):
    """The oracle's dense local rows -> the padded numbering: (inv, perm) with perm -1 on padding rows."""
    P = segment_bases(counts, e_lo, e_hi)
    inv = rinv.astype(np.int64).copy()
    live = rinv >= 0
    e = idx[live].astype(np.int64)
    inv[live] = rinv[live] - (offsets[e] - offsets[e_lo]) + P[e - e_lo]
    perm = np.full(int(P[-1]), -1, dtype=np.int64)
    for k in range(e_hi - e_lo):
        ee = e_lo + k
        n = int(counts[ee])
        d0 = int(offsets[ee] - offsets[e_lo])
        perm[P[k]:P[k] + n] = rperm[d0:d0 + n]
    return inv.astype(np.int32), perm.astype(np.int32)


@dataclasses.dataclass
class DeviceInputs:
    x: torch.Tensor
    w_router: torch.Tensor
    bias: torch.Tensor | None
    w_gate: torch.Tensor | None
    w_up: torch.Tensor | None
    w_down: torch.Tensor | None
    shared: tuple | None


def device_inputs(w: W.Workload, device="cuda") -> DeviceInputs:
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    E = w.e_hi - w.e_lo

    def filled(shape, tid, std, start=0, dtype=dt):
        t = torch.empty(shape, dtype=dtype, device=device)
        synth.fill_device(t, w.seed, tid, std, start)
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
    """Host-side (oracle-side) view of the same inputs, generated lazily and in pieces."""

    def __init__(self, w: W.Workload):
        self.w = w
        self.bf16 = w.dtype == "bf16"
        self._experts = {}

    def _gen(self, tid, n, std, start=0):
        return synth.normal_host(self.w.seed, tid, n, std, self.bf16, start)

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
        return synth.normal_host(w.seed, W.TID_BIAS, w.N, w.std_bias, False) if w.std_bias else None

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


def oracle_logits_all(h: HostInputs) -> np.ndarray:
    return oracle.logits(h.x_all(), h.w_router(), h.bias())


def compare_routing(w: W.Workload, gpu_idx: np.ndarray, ref_idx: np.ndarray, ref_gap: np.ndarray):
    """Returns (n_near_tie, flipped_token_ids, hard_failures)."""
    diff = np.any(gpu_idx != ref_idx, axis=1)
    near = ref_gap < NEAR_TIE
    flipped = np.nonzero(diff & near)[0]
    hard = np.nonzero(diff & ~near)[0]
    return int(near.sum()), flipped, hard


def sample_tokens(T: int, n: int, seed: int = 123) -> np.ndarray:
    rng = np.random.default_rng(seed)
    pick = set([0, T - 1]) | set(rng.choice(T, size=min(n, T), replace=False).tolist())
    return np.array(sorted(pick)[:max(n, 2)], dtype=np.int64)
