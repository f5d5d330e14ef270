"""Shared helpers for the GPU parity tests and the smoke check.

Inputs come from the ``synth`` generator on both sides (device buffers filled by its HIP
kernel, host arrays for the oracle by its C filler: identical bytes).  The GPU side runs
only through the libmoge C ABI (``mixture_grouped_experts_amd``); the expected values
come only from ``oracle``.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from synth import workloads as W
from synth.inputs import DeviceInputs, HostInputs, device_inputs, sample_tokens  # noqa: F401

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


def oracle_logits_all(h: HostInputs) -> np.ndarray:
    return oracle.logits(h.x_all(), h.w_router(), h.bias())


def order_gap(lg: np.ndarray, M: int, Kp: int, mode: str = "grouped") -> np.ndarray:
    """Per token, the smallest softmax-probability gap between adjacent ranks 1 .. k + 1 inside
    any group (k = K'; in global mode one group of all N experts with k = M K').  The slot order
    of the chosen experts is their rank order, so where two chosen experts are this close,
    float32 scores summed in another order may list them in the other order."""
    l = lg.astype(np.float64)
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    T, N = p.shape
    groups, k = (M, Kp) if mode == "grouped" else (1, M * Kp)
    q = -np.sort(-p.reshape(T, groups, N // groups), axis=2)[:, :, :k + 1]
    if q.shape[2] < 2:
        return np.full(T, np.inf)
    return (q[:, :, :-1] - q[:, :, 1:]).min(axis=(1, 2))


def compare_routing(w: W.Workload, gpu_idx: np.ndarray, ref_idx: np.ndarray, ref_gap: np.ndarray,
                    ord_gap: np.ndarray = None, mode: str = "grouped"):
    """Returns (n_near_tie, flipped_token_ids, hard_failures).  A token may route differently
    only when its K'-th vs (K'+1)-th in-group gap is a near-tie; with ord_gap (order_gap of the
    same scores) it may also list the same experts of every group in another slot order when
    that order rests on a near-tie between chosen experts."""
    diff = np.any(gpu_idx != ref_idx, axis=1)
    near = ref_gap < NEAR_TIE
    ok = near.copy()
    if ord_gap is not None:
        groups = w.M if mode == "grouped" else 1
        T = gpu_idx.shape[0]
        same_sets = np.all(np.sort(gpu_idx.reshape(T, groups, -1), axis=2) ==
                           np.sort(ref_idx.reshape(T, groups, -1), axis=2), axis=(1, 2))
        ok |= same_sets & (ord_gap < NEAR_TIE)
    flipped = np.nonzero(diff & ok)[0]
    hard = np.nonzero(diff & ~ok)[0]
    return int(near.sum()), flipped, hard
