"""CPU oracle for the MoGE layer forward pass.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the GPU library (``mixture_grouped_experts_amd``) and never imports it; the
two meet only in the seeded inputs of the ``synth`` package.

The arithmetic lives in ``moge_oracle.c`` (plain loops, binary64) and is driven
from here with NumPy arrays.  The steps follow the Pangu Pro MoE pages:

* router scores, then a softmax over all experts, then the top-K' experts inside
  every one of M equal groups (lsdiaocha.cn summary, section 1; hyper.ai abstract);
* the conventional global top-K router as the comparator (same section);
* dropless dispatch, a SwiGLU expert per chosen slot, a gate-weighted sum;
* per-device load and the imbalance score (busiest minus idlest device,
  lsdiaocha.cn summary, section 1).

Pins for every function are in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_HERE, "libmoge_oracle.so")

BF16 = 0
F32 = 1
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int64


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB)
        lib.oracle_logits.argtypes = [_I, _I, _I, ctypes.c_int, _P, _P, _P, _P]
        lib.oracle_route.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P]
        lib.oracle_dispatch.argtypes = [_I, _I, _I, _P, _I, _I, _P, _P, _P, _P]
        lib.oracle_ffn_row.argtypes = [_I, _I, ctypes.c_int, _P, _P, _P, _P, _P]
        lib.oracle_imbalance.argtypes = [_I, _I, _P, _P, _P]
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = ctypes.c_int
        for f in (lib.oracle_logits, lib.oracle_route, lib.oracle_dispatch, lib.oracle_ffn_row,
                  lib.oracle_imbalance):
            f.restype = None
        _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the oracle uses."""
    return int(_load().oracle_threads())


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"inputs must be bf16 bits (uint16) or float32, got {a.dtype}")


def _c(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a)


def logits(x: np.ndarray, w_router: np.ndarray, bias: np.ndarray | None = None) -> np.ndarray:
    """x [T,d], w_router [N,d] (both uint16 bf16 bits or both float32), bias [N] float32 or None.
    Returns binary32 logits [T,N] (binary64 sum, one rounding)."""
    x, w_router = _c(x), _c(w_router)
    T, d = x.shape
    N = w_router.shape[0]
    dt = _dtype_code(x)
    assert _dtype_code(w_router) == dt and w_router.shape[1] == d
    out = np.empty((T, N), dtype=np.float32)
    b = None
    if bias is not None:
        b = _c(bias.astype(np.float32))
    _load().oracle_logits(T, d, N, dt, x.ctypes.data, w_router.ctypes.data, None if b is None else b.ctypes.data,
                          out.ctypes.data)
    return out


def route(lg: np.ndarray, M: int, Kp: int, mode: str = "grouped"):
    """Grouped (MoGE) or global top-K routing on binary32 logits [T,N].

    Returns (idx int32 [T,K], gate float64 [T,K], gap float64 [T]) with K = M*Kp.
    mode "grouped": M groups, K' = Kp per group.  mode "global": one group, K = M*Kp."""
    lg = _c(lg.astype(np.float32, copy=False))
    T, N = lg.shape
    if N % M or not (1 <= Kp <= N // M):
        raise ValueError("need N % M == 0 and 1 <= K' <= N/M")
    if mode == "grouped":
        n_groups, k = M, Kp
    elif mode == "global":
        n_groups, k = 1, M * Kp
    else:
        raise ValueError(mode)
    K = n_groups * k
    idx = np.full((T, K), -1, dtype=np.int32)
    gate = np.zeros((T, K), dtype=np.float64)
    gap = np.zeros(T, dtype=np.float64)
    _load().oracle_route(T, N, n_groups, k, lg.ctypes.data, idx.ctypes.data, gate.ctypes.data, gap.ctypes.data)
    return idx, gate, gap


def dispatch(idx: np.ndarray, N: int, e_lo: int = 0, e_hi: int | None = None):
    """Returns (counts [N], offsets [N+1], inv [T,K], perm [rows in range]) as int32."""
    idx = _c(idx.astype(np.int32, copy=False))
    T, K = idx.shape
    if e_hi is None:
        e_hi = N
    counts = np.zeros(N, dtype=np.int32)
    offsets = np.zeros(N + 1, dtype=np.int32)
    inv = np.empty((T, K), dtype=np.int32)
    perm = np.full(T * K, -1, dtype=np.int32)
    _load().oracle_dispatch(T, K, N, idx.ctypes.data, e_lo, e_hi, counts.ctypes.data, offsets.ctypes.data,
                            inv.ctypes.data, perm.ctypes.data)
    rows = int(offsets[e_hi] - offsets[e_lo])
    return counts, offsets, inv, perm[:rows].copy()


def ffn_row(x_row: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """One SwiGLU expert on one row: x_row [d], w_gate/w_up [F,d], w_down [d,F] -> float64 [d]."""
    x_row, w_gate, w_up, w_down = _c(x_row), _c(w_gate), _c(w_up), _c(w_down)
    d = x_row.shape[0]
    F = w_gate.shape[0]
    dt = _dtype_code(x_row)
    assert w_gate.shape == (F, d) and w_up.shape == (F, d) and w_down.shape == (d, F)
    assert all(_dtype_code(a) == dt for a in (w_gate, w_up, w_down))
    out = np.empty(d, dtype=np.float64)
    _load().oracle_ffn_row(d, F, dt, x_row.ctypes.data, w_gate.ctypes.data, w_up.ctypes.data, w_down.ctypes.data,
                           out.ctypes.data)
    return out


def imbalance(counts: np.ndarray, M: int):
    """Returns (group_load int32 [M], IS_raw int)."""
    counts = _c(counts.astype(np.int32, copy=False))
    N = counts.shape[0]
    gl = np.zeros(M, dtype=np.int32)
    isr = np.zeros(1, dtype=np.int32)
    _load().oracle_imbalance(N, M, counts.ctypes.data, gl.ctypes.data, isr.ctypes.data)
    return gl, int(isr[0])


def combine_rows(x_rows: np.ndarray, idx_rows: np.ndarray, gate_rows: np.ndarray, e_lo: int, e_hi: int,
                 expert_weights, shared_weights=None) -> np.ndarray:
    """Layer output for a set of token rows, computed one token at a time.

    x_rows [n,d]; idx_rows, gate_rows [n,K]; expert_weights(e) -> (w_gate [F,d], w_up [F,d], w_down [d,F]) for
    e in [e_lo, e_hi); shared_weights: None or the same triple for the always-on shared expert (weight 1).
    y[t] = sum over slots s in slot order of gate[t,s] * FFN_idx[t,s](x[t]) for experts in range, plus the shared
    expert's output.  Returns float64 [n,d]."""
    n, d = x_rows.shape
    K = idx_rows.shape[1]
    y = np.zeros((n, d), dtype=np.float64)
    for r in range(n):
        acc = np.zeros(d, dtype=np.float64)
        for s in range(K):
            e = int(idx_rows[r, s])
            if e_lo <= e < e_hi:
                wg, wu, wd = expert_weights(e)
                acc = acc + gate_rows[r, s] * ffn_row(x_rows[r], wg, wu, wd)
        if shared_weights is not None:
            acc = acc + ffn_row(x_rows[r], *shared_weights)
        y[r] = acc
    return y
