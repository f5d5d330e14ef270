"""Pins for the oracle's router scores and SwiGLU expert.

Fixed by NumPy float64 matrix products (a library routine), exactly-summed dot products (math.fsum),
closed forms of silu, and the dense-mixture special case K' = group size."""
import math

import numpy as np
import pytest
import scipy.special

import oracle
import synth


def _f32(bits):
    return synth.bf16_bits_to_f32(bits)


@pytest.mark.parametrize("bf16", [True, False])
def test_logits_vs_exact_sum(bf16):
    T, d, N = 20, 96, 8
    x = synth.normal_host(9, 1, T * d, 1.0, bf16).reshape(T, d)
    w = synth.normal_host(9, 2, N * d, 0.1, bf16).reshape(N, d)
    b = synth.normal_host(9, 3, N, 2.0, False)
    lg = oracle.logits(x, w, b)
    xf = _f32(x) if bf16 else x
    wf = _f32(w) if bf16 else w
    exact = np.array([[math.fsum(list(xf[t].astype(np.float64) * wf[e].astype(np.float64)) + [float(b[e])])
                       for e in range(N)] for t in range(T)]).astype(np.float32)
    ulp = np.spacing(np.abs(exact))
    assert (np.abs(lg - exact) <= ulp).all()
    assert (lg == exact).mean() > 0.98
    # transposed-operand mistake would fail: compare with a NumPy product too
    ref = (xf.astype(np.float64) @ wf.astype(np.float64).T + b.astype(np.float64)).astype(np.float32)
    assert np.allclose(lg, ref, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("bf16", [True, False])
def test_ffn_row_vs_numpy(bf16):
    d, F = 64, 40
    x = synth.normal_host(4, 1, d, 1.0, bf16)
    wg = synth.normal_host(4, 4, F * d, 0.2, bf16).reshape(F, d)
    wu = synth.normal_host(4, 5, F * d, 0.2, bf16).reshape(F, d)
    wd = synth.normal_host(4, 6, d * F, 0.2, bf16).reshape(d, F)
    cv = (lambda a: _f32(a).astype(np.float64)) if bf16 else (lambda a: a.astype(np.float64))
    a = cv(wg) @ cv(x)
    b = cv(wu) @ cv(x)
    h = a * scipy.special.expit(a) * b
    ref = cv(wd) @ h
    out = oracle.ffn_row(x, wg, wu, wd)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_silu_closed_forms():
    d, F = 8, 4
    x = np.zeros(d, np.float32)
    x[0] = 1.0
    wg = np.zeros((F, d), np.float32)
    wu = np.zeros((F, d), np.float32)
    wd = np.zeros((d, F), np.float32)
    wu[:, 0] = 1.0
    wd[0, :] = 1.0
    assert (oracle.ffn_row(x, wg, wu, wd) == 0).all()        # silu(0) = 0
    wg[:, 0] = 40.0                                        # silu(z) -> z for large z
    out = oracle.ffn_row(x, wg, wu, wd)
    assert math.isclose(out[0], 4 * 40.0, rel_tol=1e-15)
    wg[:, 0] = -40.0                                       # silu(z) -> 0 for very negative z
    assert abs(oracle.ffn_row(x, wg, wu, wd)[0]) < 1e-15
    wg[:, 0] = 1.0                                         # silu(1) = 1 / (1 + e^-1)
    assert math.isclose(oracle.ffn_row(x, wg, wu, wd)[0], 4 / (1 + math.exp(-1)), rel_tol=1e-15)


def test_dense_mixture_when_every_expert_chosen():
    # K' = group size: y = sum_e p_e FFN_e(x), a dense softmax mixture; slots in any order
    T, d, N, M, F = 3, 32, 4, 2, 16
    x = synth.normal_host(2, 1, T * d, 1.0, False).reshape(T, d)
    wr = synth.normal_host(2, 2, N * d, 0.3, False).reshape(N, d)
    wg = synth.normal_host(2, 4, N * F * d, 0.2, False).reshape(N, F, d)
    wu = synth.normal_host(2, 5, N * F * d, 0.2, False).reshape(N, F, d)
    wd = synth.normal_host(2, 6, N * d * F, 0.2, False).reshape(N, d, F)
    lg = oracle.logits(x, wr)
    idx, gate, _ = oracle.route(lg, M, N // M, "grouped")
    y = oracle.combine_rows(x, idx, gate, 0, N, lambda e: (wg[e], wu[e], wd[e]))
    p = scipy.special.softmax(lg.astype(np.float64), axis=1)
    ref = np.zeros((T, d))
    for t in range(T):
        for e in range(N):
            xv = x[t].astype(np.float64)
            a = wg[e].astype(np.float64) @ xv
            b = wu[e].astype(np.float64) @ xv
            ref[t] += p[t, e] * (wd[e].astype(np.float64) @ (a * scipy.special.expit(a) * b))
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-13)
    assert np.allclose(gate.sum(1), 1.0, rtol=0, atol=1e-15)


def test_combine_range_and_shared():
    T, d, N, M, F = 4, 16, 8, 4, 8
    x = synth.normal_host(6, 1, T * d, 1.0, False).reshape(T, d)
    wg = synth.normal_host(6, 4, N * F * d, 0.2, False).reshape(N, F, d)
    wu = synth.normal_host(6, 5, N * F * d, 0.2, False).reshape(N, F, d)
    wd = synth.normal_host(6, 6, N * d * F, 0.2, False).reshape(N, d, F)
    sh = (wg[0] * 0.5, wu[1] * 0.5, wd[2] * 0.5)
    lg = synth.normal_host(6, 2, T * N, 1.0, False).reshape(T, N)
    idx, gate, _ = oracle.route(lg, M, 1, "grouped")
    ew = lambda e: (wg[e], wu[e], wd[e])
    full = oracle.combine_rows(x, idx, gate, 0, N, ew)
    lo = oracle.combine_rows(x, idx, gate, 0, 4, ew)
    hi = oracle.combine_rows(x, idx, gate, 4, 8, ew)
    assert np.allclose(lo + hi, full, rtol=1e-13, atol=1e-14)
    with_sh = oracle.combine_rows(x, idx, gate, 0, N, ew, sh)
    shared = np.stack([oracle.ffn_row(x[t], *sh) for t in range(T)])
    assert np.allclose(with_sh - full, shared, rtol=1e-12, atol=1e-13)
