"""GPU parity of the whole layer forward (route -> dispatch -> grouped FFN -> shared -> combine ->
imbalance, plus the global top-K comparator) through the C ABI, against the oracle.

Bar (bf16 in, float32 accumulate): max|y_gpu - y_ref| <= 1e-2 * max|y_ref| + 1e-3 over the compared
tokens.  Tokens whose K'-th vs (K'+1)-th in-group softmax gap is below 1e-5 are counted; if such a
token's choice flips it is excluded from the y check (reported), any other flip fails."""
import dataclasses

import numpy as np
import pytest
import torch

import mixture_grouped_experts_amd as moge
from mixture_grouped_experts_amd.layer import MoGELayer
import oracle
from synth import workloads as W
from tests import moge_harness as H

pytestmark = pytest.mark.gpu


def packed_inputs(w, layer):
    """Device inputs with the expert weights packed once (the row-major copies are dropped)."""
    dv = H.device_inputs(w)
    if w.F:
        (pg, pu, pd), ps = layer.pack_expert_weights(dv.w_gate, dv.w_up, dv.w_down, dv.shared)
        dv = dataclasses.replace(dv, w_gate=pg, w_up=pu, w_down=pd, shared=ps)
    return dv


def run_layer(w):
    layer = MoGELayer(w.T, w.d, w.N, w.M, w.Kp, w.F, w.F_shared, w.dtype, w.e_lo, w.e_hi)
    dv = packed_inputs(w, layer)
    y = layer.forward(dv.x, dv.w_router, dv.bias, dv.w_gate, dv.w_up, dv.w_down, dv.shared)
    torch.cuda.synchronize()
    return dv, layer, y


def check_layer(w, n_sample=None):
    print(f"[layer] {w.name}", flush=True)
    dv, layer, y = run_layer(w)
    hi = H.HostInputs(w)
    lg = H.oracle_logits_all(hi)
    ridx, rgate, rgap = oracle.route(lg, w.M, w.Kp, "grouped")
    gidx = layer.idx.cpu().numpy()
    n_near, flipped, hard = H.compare_routing(w, gidx, ridx, rgap, H.order_gap(lg, w.M, w.Kp))
    print(f"  near-tie {n_near}, flipped {len(flipped)}", flush=True)
    assert hard.size == 0
    # imbalance: MoGE 0 by construction, group loads T*K'; the global comparator on the same scores
    assert int(layer.is_raw.item()) == 0
    assert (layer.group_load.cpu().numpy() == w.T * w.Kp).all()
    assert layer.is_norm.item() == 0.0
    rgidx, _, _ = oracle.route(lg, w.M, w.Kp, "global")
    _, g_isr_ref = oracle.imbalance(np.bincount(rgidx.ravel(), minlength=w.N), w.M)
    g_isr = int(layer.g_is_raw.item())
    print(f"  global top-K imbalance: gpu {g_isr} oracle {g_isr_ref}", flush=True)
    if w.routing_only:
        return layer, None
    tokens = np.arange(w.T) if n_sample is None else H.sample_tokens(w.T, n_sample)
    tokens = np.array([t for t in tokens if t not in set(flipped.tolist())])
    ref = oracle.combine_rows(hi.x_rows(tokens), ridx[tokens], rgate[tokens], w.e_lo, w.e_hi, hi.expert,
                              hi.shared())
    got = y[torch.from_numpy(tokens).long().cuda()].cpu().numpy()
    ok, err, bound = H.tol_ok(got, ref)
    print(f"  y: max err {err:.3e} bound {bound:.3e} over {len(tokens)} tokens", flush=True)
    assert ok
    return layer, y


def test_layer_tiny_fp32(gpu):
    layer, y = check_layer(W.tiny())
    assert int(layer.g_is_raw.item()) > 0   # conventional top-4 is unbalanced on the same scores (seed 0)


def test_layer_mid_ragged(gpu):
    w = W.variant(W.decode(), name="mid", T=1000, d=520, N=16, M=4, Kp=2, F=200, std_bias=1.0)
    check_layer(w)


def test_layer_mid_shared_and_range(gpu):
    w = W.variant(W.decode(), name="mid_shared", T=257, d=256, N=32, M=4, Kp=1, F=136, F_shared=264,
                            e_lo=8, e_hi=16, std_shared_down=0.02)
    check_layer(w)


def test_layer_shared_tiled_rows(gpu):
    # hidden size not a multiple of 32: dispatch copies the rows (tiled x_perm and x) for the fused launches
    w = W.variant(W.decode(), name="mid_shared_d264", T=257, d=264, N=32, M=4, Kp=1, F=136, F_shared=264,
                  std_shared_down=0.02)
    layer, _ = check_layer(w)
    assert not layer.gather


def test_layer_one_group_combined_in_gemm(gpu):
    # one device's share of one group with K' = 1: GEMM 2 writes y (no combine pass)
    w = W.variant(W.decode(), name="group1_fused", T=300, Kp=1, e_lo=8, e_hi=16, std_bias=1.0)
    layer, _ = check_layer(w)
    assert layer.fuse_combine and layer.o is None


def test_layer_decode(gpu):
    check_layer(W.decode())


def test_layer_routing_only(gpu):
    w = W.routing()
    layer, _ = check_layer(w)
    assert int(layer.g_is_raw.item()) > 0


# the full-size workloads (Ultra, the one-group share of 65536 tokens, Pro) are checked row by row in
# test_gpu_fullsize.py


@pytest.mark.parametrize("T", [1, 15, 17])
def test_layer_few_tokens(gpu, T):
    # fewer tokens than one 16-row tile, one past it; every expert segment is padded
    check_layer(W.variant(W.decode(), name=f"few_T{T}", T=T, F_shared=264, std_shared_down=0.02))


def test_layer_one_expert_range(gpu):
    w = W.variant(W.decode(), name="one_expert", T=400, Kp=1, e_lo=37, e_hi=38, std_bias=1.0)
    check_layer(w)


def test_layer_empty_expert_range(gpu):
    # a computed range that no token chooses: every GEMM's routed tile list is empty, and y is
    # the shared expert's output alone, or all zeros without one
    base = W.variant(W.decode(), name="empty_range", T=300, Kp=1, std_bias=20.0, F_shared=264,
                     std_shared_down=0.02)
    ridx, _, _ = oracle.route(H.oracle_logits_all(H.HostInputs(base)), base.M, base.Kp, "grouped")
    empty = np.flatnonzero(np.bincount(ridx.ravel(), minlength=base.N) == 0)
    assert empty.size, "a bias of std 20 leaves some experts unchosen"
    e = int(empty[0])
    for fs in (264, 0):
        w = W.variant(base, name=f"empty_range_e{e}_Fs{fs}", e_lo=e, e_hi=e + 1, F_shared=fs)
        layer, y = check_layer(w)
        assert int(layer.counts[e].item()) == 0
        if not fs:
            assert bool((y == 0).all())


def test_layer_deterministic(gpu):
    w = W.variant(W.decode(), name="det", T=600, std_bias=2.0)
    layer = MoGELayer(w.T, w.d, w.N, w.M, w.Kp, w.F, 0, "bf16")
    dv = packed_inputs(w, layer)
    outs = []
    for _ in range(2):
        y = layer.forward(dv.x, dv.w_router, dv.bias, dv.w_gate, dv.w_up, dv.w_down)
        torch.cuda.synchronize()
        outs.append((y.clone(), layer.idx.clone(), layer.inv.clone(), layer.perm.clone(), layer.h.clone(),
                     layer.o.clone()))
    for a, b in zip(*outs):
        assert H.same_bits(a, b)


def test_abi_errors_on_gpu(gpu):
    s = moge.Shape(64, 128, 8, 4, 1, 64, moge.BF16)
    with pytest.raises(moge.MogeError, match="ARG"):
        moge.route(s, 7, None, None, None, torch.zeros(64, 8, device="cuda"),
                   torch.zeros(64, 4, dtype=torch.int32, device="cuda"), torch.zeros(64, 4, device="cuda"))
    with pytest.raises(moge.MogeError, match="ARG"):
        moge.route(s, 0, None, None, torch.zeros(8, device="cuda"), torch.zeros(64, 8, device="cuda"),
                   torch.zeros(64, 4, dtype=torch.int32, device="cuda"), torch.zeros(64, 4, device="cuda"))


def test_layer_every_expert_chosen(gpu):
    # K' = N/M at 256 experts: the dense softmax mixture of all experts (K = 256 slots per token)
    w = W.variant(W.decode(), name="dense_N256_M8_K32", T=40, d=256, N=256, M=8, Kp=32, F=64, std_bias=1.0)
    layer, y = check_layer(w)
    assert (layer.counts.cpu().numpy() == w.T).all()
    # the gates of a token are its whole softmax: they sum to 1
    assert np.allclose(layer.gate.sum(1).cpu().numpy(), 1.0, atol=1e-5)


def test_layer_check_scores(gpu):
    w = W.variant(W.decode(), name="check_T64", T=64, d=256, N=16, M=4, Kp=1, F=64)
    layer = MoGELayer(w.T, w.d, w.N, w.M, w.Kp, w.F, 0, "bf16", store_scores=True)
    dv = packed_inputs(w, layer)
    layer.forward(dv.x, dv.w_router, dv.bias, dv.w_gate, dv.w_up, dv.w_down)
    layer.check_scores()                         # finite scores pass
    layer.logits[3, 5] = float("nan")
    with pytest.raises(moge.MogeError, match="NONFINITE"):
        layer.check_scores()


def _random_shapes(n, seed):
    """Seeded layer shapes across the validated range: N up to 256 with every group size,
    K' from 1 to the group size, hidden sizes on and off the 32-column grid (the gathered and
    the copied token rows), narrow and ragged expert widths, routing-only layers, shared experts,
    expert ranges, both dtypes and a skewing router bias."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        N = int(rng.choice([1, 8, 12, 16, 40, 64, 96, 128, 200, 256]))
        divs = [m for m in range(1, min(N, 8) + 1) if N % m == 0]
        M = int(rng.choice(divs))
        Kp = int(rng.integers(1, min(N // M, 4) + 1))
        T = int(rng.choice([1, 7, 63, 300, 777, 1500]))
        d = int(8 * rng.integers(1, 65))                      # 8 .. 512
        F = int(rng.choice([0, 8 * int(rng.integers(1, 49))]))  # routing only, or 8 .. 384
        dtype = "f32" if rng.random() < 0.2 else "bf16"
        Fs = int(8 * rng.integers(1, 33)) if F and rng.random() < 0.3 else 0
        lo = int(rng.integers(0, N))
        hi = int(rng.integers(lo + 1, N + 1))
        out.append(W.variant(W.decode(), name=f"rand{seed}_{i}_T{T}_d{d}_N{N}_M{M}_K{Kp}_F{F}_S{Fs}_{dtype}_{lo}_{hi}",
                             T=T, d=d, N=N, M=M, Kp=Kp, F=F, F_shared=Fs, dtype=dtype,
                             std_bias=float(rng.choice([0.0, 1.0, 3.0])), std_shared_down=0.02 if Fs else 0.0,
                             e_lo=lo, e_hi=hi, seed=int(seed * 100 + i)))
    return out


@pytest.mark.parametrize("w", _random_shapes(16, 7) + _random_shapes(16, 11), ids=lambda w: w.name)
def test_layer_random_shapes(gpu, w):
    # every token against the oracle on seeded shapes drawn across the validated range
    check_layer(w)


TUNE_CASES = [W.variant(W.decode(), name="tune_T300_d256_shared", T=300, d=256, N=32, M=4, Kp=1, F=136, F_shared=264,
                        std_shared_down=0.02),
              W.variant(W.decode(), name="tune_T200_d264_copy", T=200, d=264, N=16, M=4, Kp=2, F=200)]


@pytest.mark.parametrize("w", TUNE_CASES, ids=lambda w: w.name)
def test_tune_tiles_measured_choice(gpu, w):
    # the measured tile choice (per GEMM, cached per shape) changes the kernels' tiles only: y stays
    # bit-identical to the library's own choice, and a second layer of the shape reuses the result
    import mixture_grouped_experts_amd.layer as layer_mod
    print(f"[tune tiles] {w.name}", flush=True)
    _, ref_layer, y_ref = run_layer(w)
    layer = MoGELayer(w.T, w.d, w.N, w.M, w.Kp, w.F, w.F_shared, w.dtype, w.e_lo, w.e_hi)
    dv = packed_inputs(w, layer)
    args = (dv.x, dv.w_router, dv.bias, dv.w_gate, dv.w_up, dv.w_down, dv.shared)
    before = len(layer_mod._TILE_CACHE)
    up, down = layer.tune_tiles(*args, reps=3)
    assert up in (moge.TILES_TALL, moge.TILES_WIDE, moge.TILES_BALANCED)
    assert down in (moge.TILES_TALL, moge.TILES_WIDE)
    assert (layer.shape_up.tiles, layer.shape_down.tiles) == (up, down)
    assert len(layer_mod._TILE_CACHE) == before + 1
    y = layer.forward(*args)
    torch.cuda.synchronize()
    assert H.same_bits(y, y_ref)
    other = MoGELayer(w.T, w.d, w.N, w.M, w.Kp, w.F, w.F_shared, w.dtype, w.e_lo, w.e_hi)
    calls = []
    real_forward = other.forward
    other.forward = lambda *a, **k: (calls.append(1), real_forward(*a, **k))[1]
    assert other.tune_tiles(*args) == (up, down) and not calls      # cached: nothing is timed again
    assert len(layer_mod._TILE_CACHE) == before + 1
