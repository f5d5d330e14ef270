"""The layer forward recorded in a HIP graph (MoGELayer.capture): every replay gives exactly the
eager result, with eager work and synchronisations between replays, and a replay after the inputs
are refilled in place gives the eager result on the new inputs."""
import pytest
import torch

import synth
from mixture_grouped_experts_amd.layer import MoGELayer
from synth import workloads as W
from tests import moge_harness as H
from tests.test_gpu_layer import packed_inputs

pytestmark = pytest.mark.gpu


def _state(layer):
    return [t.clone() for t in (layer.y, layer.idx, layer.gate, layer.counts, layer.offsets, layer.is_raw,
                                layer.g_is_raw, layer.gcounts)]


@pytest.mark.parametrize("w", [
    W.decode(),
    W.variant(W.decode(), name="graph_shared_T300_d256", T=300, d=256, N=32, M=4, Kp=1, F=136, F_shared=264,
              std_shared_down=0.02),
    W.variant(W.decode(), name="graph_group_fused", T=400, Kp=1, e_lo=8, e_hi=16, std_bias=1.0),
], ids=lambda w: w.name)
def test_graph_replays_match_eager(gpu, w):
    layer = MoGELayer(w.T, w.d, w.N, w.M, w.Kp, w.F, w.F_shared, w.dtype, w.e_lo, w.e_hi)
    dv = packed_inputs(w, layer)
    args = (dv.x, dv.w_router, dv.bias, dv.w_gate, dv.w_up, dv.w_down, dv.shared)
    layer.forward(*args)
    torch.cuda.synchronize()
    ref = _state(layer)
    g = layer.capture(*args)
    for i in range(3):
        layer.y.fill_(float("nan"))          # eager work between replays
        layer.idx.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, _state(layer)):
            assert H.same_bits(a, b), i
        layer.forward(*args)                 # an eager forward between replays
        torch.cuda.synchronize()
    # inputs are bound by address: refill x in place, replay, compare with eager on the new x
    x2 = torch.empty_like(dv.x)
    synth.fill_device(x2, 99, 1, 1.0)
    dv.x.copy_(x2)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    got = _state(layer)
    layer.forward(*args)
    torch.cuda.synchronize()
    for a, b in zip(_state(layer), got):
        assert H.same_bits(a, b)
