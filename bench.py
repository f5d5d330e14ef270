"""Benchmark: MoGE layer forward tokens/s on one MI355X, through the libmoge C ABI.

A step is one pass of the whole hot path over one batch of synthetic input already resident in
HBM: grouped routing (router GEMM + global softmax + top-K' per group), dispatch (counts, offsets,
permutation, row gather), the routed experts' gate/up and down grouped GEMMs, the shared expert,
the gate-weighted combine, the imbalance score, and the global top-K comparator with its score.

Default workload: the Pangu Ultra MoE shape (T=8192 tokens, hidden 7680, 256 routed experts in 8
groups, K'=1, expert width 2048, one shared expert of width 2048, bf16), the largest layer
configuration that runs on one GPU.

Prints ONE JSON line.  The last warm-up step is marked with a HIP event after every library call
(on the stream the kernels run on) to find the dominant call; the K timed steps then carry events
only around that call, so the timed region is the layer with next to no host work added, and its
roofline uses the call's event-measured duration with its algorithmic bytes (weights +
activations it must move) and FLOPs per launch.  The per-stage table comes from K more steps
with every call marked, after the timed region.

With the default workload the same process then measures the metric's other two parts on their
own shapes (key "extra"): the router's HBM rate on the 65536-token x 4096 x 64-expert routing
shape, and the grouped GEMMs' MFMA rate on one device's share of a 65536-token batch (group 0's
8 experts).  The line also carries each expert's share of its group's load (min / mean / max;
1/(N/M) when even) for MoGE and for the global top-K comparator, and the parity statistics of the
CPU-baseline sample (near-tie and flipped tokens, max |y_gpu - y_oracle| against the bar).

    python bench.py [--steps K] [--warmup W] [--workload ultra|group0|decode|routing|tiny|pro]
                    [--tokens T] [--rows auto|gather|copy] [--tiles auto|tall|wide]
                    [--no-cpu-baseline] [--cpu-seconds S] [--no-extra] [--extra-steps K]
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
F32_PEAK_TFLOPS = 157.3        # MI355X fp32 vector, published
METRIC = "MoGE layer tokens/sec at 1 MI355X; MFMA util % and routing HBM GB/s vs peak"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="ultra", choices=["ultra", "group0", "decode", "routing", "tiny", "pro"])
    p.add_argument("--rows", default="auto", choices=["auto", "gather", "copy"],
                   help="gate/up token rows: read from x through perm, or copied by dispatch (auto: the layer's choice)")
    p.add_argument("--tiles", default="auto", choices=["auto", "tall", "wide", "balanced", "tuned"],
                   help="expert-GEMM tile shape: 320x256 (tall), 96x512 (wide), tall with gate/up's columns in "
                        "balanced 128/96-column tiles (balanced), the library's choice (auto), or each GEMM's "
                        "fastest measured on the workload before the timed steps (tuned)")
    p.add_argument("--tokens", type=int, default=0,
                   help="run the workload's shape with this many tokens instead (its name records the count)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the routing-shape router and one-group-share GEMM measurements (ultra only)")
    p.add_argument("--extra-steps", type=int, default=10)
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy (to scale HBM byte counters)")
    p.add_argument("--blas-reference", action="store_true",
                   help="only time the vendor GEMM library (torch.bmm, bf16) on dense batches shaped like "
                        "the Ultra and one-group-share expert GEMMs, for comparison with the grouped kernels")
    return p.parse_args()


def copy_calibration():
    """A plain copy kernel of known size: 1 GiB read + 1 GiB written per launch, 3 launches."""
    import torch

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read_per_launch": n, "bytes_written_per_launch": n, "launches": 3}))


def blas_reference():
    """The vendor library on the expert GEMMs' shapes as dense batches (every expert the average row
    count, contiguous operands, bf16 in and out): what a grouped kernel with ideal load balance and no
    gather, SwiGLU or shared expert would be compared with.  Prints one JSON line."""
    import torch

    def run(name, E, m, k, n, reps=10):
        a = torch.randn(E, m, k, device="cuda").to(torch.bfloat16)
        b = torch.randn(E, k, n, device="cuda").to(torch.bfloat16)   # contiguous right operand
        for _ in range(3):
            torch.bmm(a, b)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            torch.bmm(a, b)
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1000.0 / reps
        flops = 2.0 * E * m * k * n
        del a, b
        torch.cuda.empty_cache()
        return {"gemm": name, "batch": E, "m": m, "k": k, "n": n, "us": round(us, 1),
                "TFLOP/s": round(flops / (us * 1e-6) / 1e12, 1),
                "mfma_frac": round(flops / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)}

    rows = [run("dense square (the library's best case)", 1, 8192, 8192, 8192),
            run("ultra gate/up (gate and up rows as one operand)", 256, 256, 7680, 4096),
            run("ultra down", 256, 256, 2048, 7680),
            run("group-0 share gate/up", 8, 8192, 4096, 2816),
            run("group-0 share down", 8, 8192, 1408, 4096)]
    print(json.dumps({"blas_reference": rows, "library": "torch.bmm (hipBLASLt) bf16"}), flush=True)


def algorithmic_work(w, counts, fused_shared=False, gather=False, fused_combine=False):
    """Bytes and FLOPs each call must move / compute (unique HBM traffic; no re-reads counted).
    gather: dispatch copies no rows and gate/up reads the token rows from x (each row once).
    fused_combine: the down GEMM writes y itself (one row per token, no combine pass)."""
    import numpy as np

    b = 2 if w.dtype == "bf16" else 4
    T, d, N, K, F = w.T, w.d, w.N, w.K, w.F
    counts = np.asarray(counts)
    rng = counts[w.e_lo:w.e_hi]
    R = int(rng.sum())
    active = int((rng > 0).sum())
    work = {}
    # both routers' choices (MoGE and the global comparator) from one pass over x; no scores stored
    work["route"] = dict(bytes=T * d * b + N * d * b + 2 * T * K * 8, flops=2 * T * d * N)
    work["dispatch"] = dict(bytes=T * K * 4 * 3 + (T * d * b + R * d * b if F and not gather else 0), flops=0)
    if F:
        a_bytes = T * d * b if gather else R * d * b
        work["gate_up"] = dict(bytes=active * 2 * F * d * b + a_bytes + R * F * b, flops=2 * R * d * 2 * F)
        work["down"] = dict(bytes=active * d * F * b + R * F * b + R * d * b, flops=2 * R * F * d)
        work["combine"] = dict(bytes=R * d * b + T * d * 4 + T * K * 8 + (T * d * b if w.F_shared else 0), flops=0)
        if fused_combine:
            work["down"] = dict(bytes=active * d * F * b + R * F * b + T * d * 4 + T * 4 + R * 4, flops=2 * R * F * d)
            del work["combine"]
    if w.F_shared:
        Fs = w.F_shared
        gu = dict(bytes=2 * Fs * d * b + (0 if gather else T * d * b) + T * Fs * b, flops=2 * T * d * 2 * Fs)
        dn = dict(bytes=Fs * d * b + T * Fs * b + T * d * b, flops=2 * T * Fs * d)
        if fused_shared:
            # the shared expert runs inside the routed experts' gate/up and down launches
            for stage, extra in (("gate_up", gu), ("down", dn)):
                work[stage] = {k: work[stage][k] + extra[k] for k in ("bytes", "flops")}
        else:
            work["shared"] = {k: gu[k] + dn[k] for k in ("bytes", "flops")}
    return work


# Source files each stage's kernels are built from; a stored HBM byte count is used only while
# these files are unchanged since the counters were taken.
STAGE_SOURCES = {
    "route": ("route.hip", "moge_internal.hpp"),
    "dispatch": ("dispatch.hip", "moge_internal.hpp"),
    "gate_up": ("ggemm.hip", "moge_internal.hpp"),
    "down": ("ggemm.hip", "moge_internal.hpp"),
    "shared": ("ggemm.hip", "moge_internal.hpp"),
    "combine": ("combine.hip", "moge_internal.hpp"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def sources_sha256(stage):
    import hashlib

    h = hashlib.sha256()
    for name in STAGE_SOURCES.get(stage, ()):
        with open(os.path.join(ROOT, "mixture_grouped_experts_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, stage):
    """HBM bytes per launch of `stage` on `workload` from the stored rocprofv3 FETCH_SIZE/WRITE_SIZE
    counts (already scaled by the copy-kernel calibration), or None when there is no record or the
    kernel's sources changed after it was taken."""
    if stage not in STAGE_SOURCES or not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f).get(workload, {}).get(stage)
    if not rec or rec.get("sources_sha256") != sources_sha256(stage):
        return None
    return rec["read_bytes"] + rec["written_bytes"]


def cpu_baseline(w, seconds: float, gpu_idx=None, gpu_y=None):
    """The oracle, as it stands, on a bounded sample of tokens of the same workload (route on the
    sampled tokens' scores + every routed and shared expert they use + the weighted sum).  With the
    GPU's idx and y of the same inputs, the sample's parity statistics are returned as well: the
    tokens whose in-group probability gap is below 1e-5 (near-tie), those routed differently on such
    a gap (flipped, excluded from the y comparison) or on a larger one (hard flips: a failure), and
    the largest |y_gpu - y_oracle| against the bound 1e-2 max|y_oracle| + 1e-3."""
    import numpy as np

    import oracle
    from synth.inputs import HostInputs, sample_tokens

    hi = HostInputs(w)
    wr, bias = hi.w_router(), hi.bias()
    threads = oracle.threads()

    def run(tokens):
        x = hi.x_rows(tokens)
        # generate the experts' weights the sample uses before the timed region
        lg = oracle.logits(x, wr, bias)
        idx, gate, _ = oracle.route(lg, w.M, w.Kp, "grouped")
        for e in np.unique(idx):
            if w.e_lo <= e < w.e_hi:
                hi.expert(int(e))
        t0 = time.perf_counter()
        lg = oracle.logits(x, wr, bias)
        idx, gate, gap = oracle.route(lg, w.M, w.Kp, "grouped")
        y = oracle.combine_rows(x, idx, gate, w.e_lo, w.e_hi, hi.expert, hi.shared()) if w.F else None
        return time.perf_counter() - t0, idx, gap, y

    # size the sample to about `seconds` of oracle time: a small probe, then one correction
    probe = sample_tokens(w.T, 8, seed=7)[:8]
    dt = run(probe)[0]
    n = int(max(2, min(w.T, 4096, seconds / max(dt / len(probe), 1e-9))))
    tokens = sample_tokens(w.T, n, seed=11)[:n]
    dt, idx, gap, yref = run(tokens)
    if dt < 0.6 * seconds and n < min(w.T, 4096):
        n = int(min(w.T, 4096, n * seconds / max(dt, 1e-9)))
        tokens = sample_tokens(w.T, n, seed=11)[:n]
        dt, idx, gap, yref = run(tokens)
    out = {"value": len(tokens) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{len(tokens)} of {w.T} tokens (seeded sample), full layer per token in binary64; "
                     f"{dt:.1f} s"}
    if gpu_idx is not None:
        diff = np.any(gpu_idx[tokens] != idx, axis=1)
        near = gap < 1e-5
        par = {"tokens": int(len(tokens)), "near_tie": int(near.sum()), "flipped": int((diff & near).sum()),
               "hard_flips": int((diff & ~near).sum())}
        if yref is not None and gpu_y is not None:
            keep = ~diff
            ref = yref[keep]
            err = float(np.max(np.abs(gpu_y[tokens][keep].astype(np.float64) - ref))) if ref.size else 0.0
            bound = 1e-2 * float(np.max(np.abs(ref))) + 1e-3 if ref.size else 1e-3
            par.update({"y_max_abs_err": err, "y_bound": bound, "y_within_bound": bool(err <= bound)})
        out["parity"] = par
    return out


def expert_share(counts, w):
    """Each expert's share of its group's assignments, counts[e] / (T K'); MoGE puts exactly T K'
    assignments in every group, so the shares of a group sum to 1 and average 1 / (N/M)."""
    import numpy as np

    c = np.asarray(counts, dtype=np.float64)
    sh = c / float(w.T * w.Kp)
    return {"mean": float(sh.mean()), "min": float(sh.min()), "max": float(sh.max()),
            "uniform": 1.0 / (w.N // w.M)}


def _layer(w, rows="auto", tiles="auto"):
    import torch

    import mixture_grouped_experts_amd as moge
    from mixture_grouped_experts_amd.layer import MoGELayer
    from synth.inputs import device_inputs

    dv = device_inputs(w)
    layer = MoGELayer(w.T, w.d, w.N, w.M, w.Kp, w.F, w.F_shared, w.dtype, w.e_lo, w.e_hi,
                      gather={"auto": None, "gather": True, "copy": False}[rows],
                      tiles={"auto": moge.TILES_AUTO, "tall": moge.TILES_TALL, "wide": moge.TILES_WIDE,
                             "balanced": moge.TILES_BALANCED, "tuned": moge.TILES_AUTO}[tiles])
    if w.F:
        # expert weights are packed once, at load time (outside the timed steps)
        (pg, pu, pd), ps = layer.pack_expert_weights(dv.w_gate, dv.w_up, dv.w_down, dv.shared)
        dv = dataclasses.replace(dv, w_gate=pg, w_up=pu, w_down=pd, shared=ps)
        torch.cuda.synchronize()
        if tiles == "tuned":  # measured once per shape, before any timed step
            layer.tune_tiles(dv.x, dv.w_router, dv.bias, dv.w_gate, dv.w_up, dv.w_down, dv.shared)
    return layer, dv


def _stepper(layer, dv):
    import torch

    stream = torch.cuda.current_stream()

    def step(marks=None, only=None):
        """One layer forward; with `marks`, a stream event after each library call (or only after
        the calls named in `only`)."""
        rec = None
        if marks is not None:
            def rec(name):
                if only is None or name in only:
                    ev = torch.cuda.Event(enable_timing=True)
                    ev.record(stream)
                    marks.append((name, ev))
        layer.forward(dv.x, dv.w_router, dv.bias, dv.w_gate, dv.w_up, dv.w_down, dv.shared, mark=rec)

    def run_marked(n, only=None):
        """n steps, each with a begin event and the requested marks; returns their per-stage times (ms)."""
        per = []
        for _ in range(n):
            ev0 = torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            marks = [("begin", ev0)]
            step(marks, only)
            per.append(marks)
        torch.cuda.synchronize()
        out = {}
        for marks in per:
            for (n0, e0), (n1, e1) in zip(marks[:-1], marks[1:]):
                out.setdefault(n1, []).append(e0.elapsed_time(e1))
        return out
    return stream, step, run_marked


def _stage_table(stage_us, work):
    stages = {}
    for k, us in stage_us.items():
        entry = {"us": round(us, 2)}
        if k in work:
            wk = work[k]
            entry["GB/s"] = round(wk["bytes"] / (us * 1e-6) / 1e9, 1)
            if wk["flops"]:
                entry["TFLOP/s"] = round(wk["flops"] / (us * 1e-6) / 1e12, 1)
                entry["mfma_frac"] = round(wk["flops"] / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)
            entry["hbm_frac"] = round(wk["bytes"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        stages[k] = entry
    return stages


def side_workload(w, steps, warmup, keys):
    """The stages `keys` of another workload's layer, measured in the same process (every call
    marked, `steps` steps after `warmup`): what the metric asks for beside the main workload's
    tokens/s -- the router's HBM rate at the routing shape, the grouped GEMMs' MFMA rate at the
    one-group share."""
    import numpy as np
    import torch

    layer, dv = _layer(w)
    _, step, run_marked = _stepper(layer, dv)
    for _ in range(warmup):
        step()
    times = run_marked(steps)
    work = algorithmic_work(w, layer.counts.cpu().numpy(), fused_shared=bool(w.F_shared) and layer.fuse_shared,
                            gather=layer.gather, fused_combine=layer.fuse_combine)
    stage_us = {k: 1000.0 * float(np.mean(v)) for k, v in times.items() if k in keys}
    out = {"workload": w.name, "steps": steps, "stages": _stage_table(stage_us, work),
           "per_expert_share": expert_share(layer.counts.cpu().numpy()[w.e_lo:w.e_hi], w),
           "imbalance": {"moge_is_raw": int(layer.is_raw.item()),
                         "global_topk_is_raw": int(layer.g_is_raw.item())}}
    if w.e_hi - w.e_lo == w.N:
        out["per_expert_share_global_topk"] = expert_share(layer.gcounts.cpu().numpy(), w)
    if not w.F:
        # the MoGE router alone (moge_route, no comparator, no stored scores): x read once, the
        # choice written, between reads of a 512 MiB buffer so x comes from HBM each time
        import mixture_grouped_experts_amd as moge

        flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
        ts = []
        for rep in range(steps + warmup):
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            moge.route(layer.shape, moge.ROUTE_GROUPED, dv.x, dv.w_router, dv.bias, None, layer.idx, layer.gate,
                       layer.rws)
            b.record()
            torch.cuda.synchronize()
            if rep >= warmup:
                ts.append(a.elapsed_time(b) * 1000.0)
        us = float(np.median(ts))
        nbytes = w.T * w.d * 2 + w.N * w.d * 2 + w.T * w.K * 8
        out["router_alone"] = {"us": round(us, 2), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                               "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                               "algorithmic_bytes": nbytes}
        del flush
    del layer, dv
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the expert-parallel "
              f"sharding of the layer over several GPUs is described, not implemented", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return
    if args.blas_reference:
        blas_reference()
        return

    import numpy as np
    import torch

    import mixture_grouped_experts_amd as moge
    from synth import workloads as W

    w = {"ultra": W.ultra, "group0": W.group0, "decode": W.decode, "routing": W.routing, "tiny": W.tiny,
         "pro": W.pro}[
        args.workload]()
    if args.tokens:
        import re

        w = W.variant(w, T=args.tokens, e_lo=w.e_lo, e_hi=w.e_hi,
                      name=re.sub(r"_T\d+_", f"_T{args.tokens}_", w.name))
    torch.cuda.set_device(0)
    layer, dv = _layer(w, args.rows, args.tiles)
    stream, step, run_marked = _stepper(layer, dv)

    for _ in range(max(args.warmup - 1, 0)):
        step()
    # one marked warm-up step names the dominant stage and the call before it
    probe = run_marked(1)
    counts = layer.counts.cpu().numpy()
    work = algorithmic_work(w, counts, fused_shared=bool(w.F_shared) and layer.fuse_shared, gather=layer.gather,
                            fused_combine=layer.fuse_combine)
    order = list(probe)
    dom = max((k for k in work if k in probe), key=lambda k: probe[k][0])
    prev = order[order.index(dom) - 1] if order.index(dom) > 0 else "begin"

    # the timed region: exactly K steps with events only around the dominant stage's call (two
    # per step; each event is a packet in the stream, so no more are recorded than that needs)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    per_step = []
    for _ in range(args.steps):
        marks = []
        if prev == "begin":
            ev0 = torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            marks.append(("begin", ev0))
        step(marks, only={prev, dom})
        per_step.append(marks)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    dom_ms = []
    for marks in per_step:
        names = [n for n, _ in marks]
        e0 = marks[names.index(prev)][1]
        e1 = marks[names.index(dom)][1]
        dom_ms.append(e0.elapsed_time(e1))
    ms_per_step = total_ms / args.steps
    value = w.T * args.steps / (total_ms / 1000.0)

    # the per-stage table from K more steps with every call marked (outside the timed region)
    stage_us = {k: 1000.0 * float(np.mean(v)) for k, v in run_marked(args.steps).items()}
    stage_us[dom] = 1000.0 * float(np.mean(dom_ms))  # the dominant stage as timed inside the timed region
    t = stage_us[dom] * 1e-6
    wb, wf = work[dom]["bytes"], work[dom]["flops"]
    inten = wf / wb if wb else 0.0
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if wf and inten >= ridge:
        roof = {"bound": "mfma", "achieved": wf / t / 1e12, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": wb / t / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(w.name, dom)  # HBM bytes per launch (rocprofv3 counters)
    roof["kernel"] = dom
    roof["algorithmic_bytes"] = wb
    roof["algorithmic_flops"] = wf
    roof["avg_us"] = stage_us[dom]
    roof["mfma_frac"] = wf / t / 1e12 / BF16_PEAK_TFLOPS if wf else None

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "N": w.N, "M": w.M, "k_per_group": w.Kp, "F": w.F,
                   "F_shared": w.F_shared, "experts_computed": [w.e_lo, w.e_hi], "seed": w.seed,
                   "rows": "gather" if layer.gather else "copy",
                   "tiles": ({g: {moge.TILES_TALL: "tall", moge.TILES_WIDE: "wide",
                                  moge.TILES_BALANCED: "balanced"}.get(
                                  moge.tile_choice(shp, i, w.e_lo, w.e_hi, w.F_shared), "none")
                              for i, g, shp in ((1, "gate_up", layer.shape_up), (2, "down", layer.shape_down))}
                             if w.F else None)},
        "roofline": roof,
        "stages": _stage_table(stage_us, work),
        "imbalance": {"moge_is_raw": int(layer.is_raw.item()),
                      "global_topk_is_raw": int(layer.g_is_raw.item()) if layer.comparator else None},
        "per_expert_share": expert_share(counts[w.e_lo:w.e_hi], w),
    }
    if layer.comparator and w.e_hi - w.e_lo == w.N:
        out["per_expert_share_global_topk"] = expert_share(layer.gcounts.cpu().numpy(), w)
    gpu_idx = layer.idx.cpu().numpy()
    gpu_y = layer.y.cpu().numpy() if w.F else None
    del layer, dv
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_extra and args.workload == "ultra" and not args.tokens:
        # the metric's other two parts, on their own workloads, in this same process
        out["extra"] = {
            "routing_router": side_workload(W.routing(), args.extra_steps, 3, {"route", "dispatch",
                                                                                "global_comparator"}),
            "group0_gemms": side_workload(W.group0(), args.extra_steps, 3, {"gate_up", "down", "dispatch",
                                                                             "route"}),
        }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, gpu_idx, gpu_y)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
