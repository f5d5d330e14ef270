"""One MoGE layer forward as a sequence of libmoge C-ABI calls on one stream.

Order (Pangu Pro MoE, lsdiaocha.cn summary, section 1; Pangu Ultra MoE digests on
reportify.cn for the shared expert):

  1. moge_route_pair     scores, softmax over all N, top-K' in every group (MoGE) and, from the
                          same scores in the same pass, the conventional global top-K comparator
  2. moge_dispatch        counts, offsets, stable permutation of [e_lo, e_hi); the rows
                          themselves are copied (tiled x_perm, and the tiled x for the
                          shared expert) only where step 3 cannot read them from x
  3. moge_expert_gate_up_gather, moge_expert_down(_with_shared)
                          SwiGLU experts on their row segments, the gate/up GEMM reading
                          each row straight from x through perm, and the always-on shared
                          expert over all tokens in the same two launches (bf16 with
                          d % 32 == 0); other bf16 shapes use the tiled x_perm with
                          moge_expert_gate_up_with_shared; float32 shapes use
                          moge_expert_gate_up / _down and a one-expert moge_grouped_ffn for
                          the shared expert
  4. moge_combine         gate-weighted sum (+ shared output) -> y (float32); for one whole group
                          with K' = 1 and no shared expert GEMM 2 writes y itself
                          (moge_expert_down_combine)
  5. moge_imbalance       per-group load and imbalance score (0 by construction)
  6. moge_dispatch        the comparator's counts only, and moge_imbalance of that load -- with
     moge_imbalance       expert FFNs, on a second stream: it starts when step 1's choices exist
                          and overlaps steps 2-5 (its calls are enqueued after step 2's, so the
                          GPU never waits on them).  Without the comparator step 1 is moge_route.

The scores themselves are stored only when asked for (``store_scores``): neither router needs them
once step 1 has run.

Tile shapes of the two expert GEMMs: the library picks them from the call's shape (a cost table,
``moge_tile_choice``) unless the call's ``tiles`` field forces one.  ``tune_tiles`` replaces the
table by measurement, as the grouped matmul of the pages does (Pangu Pro MoE, lsdiaocha.cn summary,
section 3: tilings cached per shape from profiling, and a switch of mode by workload): it times each
GEMM of this layer under every tile shape on the real routed rows and keeps the fastest, per
process, keyed by the layer's shape.  All tile shapes give bit-identical outputs, so tuning changes
time only.

Buffers are allocated once here (torch supplies device memory); ``forward`` only issues
library calls, so it allocates nothing and does not synchronise.  Expert weights are
passed packed (``pack_expert_weights``, once, when they are loaded).
"""
from __future__ import annotations

import torch

from . import _lib as L

# Measured tile shapes, keyed by everything that decides a layer's GEMM problems and the device:
# (T, d, N, M, K', F, F_shared, dtype, e_lo, e_hi, gather, device name, CUs) -> (gate/up, down).
_TILE_CACHE: dict = {}


class MoGELayer:
    def __init__(self, T: int, d: int, N: int, M: int, Kp: int, F: int, F_shared: int = 0, dtype: str = "bf16",
                 e_lo: int = 0, e_hi: int | None = None, device="cuda", comparator: bool = True,
                 gather: bool | None = None, tiles: int = L.TILES_AUTO, store_scores: bool = False):
        self.dtype_code = L.BF16 if dtype == "bf16" else L.F32
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.shape = L.Shape(T, d, N, M, Kp, F, self.dtype_code, tiles)
        # the two expert GEMMs' calls carry their own tile shape (tune_tiles may set them apart)
        self.shape_up = L.Shape(T, d, N, M, Kp, F, self.dtype_code, tiles)
        self.shape_down = L.Shape(T, d, N, M, Kp, F, self.dtype_code, tiles)
        st = L.validate(self.shape)
        if st != 0:
            raise L.MogeError("moge_validate", st, L.last_error())
        self.T, self.d, self.N, self.M, self.Kp, self.F = T, d, N, M, Kp, F
        self.K = M * Kp
        self.e_lo, self.e_hi = e_lo, (N if e_hi is None else e_hi)
        self.F_shared = F_shared
        self.fuse_shared = dtype == "bf16"  # the fused routed + shared launches are bf16 only
        # gate/up reads the token rows from x through perm (no row copy); None: wherever it can
        can_gather = dtype == "bf16" and d % 32 == 0 and F > 0
        if gather and not can_gather:
            raise ValueError("reading rows through perm needs bf16, d % 32 == 0 and F > 0")
        self.gather = can_gather if gather is None else bool(gather)
        # one whole group with K' = 1 and no shared expert: every token owns exactly one row, so
        # GEMM 2's epilogue writes y itself (moge_expert_down_combine) and no combine pass runs
        G = N // M
        self.fuse_combine = (dtype == "bf16" and F > 0 and not F_shared and Kp == 1 and self.e_lo % G == 0
                             and self.e_hi == self.e_lo + G)
        self.comparator = comparator
        self.routing_only = F == 0
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        K = self.K
        self.logits = torch.empty(T, N, **f32) if store_scores else None
        rws = L.workspace_size(self.shape, L.STAGE_ROUTE)
        self.rws = torch.empty(rws, dtype=torch.uint8, device=dev) if rws else None
        self.idx = torch.empty(T, K, **i32)
        self.gate = torch.empty(T, K, **f32)
        self.counts = torch.empty(N, **i32)
        self.offsets = torch.empty(N + 1, **i32)
        self.ws = torch.empty(max(L.workspace_size(self.shape), 4), dtype=torch.uint8, device=dev)
        self.group_load = torch.empty(M, **i32)
        self.is_raw = torch.empty(1, **i32)
        self.is_norm = torch.empty(1, dtype=torch.float64, device=dev)
        if comparator:
            # the comparator only needs the stored scores: with expert FFNs to hide behind it
            # runs on a second stream (default priority), with a workspace of its own
            self.side = torch.cuda.Stream(device=dev) if F else None
            self.route_done = torch.cuda.Event() if F else None
            self.gws = torch.empty(max(L.workspace_size(self.shape), 4), dtype=torch.uint8, device=dev)
            self.gidx = torch.empty(T, K, **i32)
            self.ggate = torch.empty(T, K, **f32)
            self.gcounts = torch.empty(N, **i32)
            self.goffsets = torch.empty(N + 1, **i32)
            self.g_group_load = torch.empty(M, **i32)
            self.g_is_raw = torch.empty(1, **i32)
            self.g_is_norm = torch.empty(1, dtype=torch.float64, device=dev)
        if not self.routing_only:
            self.rows_cap = L.rows_bound(self.shape, L.ROUTE_GROUPED, self.e_lo, self.e_hi)
            R = self.rows_cap
            self.inv = torch.empty(T, K, **i32)
            self.perm = torch.empty(R, **i32)
            self.x_perm = None if self.gather else torch.empty(L.tiled_elems(R, d), dtype=self.tdtype, device=dev)
            self.h = torch.empty(L.tiled_elems(R, F), dtype=self.tdtype, device=dev)
            self.o = None if self.fuse_combine else torch.empty(R, d, dtype=self.tdtype, device=dev)
            self.y = torch.empty(T, d, **f32)
        if F_shared:
            self.sshape = L.Shape(T, d, 1, 1, 1, F_shared, self.dtype_code, tiles)
            self.soffsets = torch.tensor([0, T], **i32)
            self.x_tiled = None if self.gather else torch.empty(L.tiled_elems(T, d), dtype=self.tdtype, device=dev)
            self.sh = torch.empty(L.tiled_elems(T, F_shared), dtype=self.tdtype, device=dev)
            self.so = torch.empty(T, d, dtype=self.tdtype, device=dev)

    def pack_expert_weights(self, w_gate, w_up, w_down, shared=None, stream=None):
        """Row-major expert weights ([E][F][d], [E][F][d], [E][d][F]; shared: three 2-d matrices)
        -> packed tensors for ``forward``.  Done once, when the weights are loaded."""
        def pack(w):
            w3 = w if w.dim() == 3 else w.unsqueeze(0)
            out = torch.empty(w3.shape[0] * L.packed_weight_elems(w3.shape[1], w3.shape[2]), dtype=w.dtype,
                              device=w.device)
            L.pack_weights(self.dtype_code, w3, out, stream)
            return out
        packed = (pack(w_gate), pack(w_up), pack(w_down))
        return packed, (tuple(pack(m) for m in shared) if shared is not None else None)

    def forward(self, x, w_router, bias, w_gate=None, w_up=None, w_down=None, shared=None, stream=None, mark=None):
        """Enqueues the layer on `stream` (default: current).  Returns y (None for routing only).
        w_gate, w_up, w_down and the shared expert's three matrices are packed weights.

        `mark(name)`, if given, is called right after each library call is enqueued (a timing hook:
        the caller may record a stream event there)."""
        s = self.shape
        mk = mark if mark is not None else (lambda name: None)
        main = stream if stream is not None else torch.cuda.current_stream()
        if self.comparator:
            L.route_pair(s, x, w_router, bias, self.logits, self.idx, self.gate, self.gidx, self.ggate, self.rws,
                         main)
        else:
            L.route(s, L.ROUTE_GROUPED, x, w_router, bias, self.logits, self.idx, self.gate, self.rws, main)
        mk("route")
        def comparator(on):
            # the conventional global top-K's loads (its choice came with the scores) and imbalance
            L.dispatch(s, L.ROUTE_GLOBAL, self.gidx, None, 0, self.N, 0, self.gcounts, self.goffsets, None, None,
                       None, self.gws, stream=on)
            L.imbalance(s, self.gcounts, self.g_group_load, self.g_is_raw, self.g_is_norm, on)
        side = self.side if self.comparator else None
        if side is not None:
            self.route_done.record(main)  # the comparator needs only its choice

        def side_comparator():
            # enqueued after the layer's own dispatch, so the GPU never waits on these host calls;
            # it runs beside the layer from the moment the scores exist and is joined at the end
            if side is not None:
                side.wait_event(self.route_done)
                comparator(side)
        stream = main
        if self.routing_only:
            L.dispatch(s, L.ROUTE_GROUPED, self.idx, None, 0, self.N, 0, self.counts, self.offsets, None, None, None,
                       self.ws, stream=stream)
            mk("dispatch")
        else:
            if self.gather:
                L.dispatch(s, L.ROUTE_GROUPED, self.idx, None, self.e_lo, self.e_hi, self.rows_cap, self.counts,
                           self.offsets, self.inv, self.perm, None, self.ws, None, stream)
                mk("dispatch")
                side_comparator()
                Fs = self.F_shared
                L.expert_gate_up_gather(self.shape_up, x, self.perm, self.offsets, self.e_lo, self.e_hi,
                                        self.rows_cap, w_gate, w_up, self.h, Fs, shared[0] if Fs else None,
                                        shared[1] if Fs else None, self.sh if Fs else None, stream)
                mk("gate_up")
                if Fs:
                    L.expert_down_with_shared(self.shape_down, Fs, self.h, self.offsets, self.e_lo, self.e_hi,
                                              self.rows_cap, w_down, self.o, self.sh, shared[2], self.so, stream)
                elif self.fuse_combine:
                    L.expert_down_combine(self.shape_down, self.h, self.offsets, self.e_lo, self.e_hi, self.rows_cap,
                                          w_down, self.perm, self.gate, self.y, stream)
                else:
                    L.expert_down(self.shape_down, self.h, self.offsets, self.e_lo, self.e_hi, self.rows_cap, w_down,
                                  self.o, stream)
                mk("down")
            else:
                L.dispatch(s, L.ROUTE_GROUPED, self.idx, x, self.e_lo, self.e_hi, self.rows_cap, self.counts,
                           self.offsets, self.inv, self.perm, self.x_perm, self.ws,
                           self.x_tiled if self.F_shared else None, stream)
                mk("dispatch")
                side_comparator()
                if self.F_shared and self.fuse_shared:
                    # routed and shared experts in the same two launches
                    L.expert_gate_up_with_shared(self.shape_up, self.F_shared, self.x_perm, self.offsets,
                                                 self.e_lo, self.e_hi, self.rows_cap, w_gate, w_up, self.h,
                                                 self.x_tiled, shared[0], shared[1], self.sh, stream)
                    mk("gate_up")
                    L.expert_down_with_shared(self.shape_down, self.F_shared, self.h, self.offsets, self.e_lo,
                                              self.e_hi, self.rows_cap, w_down, self.o, self.sh, shared[2], self.so,
                                              stream)
                    mk("down")
                else:
                    L.expert_gate_up(self.shape_up, self.x_perm, self.offsets, self.e_lo, self.e_hi, self.rows_cap,
                                     w_gate, w_up, self.h, stream)
                    mk("gate_up")
                    if self.fuse_combine:
                        L.expert_down_combine(self.shape_down, self.h, self.offsets, self.e_lo, self.e_hi,
                                              self.rows_cap, w_down, self.perm, self.gate, self.y, stream)
                    else:
                        L.expert_down(self.shape_down, self.h, self.offsets, self.e_lo, self.e_hi, self.rows_cap,
                                      w_down, self.o, stream)
                    mk("down")
                    if self.F_shared:
                        L.grouped_ffn(self.sshape, self.x_tiled, self.soffsets, 0, 1, self.T, shared[0], shared[1],
                                      shared[2], self.sh, self.so, stream)
                        mk("shared")
            if not self.fuse_combine:
                L.combine(s, self.o, self.inv, self.gate, self.rows_cap, self.so if self.F_shared else None, self.y,
                          stream)
                mk("combine")
        L.imbalance(s, self.counts, self.group_load, self.is_raw, self.is_norm, stream)
        mk("imbalance")
        if self.comparator:
            if self.side is not None:
                main.wait_stream(self.side)  # (the mark then times the part not hidden by the layer)
            else:
                comparator(main)
            mk("global_comparator")
        return None if self.routing_only else self.y

    def tune_tiles(self, x, w_router, bias, w_gate, w_up, w_down, shared=None, reps: int = 5) -> tuple:
        """Sets the gate/up and down GEMMs' tile shapes to the fastest measured on these inputs
        (bf16 layers with expert FFNs; others keep the library's choice) and returns them.  Each
        candidate runs ``reps`` whole forwards; a GEMM's time is the median between its stream
        events.  The result is cached per process under the layer's shape and device, so another
        layer of the same shape reuses it without timing.  Synchronises; not for graph capture."""
        if self.routing_only or self.dtype_code != L.BF16:
            return (self.shape_up.tiles, self.shape_down.tiles)
        dev = self.idx.device
        props = torch.cuda.get_device_properties(dev)
        key = (self.T, self.d, self.N, self.M, self.Kp, self.F, self.F_shared, self.dtype_code, self.e_lo,
               self.e_hi, self.gather, props.name, props.multi_processor_count)
        if key not in _TILE_CACHE:
            stream = torch.cuda.current_stream(dev)

            def gemm_us(name):
                ts = []
                for _ in range(reps):
                    marks = []

                    def rec(n):
                        ev = torch.cuda.Event(enable_timing=True)
                        ev.record(stream)
                        marks.append((n, ev))
                    self.forward(x, w_router, bias, w_gate, w_up, w_down, shared, mark=rec)
                    torch.cuda.synchronize(dev)
                    names = [n for n, _ in marks]
                    i = names.index(name)
                    ts.append(marks[i - 1][1].elapsed_time(marks[i][1]))
                return sorted(ts)[len(ts) // 2]

            best = []
            for shp, name, cands in ((self.shape_up, "gate_up", (L.TILES_TALL, L.TILES_WIDE, L.TILES_BALANCED)),
                                     (self.shape_down, "down", (L.TILES_TALL, L.TILES_WIDE))):
                keep = shp.tiles
                times = {}
                for c in cands:
                    shp.tiles = c
                    self.forward(x, w_router, bias, w_gate, w_up, w_down, shared)  # warm-up of this shape
                    times[c] = gemm_us(name)
                shp.tiles = keep
                best.append(min(times, key=times.get))
            _TILE_CACHE[key] = tuple(best)
        self.shape_up.tiles, self.shape_down.tiles = _TILE_CACHE[key]
        return _TILE_CACHE[key]

    def check_scores(self, stream=None) -> None:
        """Raises MogeError (MOGE_ERR_NONFINITE) if the router scores of the last forward hold a NaN
        or an infinity.  Waits for the stream.  Needs the layer built with store_scores=True."""
        if self.logits is None:
            raise ValueError("the layer keeps no scores: build it with store_scores=True")
        if not hasattr(self, "check_ws"):
            self.check_ws = torch.empty(L.workspace_size(self.shape, L.STAGE_CHECK), dtype=torch.uint8,
                                        device=self.logits.device)
        L.check_finite(self.logits, self.check_ws, stream)

    def capture(self, x, w_router, bias, w_gate=None, w_up=None, w_down=None, shared=None, warmup: int = 1):
        """Records one ``forward`` on these tensors into a HIP graph and returns it; ``g.replay()``
        then enqueues the whole layer (both streams) with one host call.  The library calls
        allocate nothing and set no memory, so the recorded work is exactly the forward's kernels.
        The inputs are bound by address: refill the same tensors between replays."""
        for _ in range(warmup):  # one-time setup (LDS limits, CU count) happens outside the capture
            self.forward(x, w_router, bias, w_gate, w_up, w_down, shared)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.forward(x, w_router, bias, w_gate, w_up, w_down, shared)
        return g
