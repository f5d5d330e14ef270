"""ctypes binding of libmoge (include/moge.h).

Argument marshalling only: every call checks that the tensors are contiguous CUDA
(HIP) tensors of the expected dtype and size, passes their device pointers and the
current stream to the C entry point of the same name, and raises MogeError when the
library returns an error.  No computation happens here.  If libmoge.so is missing
this module fails at import time; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOGE_LIB names another build of the same library (e.g. one with sanitized host code)
LIB_PATH = os.environ.get("MOGE_LIB") or os.path.join(_HERE, "libmoge.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python __graft_entry__.py` (build()) first")

_lib = ctypes.CDLL(LIB_PATH)

OK = 0
STATUS = {0: "MOGE_OK", 1: "MOGE_ERR_ARG", 2: "MOGE_ERR_SHAPE", 3: "MOGE_ERR_NULL", 4: "MOGE_ERR_WORKSPACE",
          5: "MOGE_ERR_DTYPE", 6: "MOGE_ERR_HIP", 7: "MOGE_ERR_CAPACITY", 8: "MOGE_ERR_NONFINITE"}
BF16 = 0
F32 = 1
ROUTE_GROUPED = 0
ROUTE_GLOBAL = 1
STAGE_DISPATCH = 1
STAGE_CHECK = 2
STAGE_ROUTE = 3
TILES_AUTO = 0
TILES_TALL = 1
TILES_WIDE = 2
TILES_BALANCED = 3

EXPORTS = ("moge_validate", "moge_rows_bound", "moge_tiled_elems", "moge_packed_weight_elems",
           "moge_workspace_size", "moge_pack_weights", "moge_route", "moge_route_pair", "moge_dispatch",
           "moge_dispatch_noalloc",
           "moge_grouped_ffn",
           "moge_expert_gate_up", "moge_expert_down", "moge_expert_gate_up_with_shared",
           "moge_expert_down_with_shared", "moge_expert_gate_up_gather", "moge_expert_down_combine",
           "moge_combine", "moge_imbalance", "moge_imbalance_batches", "moge_check_finite", "moge_tile_choice",
           "moge_version",
           "moge_last_error", "moge_round_bf16")


class Shape(ctypes.Structure):
    """moge_shape_t; ``tiles`` (default TILES_AUTO) picks the expert GEMMs' tile shape for the calls
    made with this shape."""
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("N", ctypes.c_int32), ("M", ctypes.c_int32),
                ("k_per_group", ctypes.c_int32), ("F", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("tiles", ctypes.c_int32)]

    @property
    def K(self) -> int:
        return self.M * self.k_per_group

    def __repr__(self):
        return (f"Shape(T={self.T}, d={self.d}, N={self.N}, M={self.M}, k_per_group={self.k_per_group}, "
                f"F={self.F}, dtype={'bf16' if self.dtype == BF16 else 'f32'}, tiles={self.tiles})")


class MogeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with {STATUS.get(status, status)}: {msg}")
        self.status = status


_P = ctypes.c_void_p
_SP = ctypes.POINTER(Shape)
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64

_lib.moge_validate.argtypes = [_SP]
_lib.moge_validate.restype = ctypes.c_int
_lib.moge_rows_bound.argtypes = [_SP, _I32, _I32, _I32]
_lib.moge_rows_bound.restype = _I64
_lib.moge_tiled_elems.argtypes = [_I64, _I64]
_lib.moge_tiled_elems.restype = _I64
_lib.moge_packed_weight_elems.argtypes = [_I64, _I64]
_lib.moge_packed_weight_elems.restype = _I64
_lib.moge_pack_weights.argtypes = [_I32, _I64, _I64, _I64, _P, _P, _P]
_lib.moge_pack_weights.restype = ctypes.c_int
_lib.moge_round_bf16.argtypes = [_P, _P, _I64, _P]
_lib.moge_round_bf16.restype = ctypes.c_int
_lib.moge_workspace_size.argtypes = [_SP, _I32]
_lib.moge_workspace_size.restype = ctypes.c_size_t
_lib.moge_route.argtypes = [_SP, _I32, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
_lib.moge_route.restype = ctypes.c_int
_lib.moge_route_pair.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
_lib.moge_route_pair.restype = ctypes.c_int
_lib.moge_dispatch.argtypes = [_SP, _I32, _P, _P, _I32, _I32, _I64, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                               _P]
_lib.moge_dispatch.restype = ctypes.c_int
_lib.moge_dispatch_noalloc.argtypes = [_SP, _I32, _P, _P, _I32, _I32, _I64, _P, _P, _P, _P, _P, _P, _P]
_lib.moge_dispatch_noalloc.restype = ctypes.c_int
_lib.moge_grouped_ffn.argtypes = [_SP, _P, _P, _I32, _I32, _I64, _P, _P, _P, _P, _P, _P]
_lib.moge_grouped_ffn.restype = ctypes.c_int
_lib.moge_expert_gate_up.argtypes = [_SP, _P, _P, _I32, _I32, _I64, _P, _P, _P, _P]
_lib.moge_expert_gate_up.restype = ctypes.c_int
_lib.moge_expert_down.argtypes = [_SP, _P, _P, _I32, _I32, _I64, _P, _P, _P]
_lib.moge_expert_down.restype = ctypes.c_int
_lib.moge_expert_gate_up_with_shared.argtypes = [_SP, _I32, _P, _P, _I32, _I32, _I64, _P, _P, _P, _P, _P, _P, _P, _P]
_lib.moge_expert_gate_up_with_shared.restype = ctypes.c_int
_lib.moge_expert_down_with_shared.argtypes = [_SP, _I32, _P, _P, _I32, _I32, _I64, _P, _P, _P, _P, _P, _P]
_lib.moge_expert_down_with_shared.restype = ctypes.c_int
_lib.moge_expert_gate_up_gather.argtypes = [_SP, _P, _P, _P, _I32, _I32, _I64, _P, _P, _P, _I32, _P, _P, _P, _P]
_lib.moge_expert_gate_up_gather.restype = ctypes.c_int
_lib.moge_expert_down_combine.argtypes = [_SP, _P, _P, _I32, _I32, _I64, _P, _P, _P, _P, _P]
_lib.moge_expert_down_combine.restype = ctypes.c_int
_lib.moge_check_finite.argtypes = [_I32, _P, _I64, _P, ctypes.c_size_t, _P]
_lib.moge_check_finite.restype = ctypes.c_int
_lib.moge_combine.argtypes = [_SP, _P, _P, _P, _I64, _P, _P, _P]
_lib.moge_combine.restype = ctypes.c_int
_lib.moge_imbalance.argtypes = [_SP, _P, _P, _P, _P, _P]
_lib.moge_imbalance.restype = ctypes.c_int
_lib.moge_imbalance_batches.argtypes = [_SP, _P, _I64, _P, _P, _P]
_lib.moge_imbalance_batches.restype = ctypes.c_int
_lib.moge_tile_choice.argtypes = [_SP, _I32, _I32, _I32, _I32]
_lib.moge_tile_choice.restype = ctypes.c_int32
_lib.moge_version.argtypes = []
_lib.moge_version.restype = ctypes.c_char_p
_lib.moge_last_error.argtypes = []
_lib.moge_last_error.restype = ctypes.c_char_p


def _check(fn: str, st: int) -> None:
    if st != OK:
        raise MogeError(fn, st, _lib.moge_last_error().decode())


def _elem_dtype(shape: Shape):
    return torch.bfloat16 if shape.dtype == BF16 else torch.float32


def _ptr(t, name: str, dtype=None, numel: int | None = None, optional: bool = False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} needs at least {numel} elements, has {t.numel()}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def validate(shape: Shape) -> int:
    return _lib.moge_validate(ctypes.byref(shape))


def rows_bound(shape: Shape, mode: int, e_lo: int, e_hi: int) -> int:
    return int(_lib.moge_rows_bound(ctypes.byref(shape), mode, e_lo, e_hi))


def tiled_elems(rows: int, cols: int) -> int:
    """Elements of a tiled activation matrix: rows rounded up to 16 times cols rounded up to 32."""
    return int(_lib.moge_tiled_elems(rows, cols))


def packed_weight_elems(rows: int, cols: int) -> int:
    """Elements of one packed expert weight matrix: rows and cols rounded up to 32."""
    return int(_lib.moge_packed_weight_elems(rows, cols))


def pack_weights(dtype: int, w, out, stream=None) -> None:
    """w [E][rows][cols] row-major -> out, E * packed_weight_elems(rows, cols) elements (tiled)."""
    if w is None or w.dim() != 3:
        raise ValueError("w must be a 3-d tensor [E][rows][cols]")
    E, rows, cols = w.shape
    et = torch.bfloat16 if dtype == BF16 else torch.float32
    st = _lib.moge_pack_weights(dtype, E, rows, cols, _ptr(w, "w", et, E * rows * cols),
                                _ptr(out, "out", et, E * packed_weight_elems(rows, cols)), _stream(stream))
    _check("moge_pack_weights", st)


def round_bf16(x, y, stream=None) -> None:
    """y = x (float32) rounded to bf16 as the library stores bf16 values; y holds the bit patterns
    (torch.int16 or torch.bfloat16 viewed as int16) with x.numel() elements."""
    n = x.numel()
    yv = y.view(torch.int16) if y.dtype == torch.bfloat16 else y
    st = _lib.moge_round_bf16(_ptr(x, "x", torch.float32, n), _ptr(yv, "y", torch.int16, n), n, _stream(stream))
    _check("moge_round_bf16", st)


def workspace_size(shape: Shape, stage: int = STAGE_DISPATCH) -> int:
    return int(_lib.moge_workspace_size(ctypes.byref(shape), stage))


def tile_choice(shape: Shape, gemm: int, e_lo: int, e_hi: int, F_shared: int = 0) -> int:
    """The tile shape (TILES_TALL, TILES_WIDE or TILES_BALANCED) the library uses for GEMM `gemm`
    (1 gate/up, 2 down)."""
    return int(_lib.moge_tile_choice(ctypes.byref(shape), gemm, e_lo, e_hi, F_shared))


def version() -> str:
    return _lib.moge_version().decode()


def last_error() -> str:
    return _lib.moge_last_error().decode()


def _ws(ws):
    return (_ptr(ws, "ws", None, None), ws.numel() * ws.element_size()) if ws is not None else (None, 0)


def route(shape: Shape, mode: int, x, w_router, bias, logits, idx, gate, ws=None, stream=None) -> None:
    """ws: workspace_size(shape, STAGE_ROUTE) bytes (None when that is 0)."""
    T, N, K, d = shape.T, shape.N, shape.K, shape.d
    et = _elem_dtype(shape)
    wsp, wsb = _ws(ws)
    st = _lib.moge_route(ctypes.byref(shape), mode, _ptr(x, "x", et, T * d, optional=True),
                         _ptr(w_router, "w_router", et, N * d, optional=x is None),
                         _ptr(bias, "bias", torch.float32, N, optional=True),
                         _ptr(logits, "logits", torch.float32, T * N, optional=x is not None),
                         _ptr(idx, "idx", torch.int32, T * K), _ptr(gate, "gate", torch.float32, T * K), wsp, wsb,
                         _stream(stream))
    _check("moge_route", st)


def route_pair(shape: Shape, x, w_router, bias, logits, idx, gate, gidx, ggate, ws=None, stream=None) -> None:
    """Both routers on the same scores: MoGE into idx/gate, the global top-K into gidx/ggate."""
    T, N, K, d = shape.T, shape.N, shape.K, shape.d
    et = _elem_dtype(shape)
    wsp, wsb = _ws(ws)
    st = _lib.moge_route_pair(ctypes.byref(shape), _ptr(x, "x", et, T * d, optional=True),
                              _ptr(w_router, "w_router", et, N * d, optional=x is None),
                              _ptr(bias, "bias", torch.float32, N, optional=True),
                              _ptr(logits, "logits", torch.float32, T * N, optional=x is not None),
                              _ptr(idx, "idx", torch.int32, T * K), _ptr(gate, "gate", torch.float32, T * K),
                              _ptr(gidx, "gidx", torch.int32, T * K), _ptr(ggate, "ggate", torch.float32, T * K),
                              wsp, wsb, _stream(stream))
    _check("moge_route_pair", st)


def dispatch(shape: Shape, mode: int, idx, x, e_lo: int, e_hi: int, rows_cap: int, counts, offsets, inv, perm,
             x_perm, ws, x_tiled=None, stream=None) -> None:
    T, N, K, d = shape.T, shape.N, shape.K, shape.d
    et = _elem_dtype(shape)
    st = _lib.moge_dispatch(ctypes.byref(shape), mode, _ptr(idx, "idx", torch.int32, T * K),
                            _ptr(x, "x", et, T * d, optional=True), e_lo, e_hi, rows_cap,
                            _ptr(counts, "counts", torch.int32, N), _ptr(offsets, "offsets", torch.int32, N + 1),
                            _ptr(inv, "inv", torch.int32, T * K, optional=True),
                            _ptr(perm, "perm", torch.int32, rows_cap, optional=True),
                            _ptr(x_perm, "x_perm", et, tiled_elems(rows_cap, d), optional=True),
                            _ptr(x_tiled, "x_tiled", et, tiled_elems(T, d), optional=True), _ptr(ws, "ws", None, None),
                            ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    _check("moge_dispatch", st)


def dispatch_noalloc(shape: Shape, mode: int, idx, x, e_lo: int, e_hi: int, rows_cap: int, counts, offsets, inv,
                     perm, x_perm, x_tiled=None, stream=None) -> None:
    """moge_dispatch without a workspace argument (the library's fixed device array instead)."""
    T, N, K, d = shape.T, shape.N, shape.K, shape.d
    et = _elem_dtype(shape)
    st = _lib.moge_dispatch_noalloc(ctypes.byref(shape), mode, _ptr(idx, "idx", torch.int32, T * K),
                                    _ptr(x, "x", et, T * d, optional=True), e_lo, e_hi, rows_cap,
                                    _ptr(counts, "counts", torch.int32, N), _ptr(offsets, "offsets", torch.int32, N + 1),
                                    _ptr(inv, "inv", torch.int32, T * K, optional=True),
                                    _ptr(perm, "perm", torch.int32, rows_cap, optional=True),
                                    _ptr(x_perm, "x_perm", et, tiled_elems(rows_cap, d), optional=True),
                                    _ptr(x_tiled, "x_tiled", et, tiled_elems(T, d), optional=True), _stream(stream))
    _check("moge_dispatch_noalloc", st)


def grouped_ffn(shape: Shape, x_perm, offsets, e_lo: int, e_hi: int, rows_cap: int, w_gate, w_up, w_down, h, out,
                stream=None) -> None:
    d, F = shape.d, shape.F
    E = e_hi - e_lo
    et = _elem_dtype(shape)
    st = _lib.moge_grouped_ffn(ctypes.byref(shape), _ptr(x_perm, "x_perm", et, tiled_elems(rows_cap, d)),
                               _ptr(offsets, "offsets", torch.int32, shape.N + 1), e_lo, e_hi, rows_cap,
                               _ptr(w_gate, "w_gate", et, E * packed_weight_elems(F, d)),
                               _ptr(w_up, "w_up", et, E * packed_weight_elems(F, d)),
                               _ptr(w_down, "w_down", et, E * packed_weight_elems(d, F)),
                               _ptr(h, "h", et, tiled_elems(rows_cap, F)), _ptr(out, "out", et, rows_cap * d),
                               _stream(stream))
    _check("moge_grouped_ffn", st)


def expert_gate_up(shape: Shape, x_perm, offsets, e_lo: int, e_hi: int, rows_cap: int, w_gate, w_up, h,
                   stream=None) -> None:
    d, F = shape.d, shape.F
    E = e_hi - e_lo
    et = _elem_dtype(shape)
    st = _lib.moge_expert_gate_up(ctypes.byref(shape), _ptr(x_perm, "x_perm", et, tiled_elems(rows_cap, d)),
                                  _ptr(offsets, "offsets", torch.int32, shape.N + 1), e_lo, e_hi, rows_cap,
                                  _ptr(w_gate, "w_gate", et, E * packed_weight_elems(F, d)),
                                  _ptr(w_up, "w_up", et, E * packed_weight_elems(F, d)),
                                  _ptr(h, "h", et, tiled_elems(rows_cap, F)), _stream(stream))
    _check("moge_expert_gate_up", st)


def expert_down(shape: Shape, h, offsets, e_lo: int, e_hi: int, rows_cap: int, w_down, out, stream=None) -> None:
    d, F = shape.d, shape.F
    E = e_hi - e_lo
    et = _elem_dtype(shape)
    st = _lib.moge_expert_down(ctypes.byref(shape), _ptr(h, "h", et, tiled_elems(rows_cap, F)),
                               _ptr(offsets, "offsets", torch.int32, shape.N + 1), e_lo, e_hi, rows_cap,
                               _ptr(w_down, "w_down", et, E * packed_weight_elems(d, F)),
                               _ptr(out, "out", et, rows_cap * d), _stream(stream))
    _check("moge_expert_down", st)


def expert_gate_up_with_shared(shape: Shape, F_shared: int, x_perm, offsets, e_lo: int, e_hi: int, rows_cap: int,
                               w_gate, w_up, h, x_tiled, ws_gate, ws_up, hs, stream=None) -> None:
    T, d, F = shape.T, shape.d, shape.F
    E = e_hi - e_lo
    et = _elem_dtype(shape)
    st = _lib.moge_expert_gate_up_with_shared(
        ctypes.byref(shape), F_shared, _ptr(x_perm, "x_perm", et, tiled_elems(rows_cap, d)),
        _ptr(offsets, "offsets", torch.int32, shape.N + 1), e_lo, e_hi, rows_cap,
        _ptr(w_gate, "w_gate", et, E * packed_weight_elems(F, d)), _ptr(w_up, "w_up", et, E * packed_weight_elems(F, d)),
        _ptr(h, "h", et, tiled_elems(rows_cap, F)), _ptr(x_tiled, "x_tiled", et, tiled_elems(T, d)),
        _ptr(ws_gate, "ws_gate", et, packed_weight_elems(F_shared, d)),
        _ptr(ws_up, "ws_up", et, packed_weight_elems(F_shared, d)), _ptr(hs, "hs", et, tiled_elems(T, F_shared)),
        _stream(stream))
    _check("moge_expert_gate_up_with_shared", st)


def expert_gate_up_gather(shape: Shape, x, perm, offsets, e_lo: int, e_hi: int, rows_cap: int, w_gate, w_up, h,
                          F_shared: int = 0, ws_gate=None, ws_up=None, hs=None, stream=None) -> None:
    T, d, F = shape.T, shape.d, shape.F
    E = e_hi - e_lo
    et = _elem_dtype(shape)
    st = _lib.moge_expert_gate_up_gather(
        ctypes.byref(shape), _ptr(x, "x", et, T * d), _ptr(perm, "perm", torch.int32, rows_cap),
        _ptr(offsets, "offsets", torch.int32, shape.N + 1), e_lo, e_hi, rows_cap,
        _ptr(w_gate, "w_gate", et, E * packed_weight_elems(F, d)), _ptr(w_up, "w_up", et, E * packed_weight_elems(F, d)),
        _ptr(h, "h", et, tiled_elems(rows_cap, F)), F_shared,
        _ptr(ws_gate, "ws_gate", et, packed_weight_elems(F_shared, d) if F_shared else 0, optional=True),
        _ptr(ws_up, "ws_up", et, packed_weight_elems(F_shared, d) if F_shared else 0, optional=True),
        _ptr(hs, "hs", et, tiled_elems(T, F_shared) if F_shared else 0, optional=True), _stream(stream))
    _check("moge_expert_gate_up_gather", st)


def check_finite(a, ws, stream=None) -> None:
    """Raises MogeError (MOGE_ERR_NONFINITE) if the float32 or bf16 tensor `a` holds a NaN or an
    infinity.  Synchronises `stream`.  ws: workspace_size(shape, STAGE_CHECK) bytes."""
    if a.dtype == torch.float32:
        dt = F32
    elif a.dtype == torch.bfloat16:
        dt = BF16
    else:
        raise TypeError(f"a must be float32 or bfloat16, got {a.dtype}")
    n = a.numel()
    st = _lib.moge_check_finite(dt, _ptr(a, "a", None, n), n, _ptr(ws, "ws", None, None),
                                ws.numel() * ws.element_size(), _stream(stream))
    _check("moge_check_finite", st)


def expert_down_combine(shape: Shape, h, offsets, e_lo: int, e_hi: int, rows_cap: int, w_down, perm, gate, y,
                        stream=None) -> None:
    T, d, F, K = shape.T, shape.d, shape.F, shape.K
    E = e_hi - e_lo
    et = _elem_dtype(shape)
    st = _lib.moge_expert_down_combine(
        ctypes.byref(shape), _ptr(h, "h", et, tiled_elems(rows_cap, F)),
        _ptr(offsets, "offsets", torch.int32, shape.N + 1), e_lo, e_hi, rows_cap,
        _ptr(w_down, "w_down", et, E * packed_weight_elems(d, F)), _ptr(perm, "perm", torch.int32, rows_cap),
        _ptr(gate, "gate", torch.float32, T * K), _ptr(y, "y", torch.float32, T * d), _stream(stream))
    _check("moge_expert_down_combine", st)


def expert_down_with_shared(shape: Shape, F_shared: int, h, offsets, e_lo: int, e_hi: int, rows_cap: int, w_down, out,
                            hs, ws_down, out_shared, stream=None) -> None:
    T, d, F = shape.T, shape.d, shape.F
    E = e_hi - e_lo
    et = _elem_dtype(shape)
    st = _lib.moge_expert_down_with_shared(
        ctypes.byref(shape), F_shared, _ptr(h, "h", et, tiled_elems(rows_cap, F)),
        _ptr(offsets, "offsets", torch.int32, shape.N + 1), e_lo, e_hi, rows_cap,
        _ptr(w_down, "w_down", et, E * packed_weight_elems(d, F)), _ptr(out, "out", et, rows_cap * d),
        _ptr(hs, "hs", et, tiled_elems(T, F_shared)), _ptr(ws_down, "ws_down", et, packed_weight_elems(d, F_shared)),
        _ptr(out_shared, "out_shared", et, T * d), _stream(stream))
    _check("moge_expert_down_with_shared", st)


def combine(shape: Shape, o, inv, gate, rows_cap: int, shared_out, y, stream=None) -> None:
    T, K, d = shape.T, shape.K, shape.d
    et = _elem_dtype(shape)
    st = _lib.moge_combine(ctypes.byref(shape), _ptr(o, "o", et, rows_cap * d), _ptr(inv, "inv", torch.int32, T * K),
                           _ptr(gate, "gate", torch.float32, T * K), rows_cap,
                           _ptr(shared_out, "shared_out", et, T * d, optional=True),
                           _ptr(y, "y", torch.float32, T * d), _stream(stream))
    _check("moge_combine", st)


def imbalance(shape: Shape, counts, group_load, is_raw, is_norm, stream=None) -> None:
    st = _lib.moge_imbalance(ctypes.byref(shape), _ptr(counts, "counts", torch.int32, shape.N),
                             _ptr(group_load, "group_load", torch.int32, shape.M),
                             _ptr(is_raw, "is_raw", torch.int32, 1), _ptr(is_norm, "is_norm", torch.float64, 1),
                             _stream(stream))
    _check("moge_imbalance", st)


def imbalance_batches(shape: Shape, idx, tokens_per_batch: int, group_load, is_raw, stream=None) -> None:
    B = shape.T // tokens_per_batch if tokens_per_batch > 0 else 0
    st = _lib.moge_imbalance_batches(ctypes.byref(shape), _ptr(idx, "idx", torch.int32, shape.T * shape.K),
                                     tokens_per_batch, _ptr(group_load, "group_load", torch.int32, B * shape.M),
                                     _ptr(is_raw, "is_raw", torch.int32, B), _stream(stream))
    _check("moge_imbalance_batches", st)
