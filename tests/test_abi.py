"""CPU-only checks of the C ABI: the library loads without a GPU, exports every function that
include/moge.h declares, and its host-side validation returns the documented status codes.
No compute call is made here."""
import ctypes
import os
import re

import pytest

import mixture_grouped_experts_amd as moge

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "moge.h")) as f:
        txt = f.read()
    return sorted(set(re.findall(r"^\s*(?:moge_status_t|int64_t|int32_t|size_t|const char\*)\s+(moge_\w+)\s*\(", txt, re.M)))


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(moge.LIB_PATH)
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(moge.EXPORTS)


def test_version():
    assert "gfx950" in moge.version()


def S(T=64, d=128, N=8, M=4, Kp=1, F=64, dt=moge.BF16, tiles=moge.TILES_AUTO):
    return moge.Shape(T, d, N, M, Kp, F, dt, tiles)


@pytest.mark.parametrize("shape,code", [
    (S(), 0), (S(dt=moge.F32), 0), (S(F=0), 0), (S(M=1, Kp=8), 0), (S(N=256, M=8, Kp=32), 0),
    (S(T=0), 2), (S(d=100), 2), (S(d=0), 2), (S(M=3), 2), (S(M=16), 2), (S(Kp=0), 2), (S(Kp=3), 2),
    (S(F=12), 2), (S(F=-8), 2), (S(N=512, M=8), 2), (S(dt=7), 5), (S(T=2 ** 28, M=8, N=64, Kp=1), 2),
    (S(tiles=moge.TILES_TALL), 0), (S(tiles=moge.TILES_WIDE), 0), (S(tiles=moge.TILES_BALANCED), 0),
    (S(tiles=4), 1), (S(tiles=-1), 1),
    (S(N=256, M=8, Kp=32), 0), (S(N=256, M=1, Kp=256), 0),                  # K = N: every expert chosen
])
def test_validate(shape, code):
    assert moge.validate(shape) == code
    if code:
        assert moge.last_error()


def test_rows_bound_and_workspace():
    s = S(T=100, N=64, M=8, Kp=2)
    # assignment bound + 15 padding rows per expert of the range (segments start on 16-row boundaries)
    assert moge.rows_bound(s, moge.ROUTE_GROUPED, 0, 64) == 100 * 16 + 15 * 64
    assert moge.rows_bound(s, moge.ROUTE_GROUPED, 0, 8) == 100 * 2 + 15 * 8       # one group
    assert moge.rows_bound(s, moge.ROUTE_GROUPED, 7, 9) == 100 * 2 + 15 * 2       # one expert in each of two groups
    assert moge.rows_bound(s, moge.ROUTE_GROUPED, 0, 1) == 100 + 15
    assert moge.rows_bound(s, moge.ROUTE_GLOBAL, 0, 8) == 100 * 8 + 15 * 8
    assert moge.rows_bound(s, moge.ROUTE_GLOBAL, 0, 64) == 100 * 16 + 15 * 64
    assert moge.rows_bound(s, 5, 0, 8) == -1 and moge.rows_bound(s, 0, 8, 8) == -1
    assert moge.workspace_size(S(T=65536, N=64)) == 2 * 64 * 1024 * 4   # blocks of 64 tokens
    assert moge.workspace_size(S(T=1, N=8)) == 2 * 8 * 1 * 4
    assert moge.workspace_size(S(T=0)) == 2 ** 64 - 1
    assert moge.workspace_size(S(), moge.STAGE_CHECK) == 1024 * 16 + 16
    assert moge.workspace_size(S(), 9) == 2 ** 64 - 1


def test_tiled_sizes():
    # tiles of 16 rows x 32 columns; packed weights pad rows to 32
    assert moge.tiled_elems(1, 8) == 16 * 32
    assert moge.tiled_elems(16, 32) == 512 and moge.tiled_elems(17, 33) == 32 * 64
    assert moge.tiled_elems(65536 + 15 * 256, 7680) == (65536 + 15 * 256) * 7680
    assert moge.packed_weight_elems(200, 256) == 224 * 256 and moge.packed_weight_elems(2048, 7680) == 2048 * 7680
    assert moge.tiled_elems(-1, 8) == -1 and moge.packed_weight_elems(4, -1) == -1


def test_pack_weights_argument_errors():
    lib = ctypes.CDLL(moge.LIB_PATH)
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced: every case fails host validation first
    lib.moge_pack_weights.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P, P, P]
    assert lib.moge_pack_weights(9, 1, 8, 8, fake, fake, None) == 5
    assert lib.moge_pack_weights(0, 0, 8, 8, fake, fake, None) == 2
    assert lib.moge_pack_weights(0, 1, 8, 12, fake, fake, None) == 2
    assert lib.moge_pack_weights(0, 1, 0, 8, fake, fake, None) == 2
    assert lib.moge_pack_weights(0, 1, 8, 8, None, fake, None) == 3


def _call(fn, *args):
    return getattr(ctypes.CDLL(moge.LIB_PATH), fn)(*args)


def test_round_bf16_argument_errors():
    lib = ctypes.CDLL(moge.LIB_PATH)
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced: every case returns before a launch
    lib.moge_round_bf16.argtypes = [P, P, ctypes.c_int64, P]
    assert lib.moge_round_bf16(fake, fake, -1, None) == 2      # MOGE_ERR_SHAPE
    assert lib.moge_round_bf16(None, fake, 4, None) == 3       # MOGE_ERR_NULL
    assert lib.moge_round_bf16(fake, None, 4, None) == 3
    assert lib.moge_round_bf16(None, None, 0, None) == 0       # nothing to round


def test_null_and_argument_errors_before_any_launch():
    lib = ctypes.CDLL(moge.LIB_PATH)
    s = S()
    sp = ctypes.byref(s)
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced: every case fails host validation first
    lib.moge_route.argtypes = [ctypes.c_void_p, ctypes.c_int32] + [P] * 7 + [ctypes.c_size_t, P]
    assert lib.moge_route(None, 0, fake, fake, None, fake, fake, fake, None, 0, None) == 3    # NULL shape
    assert lib.moge_route(sp, 2, fake, fake, None, fake, fake, fake, None, 0, None) == 1      # bad mode
    assert lib.moge_route(sp, 0, fake, fake, None, fake, None, fake, None, 0, None) == 3      # idx NULL
    assert lib.moge_route(sp, 0, None, None, None, None, fake, fake, None, 0, None) == 3      # no x, no logits
    assert lib.moge_route(sp, 0, None, None, fake, fake, fake, fake, None, 0, None) == 1      # bias with logits-in
    assert lib.moge_route(sp, 0, fake, None, None, None, fake, fake, None, 0, None) == 3      # x without w_router
    # more than 128 experts from x: the split reduction's workspace is required
    s256 = S(T=1000, N=256, M=8)
    need = moge.workspace_size(s256, moge.STAGE_ROUTE)
    assert need == 2 * 1000 * 256 * 4          # 8 token tiles, d = 128: 4 steps of 32, 2 slices of 2 steps
    assert moge.workspace_size(S(T=1000, d=7680, N=256, M=8), moge.STAGE_ROUTE) == 32 * 1000 * 256 * 4
    assert moge.workspace_size(S(T=8192, d=7680, N=256, M=8), moge.STAGE_ROUTE) == 4 * 8192 * 256 * 4
    # up to 128 experts: the one-pass kernel, in slices of d while its token tiles do not fill the CUs
    assert moge.workspace_size(S(T=65536, d=4096, N=64, M=8), moge.STAGE_ROUTE) == 0    # 512 tiles: one pass
    assert moge.workspace_size(S(T=5000, N=64, M=8), moge.STAGE_ROUTE) == 2 * 5000 * 64 * 4   # d = 128: 2 slices
    assert moge.workspace_size(S(T=8192, d=5120, N=64, M=8), moge.STAGE_ROUTE) == 8 * 8192 * 64 * 4
    assert moge.workspace_size(S(T=5000, d=64, N=64, M=8), moge.STAGE_ROUTE) == 0      # 2 steps: no split
    assert moge.workspace_size(S(T=16384, d=4096, N=128, M=8), moge.STAGE_ROUTE) == 0  # 256 tiles of 64
    assert moge.workspace_size(S(dt=moge.F32), moge.STAGE_ROUTE) == 0
    assert lib.moge_route(ctypes.byref(s256), 0, fake, fake, None, None, fake, fake, fake, need - 1, None) == 4
    assert lib.moge_route(ctypes.byref(s256), 0, fake, fake, None, None, fake, fake, None, 0, None) == 4
    lib.moge_route_pair.argtypes = [P] * 10 + [ctypes.c_size_t, P]
    assert lib.moge_route_pair(sp, fake, fake, None, None, fake, fake, None, fake, None, 0, None) == 3  # gidx NULL
    assert lib.moge_route_pair(sp, None, None, None, None, fake, fake, fake, fake, None, 0, None) == 3  # no input
    lib.moge_dispatch.argtypes = [P, ctypes.c_int32, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                  P, P, P, P, P, P, P, ctypes.c_size_t, P]
    ws = moge.workspace_size(s)
    cap = moge.rows_bound(s, moge.ROUTE_GROUPED, 0, 8)   # 64 tokens x 4 groups x 1 + 15 x 8 padding
    assert cap == 256 + 120
    assert lib.moge_dispatch(sp, 0, fake, fake, 0, 8, cap - 1, fake, fake, fake, fake, fake, None, fake, ws,
                             None) == 7
    assert lib.moge_dispatch(sp, 0, fake, fake, 0, 8, cap, fake, fake, fake, fake, fake, None, fake, ws - 1,
                             None) == 4
    assert lib.moge_dispatch(sp, 0, fake, fake, 0, 8, cap, fake, fake, fake, fake, fake, None, None, ws, None) == 4
    assert lib.moge_dispatch(sp, 0, fake, fake, 3, 3, cap, fake, fake, fake, fake, fake, None, fake, ws, None) == 1
    assert lib.moge_dispatch(sp, 0, fake, fake, 0, 9, cap, fake, fake, fake, fake, fake, None, fake, ws, None) == 1
    assert lib.moge_dispatch(sp, 3, fake, fake, 0, 8, cap, fake, fake, fake, fake, fake, None, fake, ws, None) == 1
    assert lib.moge_dispatch(sp, 0, fake, None, 0, 8, cap, fake, fake, fake, fake, fake, None, fake, ws, None) == 3
    assert lib.moge_dispatch(sp, 0, fake, fake, 0, 8, cap, fake, fake, None, fake, fake, None, fake, ws, None) == 3
    assert lib.moge_dispatch(sp, 0, fake, fake, 0, 8, cap, fake, fake, None, None, fake, None, fake, ws, None) == 3
    # x_tiled without x
    assert lib.moge_dispatch(sp, 0, fake, None, 0, 8, cap, fake, fake, fake, fake, None, fake, fake, ws, None) == 3
    # every shape moge_validate accepts (K = M K' <= N <= 256) passes dispatch's own checks: here
    # K = 256 with an undersized rows_cap is refused for the capacity, not for K
    big = S(N=256, M=8, Kp=32)
    assert moge.validate(big) == 0
    assert lib.moge_dispatch(ctypes.byref(big), 0, fake, fake, 0, 256, 64 * 256 + 15 * 256 - 1, fake, fake, fake,
                             fake, fake, None, fake, 1 << 20, None) == 7
    lib.moge_grouped_ffn.argtypes = [P, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64] + [P] * 6
    # a bad tile shape is refused by every call that takes the shape
    bad_tiles = ctypes.byref(S(tiles=9))
    assert lib.moge_grouped_ffn(bad_tiles, fake, fake, 0, 8, 64, fake, fake, fake, fake, fake, None) == 1
    assert lib.moge_grouped_ffn(ctypes.byref(S(F=0)), fake, fake, 0, 8, 64, fake, fake, fake, fake, fake, None) == 2
    assert lib.moge_grouped_ffn(sp, fake, fake, 0, 8, 64, fake, None, fake, fake, fake, None) == 3
    assert lib.moge_grouped_ffn(sp, fake, fake, -1, 8, 64, fake, fake, fake, fake, fake, None) == 1
    assert lib.moge_grouped_ffn(sp, fake, fake, 0, 8, 0, fake, fake, fake, fake, fake, None) == 7
    lib.moge_expert_gate_up_gather.argtypes = [P, P, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, P, P, P,
                                               ctypes.c_int32, P, P, P, P]
    g = lib.moge_expert_gate_up_gather
    d256 = S(d=256)
    sg = ctypes.byref(d256)
    assert g(ctypes.byref(S(d=256, dt=moge.F32)), fake, fake, fake, 0, 8, 64, fake, fake, fake, 0, None, None, None,
             None) == 5                                                                   # bf16 only
    assert g(ctypes.byref(S(d=200)), fake, fake, fake, 0, 8, 64, fake, fake, fake, 0, None, None, None, None) == 2
    assert g(sg, None, fake, fake, 0, 8, 64, fake, fake, fake, 0, None, None, None, None) == 3     # no x
    assert g(sg, fake, None, fake, 0, 8, 64, fake, fake, fake, 0, None, None, None, None) == 3     # no perm
    assert g(sg, fake, fake, fake, 0, 8, 64, fake, fake, fake, 12, fake, fake, fake, None) == 2    # F_shared % 8
    assert g(sg, fake, fake, fake, 0, 8, 64, fake, fake, fake, 64, fake, None, fake, None) == 3    # missing ws_up
    assert g(sg, fake, fake, fake, 0, 8, 64, fake, fake, fake, 0, None, None, fake, None) == 1     # hs without F_s
    assert g(sg, fake, fake, fake, 0, 9, 64, fake, fake, fake, 0, None, None, None, None) == 1     # e_hi > N
    assert g(sg, fake, fake, fake, 0, 8, 0, fake, fake, fake, 0, None, None, None, None) == 7      # rows_cap
    lib.moge_expert_down_combine.argtypes = [P, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, P, P, P, P, P]
    dc = lib.moge_expert_down_combine
    grp = ctypes.byref(S(N=8, M=4, Kp=1))                                                # groups of 2 experts
    assert dc(ctypes.byref(S(N=8, M=4, Kp=1, dt=moge.F32)), fake, fake, 2, 4, 64, fake, fake, fake, fake,
              None) == 5                                                                  # bf16 only
    assert dc(ctypes.byref(S(N=8, M=4, Kp=2)), fake, fake, 2, 4, 64, fake, fake, fake, fake, None) == 1  # K' = 2
    assert dc(grp, fake, fake, 2, 3, 64, fake, fake, fake, fake, None) == 1              # half a group
    assert dc(grp, fake, fake, 1, 3, 64, fake, fake, fake, fake, None) == 1              # straddles two groups
    assert dc(grp, fake, fake, 0, 8, 64, fake, fake, fake, fake, None) == 1              # all groups
    assert dc(grp, fake, fake, 2, 4, 64, fake, fake, None, fake, None) == 3              # no gate
    assert dc(grp, fake, fake, 2, 4, 64, fake, None, fake, fake, None) == 3              # no perm
    assert dc(grp, fake, fake, 2, 4, 0, fake, fake, fake, fake, None) == 7               # rows_cap
    lib.moge_combine.argtypes = [P, P, P, P, ctypes.c_int64, P, P, P]
    assert lib.moge_combine(sp, fake, fake, None, 64, None, fake, None) == 3
    assert lib.moge_combine(sp, fake, fake, fake, 0, None, fake, None) == 7
    lib.moge_imbalance_batches.argtypes = [P, P, ctypes.c_int64, P, P, P]
    assert lib.moge_imbalance_batches(sp, fake, 0, fake, fake, None) == 1       # tokens per batch < 1
    assert lib.moge_imbalance_batches(sp, fake, 48, fake, fake, None) == 1      # does not divide T = 64
    assert lib.moge_imbalance_batches(sp, None, 16, fake, fake, None) == 3
    lib.moge_imbalance.argtypes = [P] * 6
    assert lib.moge_imbalance(sp, fake, fake, None, fake, None) == 3
    assert lib.moge_imbalance(ctypes.byref(S(M=3)), fake, fake, fake, fake, None) == 2


def test_check_finite_argument_errors():
    lib = ctypes.CDLL(moge.LIB_PATH)
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced: every case returns before a launch
    lib.moge_check_finite.argtypes = [ctypes.c_int32, P, ctypes.c_int64, P, ctypes.c_size_t, P]
    ws = moge.workspace_size(S(), moge.STAGE_CHECK)
    assert lib.moge_check_finite(7, fake, 4, fake, ws, None) == 5           # MOGE_ERR_DTYPE
    assert lib.moge_check_finite(moge.F32, fake, -1, fake, ws, None) == 2   # MOGE_ERR_SHAPE
    assert lib.moge_check_finite(moge.F32, None, 4, fake, ws, None) == 3    # MOGE_ERR_NULL
    assert lib.moge_check_finite(moge.BF16, fake, 4, fake, ws - 1, None) == 4  # MOGE_ERR_WORKSPACE
    assert lib.moge_check_finite(moge.BF16, fake, 4, None, ws, None) == 4
    assert lib.moge_check_finite(moge.F32, None, 0, None, 0, None) == 0     # nothing to check
    from mixture_grouped_experts_amd import _lib
    assert _lib.STATUS[8] == "MOGE_ERR_NONFINITE"


def test_dispatch_noalloc_refuses_shapes_past_its_scratch():
    # checked on the host before the device is touched: 256 experts x 2049 token blocks x 8 bytes > 4 MiB
    lib = ctypes.CDLL(moge.LIB_PATH)
    P = ctypes.c_void_p
    fake = P(0x1000)
    lib.moge_dispatch_noalloc.argtypes = [P, ctypes.c_int32, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                          P, P, P, P, P, P, P]
    big = S(T=131073, N=256, M=8, Kp=1)
    assert moge.workspace_size(big) > 4 << 20
    assert lib.moge_dispatch_noalloc(ctypes.byref(big), 0, fake, None, 0, 256, 0, fake, fake, None, None, None, None,
                                     None) == 4
    assert "4194304" in moge.last_error()
    ok_shape = S(T=131072, N=256, M=8, Kp=1)
    assert moge.workspace_size(ok_shape) == 4 << 20                  # exactly the limit
    assert lib.moge_dispatch_noalloc(ctypes.byref(S()), 0, None, None, 0, 8, 0, fake, fake, None, None, None, None,
                                     None) == 3                       # idx NULL


@pytest.mark.parametrize("T,e_hi,gemm,want", [
    # 4096 hidden, 64 experts in 8 groups, K' = 2, F = 1408: rows per expert 2T/8; the expected
    # shape of each case was also the faster one when timed (64-512 tokens, 16-64 experts)
    # 704 tall tiles = 3 rounds x 256 rows < 384 wide tiles = 2 x 512; with each expert's 1408
    # columns in 12 tiles of 128 and 96 the busiest CU streams 2 x 256 + 192 = 704 rows
    (256, 64, 1, "balanced"),
    (256, 64, 2, "wide"),    # 1024 tall tiles = 4 x 256 == 512 wide tiles = 2 x 512: tie -> wide
    (64, 64, 1, "balanced"), (64, 64, 2, "wide"),
    (512, 64, 1, "tall"), (512, 64, 2, "tall"),    # 128 rows: a wide tile splits each expert in two,
                                                   # and a column split no longer pays
    (64, 43, 1, "tall"),     # 473 tall tiles = 2 x 256 < 258 wide tiles = 2 x 512; no split does better
    (64, 32, 1, "wide"),     # 352 tall = 2 x 256 == 192 wide = 1 x 512
    (64, 16, 1, "tall"),     # 176 tall = 1 x 256 < 96 wide = 1 x 512
])
def test_tile_table(T, e_hi, gemm, want):
    s = S(T=T, d=4096, N=64, M=8, Kp=2, F=1408)
    got = moge.tile_choice(s, gemm, 0, e_hi)
    assert got == {"tall": moge.TILES_TALL, "wide": moge.TILES_WIDE, "balanced": moge.TILES_BALANCED}[want]


def test_tile_table_large_shapes_and_forced():
    ultra = S(T=8192, d=7680, N=256, M=8, Kp=1, F=2048)
    assert moge.tile_choice(ultra, 1, 0, 256, 2048) == moge.TILES_TALL
    assert moge.tile_choice(ultra, 2, 0, 256, 2048) == moge.TILES_TALL
    group0 = S(T=65536, d=4096, N=64, M=8, Kp=1, F=1408)
    assert moge.tile_choice(group0, 1, 0, 8) == moge.TILES_TALL
    forced = S(T=8192, d=7680, N=256, M=8, Kp=1, F=2048, tiles=moge.TILES_WIDE)
    assert moge.tile_choice(forced, 1, 0, 256) == moge.TILES_WIDE
    balanced = S(T=8192, d=7680, N=256, M=8, Kp=1, F=2048, tiles=moge.TILES_BALANCED)
    assert moge.tile_choice(balanced, 1, 0, 256) == moge.TILES_BALANCED    # 64 units: 17+ tiles of 4 and 3
    assert moge.tile_choice(balanced, 2, 0, 256) == moge.TILES_TALL        # the down GEMM runs tall
    narrow = S(T=8192, d=7680, N=256, M=8, Kp=1, F=64, tiles=moge.TILES_BALANCED)
    assert moge.tile_choice(narrow, 1, 0, 256) == moge.TILES_TALL          # 2 units: no split of 3 or 4
    assert moge.tile_choice(ultra, 3, 0, 256) == -1 and moge.tile_choice(ultra, 1, 5, 5) == -1
    assert moge.tile_choice(S(F=0), 1, 0, 8) == -1

