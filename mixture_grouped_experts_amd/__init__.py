"""libmoge: the forward pass of one MoGE (Mixture of Grouped Experts) layer on MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of ``include/moge.h``
(``libmoge.so``).  This package is the thin Python binding (``_lib``: ctypes marshalling)
plus ``layer.MoGELayer``, which owns device buffers and issues the ABI calls of one layer
forward in order.  PyTorch is used only for device memory and streams.
"""
from ._lib import (BF16, EXPORTS, F32, LIB_PATH, ROUTE_GLOBAL, ROUTE_GROUPED, STAGE_CHECK,  # noqa: F401
                   STAGE_DISPATCH, STAGE_ROUTE, TILES_AUTO, TILES_BALANCED, TILES_TALL, TILES_WIDE, MogeError, Shape, check_finite, combine,
                   dispatch, dispatch_noalloc, expert_down,
                   expert_down_combine, expert_down_with_shared, expert_gate_up, expert_gate_up_gather,
                   expert_gate_up_with_shared, grouped_ffn, imbalance, imbalance_batches, last_error, pack_weights,
                   packed_weight_elems, round_bf16, route, route_pair, rows_bound, tile_choice, tiled_elems, validate, version,
                   workspace_size)
