"""moge_round_bf16, the float32 -> bf16 rounding the library applies where it stores bf16
values (h and the expert outputs), against round-to-nearest-even restated on the host."""
import numpy as np
import pytest
import torch

import mixture_grouped_experts_amd as moge

pytestmark = pytest.mark.gpu


def _rne(u32: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even of binary32 bit patterns to their top 16 bits (non-NaN inputs):
    add half an ulp of the kept part, minus one unless the kept part is odd, and truncate."""
    u = u32.astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _inputs() -> np.ndarray:
    special = [0x00000000, 0x80000000, 0x00000001, 0x007FFFFF, 0x00008000, 0x00018000, 0x807F8000,
               0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x7F800000, 0xFF800000, 0x7FC00000,
               0x7F800001, 0xFF800123, 0x7F960000, 0x3F808000, 0x3F818000, 0x3F807FFF, 0x3F808001,
               0x00800000]
    # every exponent, both signs: exact, just below / at / just above the tie, odd kept part
    mant = [0x0000, 0x7FFF, 0x8000, 0x8001, 0x18000, 0x17FFF, 0x7F8000, 0x7FFFFF]
    grid = [(s << 31) | (e << 23) | m for s in (0, 1) for e in range(256) for m in mant]
    rand = np.random.default_rng(7).integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64)
    return np.concatenate([np.array(special + grid, dtype=np.uint64), rand]).astype(np.uint32)


def test_round_bf16_is_round_to_nearest_even(gpu):
    u = _inputs()
    x = torch.from_numpy(u.view(np.float32).copy()).cuda()
    y = torch.empty(u.size, dtype=torch.int16, device="cuda")
    moge.round_bf16(x, y)
    torch.cuda.synchronize()
    got = y.cpu().numpy().view(np.uint16)
    nan = ((u & 0x7F800000) == 0x7F800000) & ((u & 0x007FFFFF) != 0)
    assert np.array_equal(got[~nan], _rne(u[~nan]))
    g = got[nan]
    assert (((g & 0x7F80) == 0x7F80) & ((g & 0x007F) != 0)).all()   # a NaN stays a NaN


def test_round_bf16_empty_and_ragged(gpu):
    for n in (0, 1, 255, 257, 65536 * 256 + 3):
        x = torch.randn(n, device="cuda")
        y = torch.full((n,), -1, dtype=torch.int16, device="cuda")
        moge.round_bf16(x, y)
        torch.cuda.synchronize()
        if n:
            exp = _rne(x.cpu().numpy().view(np.uint32))
            assert np.array_equal(y.cpu().numpy().view(np.uint16), exp)
