"""The seeded input generator: C filler == NumPy transcription of the definition; distribution sanity;
bf16 rounding agrees with torch's binary32 -> bfloat16 conversion (round to nearest even)."""
import numpy as np
import torch

import synth


def test_c_matches_numpy_definition():
    for seed, tid, start, n, std, bf16 in ((0, 1, 0, 5000, 1.0, False), (7, 6, 123456789, 3000, 0.02, True),
                                           (2 ** 40, 3, 10, 100, 2.0, False)):
        a = synth.normal_host(seed, tid, n, std, bf16, start)
        b = synth.normal_np(seed, tid, n, std, bf16, start)
        assert a.dtype == b.dtype and (a.view(np.uint8) == b.view(np.uint8)).all()


def test_offsets_are_consistent():
    a = synth.normal_host(1, 2, 1000, 1.0, False)
    b = synth.normal_host(1, 2, 400, 1.0, False, start=600)
    assert (a[600:] == b).all()


def test_moments():
    v = synth.normal_host(0, 1, 2_000_000, 1.0, False).astype(np.float64)
    assert abs(v.mean()) < 3e-3 and abs(v.std() - 1.0) < 3e-3
    assert abs(((v ** 4).mean()) - 2.9) < 0.05    # twelve-uniform variate: kurtosis 3 - 1.2/12


def test_bf16_round_nearest_even_matches_torch():
    f = synth.normal_host(5, 9, 100000, 0.02, False)
    b = synth.normal_host(5, 9, 100000, 0.02, True)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (b == ref).all()
