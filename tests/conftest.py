import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library through its C ABI")
    # Load what is built; build a piece only when it is missing.
    import __graft_entry__ as g

    if not os.path.exists(os.path.join(ROOT, "oracle", "libmoge_oracle.so")):
        g.build_oracle()
    if not (os.path.exists(os.path.join(ROOT, "synth", "libsynth_cpu.so"))
            and os.path.exists(os.path.join(ROOT, "synth", "libsynth_gpu.so"))):
        g.build_synth()
    import glob

    if (not os.path.exists(os.path.join(ROOT, "mixture_grouped_experts_amd", "libmoge.so"))
            and glob.glob(os.path.join(ROOT, "mixture_grouped_experts_amd", "csrc", "*.hip"))):
        g.build_moge()


@pytest.fixture(scope="session")
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    return torch.device("cuda:0")
