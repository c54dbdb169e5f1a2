import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a real MI355X (runs the HIP library)")


@pytest.fixture(scope="session")
def k2_weights():
    """K2-shape expert weights (384 experts, d 7168, I 2048, shared expert) on the GPU,
    generated once per session: about 34 GB of bf16."""
    import torch
    import synth_inputs as S
    print("generating K2-shape weights on the GPU (384 experts, d 7168, I 2048)", flush=True)
    w = S.make_weights("k2_decode", "cuda")
    torch.cuda.synchronize()
    yield w
    del w
    torch.cuda.empty_cache()
