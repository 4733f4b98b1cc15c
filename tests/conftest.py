import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size CPU work (seconds to minutes)")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.load()
    return oracle


@pytest.fixture(scope="session")
def s2():
    """Layer 0 of the wide workload (H=4096, I=1536, 128 experts) on cuda:0, shared
    by every GPU test module (generating it takes ~15 s)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_inputs as mi
    from tests.test_gpu_parity import DevLayer
    s = mi.SHAPES["S2"]
    return DevLayer(mi.make_layer(mi.layer_seed("wide_layers", 0), s["H"], s["I"], s["E"]), torch.device("cuda:0"))
