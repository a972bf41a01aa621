import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large host-side work (full-size oracle samples)")


@pytest.fixture(scope="session")
def real_experts():
    """MXFP4 expert bytes of the real shape (6.4 GiB), generated once on the
    device by the shared input generator."""
    import torch
    from latent_mixture_experts_amd import synth

    print("generating real-shape MXFP4 expert bytes on the device", flush=True)
    ex = synth.all_expert_bytes(synth.REAL, 0, device="cuda")
    torch.cuda.synchronize()
    return ex
