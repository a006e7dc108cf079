import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: minutes of CPU work")


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


# ---------------------------------------------------------------- GPU fixtures
@pytest.fixture(scope="session")
def phi():
    import logits_parity_amd as phi_mod
    phi_mod.lib()  # raises when libphi.so is missing: no fallback path
    return phi_mod


@pytest.fixture(scope="session")
def mini_f16():
    """Host float16 weights of the Phi-3-mini-shaped model (seed 1) and their
    device copies."""
    import synth
    from logits_parity_amd.weights import to_device
    ws = synth.WeightSet(synth.MINI)
    dev = to_device(ws, synth.MINI.n_layers, "cuda")
    return ws, dev


@pytest.fixture(scope="session")
def mini_w8():
    import synth
    from logits_parity_amd.weights import to_device
    ws = synth.WeightSet(synth.MINI_W8)
    dev = to_device(ws, synth.MINI_W8.n_layers, "cuda")
    return ws, dev
