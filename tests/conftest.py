import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def tiny_shape():
    import lss_synth
    return lss_synth.SHAPES["tiny"]


@pytest.fixture(scope="session")
def tiny_weights_np(tiny_shape):
    import lss_synth
    return lss_synth.weights_to_numpy(lss_synth.make_weights(tiny_shape))


@pytest.fixture(scope="session")
def tiny_model(tiny_shape, tiny_weights_np):
    import oracle
    return oracle.OracleModel(tiny_shape, tiny_weights_np, dtype=np.float64)


@pytest.fixture(scope="session")
def tiny_prompt(tiny_shape):
    import lss_synth
    return lss_synth.make_prompt(tiny_shape, 32)
