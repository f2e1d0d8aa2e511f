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


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def oracle_gap(z):
    """top-1 minus top-2 logit."""
    s = np.sort(np.asarray(z, dtype=np.float64))
    return float(s[-1] - s[-2])


def compare_tokens(gpu, ref, ref_logits, gap_tol=1e-2):
    """GPU tokens must equal the oracle's until the first position whose oracle
    top-1/top-2 gap is below gap_tol (a legitimate divergence); returns the
    number of positions compared."""
    for i, (a, b) in enumerate(zip(gpu, ref)):
        if oracle_gap(ref_logits[i]) < gap_tol:
            return i
        assert a == b, f"token {i}: gpu {a} != oracle {b} (gap {oracle_gap(ref_logits[i]):.3g})"
    return min(len(gpu), len(ref))
