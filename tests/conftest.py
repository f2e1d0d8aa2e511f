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


def compare_dp(gpu_dec, oracle_dec, cos_tol, margin):
    """Compare the GPU's layer-selection decisions ([L+1][L+1][3] float
    triples {skip chosen, cos skip, cos exec}) with the oracle's
    (``oracle.clasp_dp``'s dict), stage by stage.

    A state (i, j) is *tainted* when the oracle's decision there has a
    skip/execute margin below ``margin`` (either path may legitimately pick
    either candidate) or the candidate it keeps came from a tainted state.
    Every cosine whose source state is untainted must agree within
    ``cos_tol``; every decision whose candidates are untainted and whose
    margin clears ``margin`` must be equal.  Returns (decisions compared,
    decisions in total, cosines compared, worst cosine error, tainted)."""
    tainted = {(0, 0): False}
    n_dec = n_cos = total = 0
    worst = 0.0
    for (i, j) in sorted(oracle_dec):
        take, cs, ce = oracle_dec[(i, j)]
        total += 1
        e_ok = ce is not None and not tainted.get((i - 1, j), True)
        s_ok = cs is not None and not tainted.get((i - 1, j - 1), True)
        if e_ok:
            err = abs(float(gpu_dec[i, j, 2]) - ce)
            worst = max(worst, err)
            n_cos += 1
            assert err <= cos_tol, f"cos(exec) at ({i},{j}): gpu {gpu_dec[i, j, 2]} oracle {ce}"
        if s_ok:
            err = abs(float(gpu_dec[i, j, 1]) - cs)
            worst = max(worst, err)
            n_cos += 1
            assert err <= cos_tol, f"cos(skip) at ({i},{j}): gpu {gpu_dec[i, j, 1]} oracle {cs}"
        cand_ok = (ce is None or e_ok) and (cs is None or s_ok)
        m = abs(cs - ce) if (cs is not None and ce is not None) else float("inf")
        if cand_ok and m >= margin:
            assert (gpu_dec[i, j, 0] != 0) == bool(take), f"decision at ({i},{j}), margin {m:.3g}"
            n_dec += 1
            tainted[(i, j)] = False
        else:
            tainted[(i, j)] = True
    return n_dec, total, n_cos, worst, tainted


def greedy_ids_vs_oracle(eng, model, prompt, st0, z0, n_steps, tol):
    """The token rule of the parity protocol along a greedy run: the GPU
    decodes ``n_steps`` tokens after the prompt (one-row verify steps, the
    autoregressive path) and the oracle re-runs every position on the GPU's
    own tokens (teacher forcing from its prefill state ``st0`` and logits
    ``z0``).  Logits must agree within ``tol`` everywhere; the GPU's token
    must be the oracle's argmax wherever the oracle's top-1/top-2 gap is at
    least 1e-2.  Returns (positions whose ids were compared, positions,
    worst logit error)."""
    import copy
    import oracle
    toks = [eng.prefill(prompt)]
    zg = [eng.read_logits(1)[0].copy()]
    for _ in range(n_steps):
        eng.verify(None, 0)
        zg.append(eng.read_logits(1)[0].copy())
        _, b, _ = eng.accept()
        toks.append(b)
    so = copy.deepcopy(st0)
    zo = [z0]
    for j in range(n_steps):
        zz, _ = oracle.forward_row(model, so, toks[j], so.p, "full")
        so.p += 1
        zo.append(zz)
    compared, worst = 0, 0.0
    for j in range(n_steps + 1):
        worst = max(worst, float(np.max(np.abs(zg[j] - zo[j]))))
        if oracle_gap(zo[j]) >= 1e-2:
            assert toks[j] == int(np.argmax(zo[j])), f"position {j}"
            compared += 1
    assert worst <= tol, worst
    return compared, n_steps + 1, worst
