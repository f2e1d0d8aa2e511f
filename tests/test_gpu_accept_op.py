"""GPU parity of the stand-alone greedy acceptance op
(``lss_op_accept_greedy``): the argmax of every verify row and the
accept-prefix / bonus rule against the oracle's (``oracle.argmax_first``,
``oracle.accept``), bit for bit (integer results), over row counts 1..16
and vocabularies that end in a ragged chunk, with planted ties (the lowest
index wins) and planted first rejections at every position."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu


def oracle_result(z, drafts):
    st = oracle.DecodeState.__new__(oracle.DecodeState)      # only the fields accept() touches
    st.p, st.valid, st.window, st.window_logits, st.tree = 0, [0], [], [], False
    n, bonus, _ = oracle.accept(st, z, [None] * len(z), list(drafts))
    return n, bonus, [oracle.argmax_first(r) for r in z]


@pytest.mark.parametrize("vocab", [1000, 4096, 4097, 32000, 128256])
def test_accept_op_vs_oracle(vocab):
    import torch
    from layer_skip_self_amd.engine import accept_greedy
    rng = np.random.default_rng(vocab)
    for rows in (1, 2, 5, 9, 16):
        z = rng.standard_normal((rows, vocab)).astype(np.float32)
        # planted ties: a row's maximum repeated at a higher index loses to the lower one
        for r in range(0, rows, 2):
            i, j = sorted(rng.choice(vocab, 2, replace=False))
            z[r, i] = z[r, j] = np.max(z[r]) + 1.0
        am = [oracle.argmax_first(r) for r in z]
        for reject in range(rows):                      # first rejected draft at `reject` (rows - 1: none)
            drafts = list(am[:rows - 1])
            if reject < rows - 1:
                drafts[reject] = (drafts[reject] + 1) % vocab
            res = accept_greedy(torch.from_numpy(z).cuda(), torch.tensor(drafts, dtype=torch.int32).cuda())
            torch.cuda.synchronize()
            got = res.cpu().numpy().tolist()
            n, bonus, amo = oracle_result(z, drafts)
            assert got[0] == n == min(reject, rows - 1), (rows, reject)
            assert got[1] == bonus
            assert got[2:] == amo


def test_accept_op_nan_rule_and_errors():
    import torch
    from layer_skip_self_amd.engine import accept_greedy, LssError
    z = np.zeros((3, 5000), np.float32)
    z[0, 4321] = 2.0
    z[0, 10] = np.nan                                   # NaN never wins
    z[1, :] = np.nan                                    # a row of NaNs gives index 0
    z[2, 4999] = 1.0
    res = accept_greedy(torch.from_numpy(z).cuda(), torch.tensor([4321, 0], dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    assert res.cpu().numpy().tolist() == [2, 4999, 4321, 0, 4999]
    with pytest.raises(LssError):
        accept_greedy(torch.zeros((65, 16), device="cuda"), torch.zeros(64, dtype=torch.int32, device="cuda"))
