"""The allocation-free acceptance entry point (``lss_op_accept_greedy_noalloc``,
library-owned scratch) against the workspace entry point
(``lss_op_accept_greedy``) through the C ABI: identical results on two calls
in a row, the second with a smaller input (the shared scratch keeps the
first call's records, which must not leak into the second), and the size
limit rejected with LSS_ECAPACITY."""
import ctypes as C

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _call(lib, z, drafts, noalloc):
    import torch
    rows, vocab = z.shape
    res = torch.full((2 + rows,), -7, dtype=torch.int32, device="cuda")
    dp = C.c_void_p(drafts.data_ptr()) if drafts.numel() else None
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if noalloc:
        rc = lib.lss_op_accept_greedy_noalloc(C.c_void_p(z.data_ptr()), rows, vocab, dp, C.c_void_p(res.data_ptr()),
                                              stream)
    else:
        nb = int(lib.lss_op_accept_greedy_workspace_bytes(rows, vocab))
        ws = torch.empty((nb,), dtype=torch.uint8, device="cuda")
        rc = lib.lss_op_accept_greedy(C.c_void_p(z.data_ptr()), rows, vocab, dp, C.c_void_p(res.data_ptr()),
                                      C.c_void_p(ws.data_ptr()), nb, stream)
    assert rc == 0, lib.lss_last_error(None)
    torch.cuda.synchronize()
    return res.cpu().numpy().tolist()


def test_noalloc_matches_workspace_entry_point():
    import torch
    from layer_skip_self_amd import _native as N
    lib = N.load()
    rng = np.random.default_rng(5)
    # first call: 12 rows of the 8B vocabulary; second: 3 rows of 5000 (smaller)
    outs = []
    for rows, vocab in ((12, 128256), (3, 5000)):
        z = torch.from_numpy(rng.standard_normal((rows, vocab)).astype(np.float32)).cuda()
        am = torch.argmax(z, dim=1).to(torch.int32)
        drafts = am[:rows - 1].clone()
        if rows > 2:
            drafts[rows - 3] += 1                       # first rejection at rows - 3
        a = _call(lib, z, drafts, noalloc=True)
        b = _call(lib, z, drafts, noalloc=False)
        assert a == b, (rows, vocab)
        assert a[0] == (rows - 3 if rows > 2 else rows - 1)
        outs.append(a)
    assert outs[0] != outs[1]
    z = torch.zeros((2, N.LSS_ACCEPT_VOCAB_MAX + 16), device="cuda")
    res = torch.zeros((4,), dtype=torch.int32, device="cuda")
    d = torch.zeros((1,), dtype=torch.int32, device="cuda")
    rc = lib.lss_op_accept_greedy_noalloc(C.c_void_p(z.data_ptr()), 2, N.LSS_ACCEPT_VOCAB_MAX + 16,
                                          C.c_void_p(d.data_ptr()), C.c_void_p(res.data_ptr()), None)
    assert rc == N.LSS_ECAPACITY
    assert b"LSS_ACCEPT_VOCAB_MAX" in lib.lss_last_error(None)
