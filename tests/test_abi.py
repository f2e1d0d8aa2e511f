"""CPU tests of the C-ABI library: it loads, exports every symbol the header
declares, validates configurations without touching a GPU, and its host-only
DyTC router agrees with the oracle's router."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import lss_synth
import oracle
from layer_skip_self_amd import _native as N
import layer_skip_self_amd as lss

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lss.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lss_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = N.load()
    names = _declared()
    assert len(names) >= 15
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(N.SIGNATURES), set(names) ^ set(N.SIGNATURES)


def test_struct_layouts_and_limits_match_the_header(tmp_path):
    """The ctypes mirrors of the header's structs have the C compiler's field
    offsets and sizes, and the binding's limits equal the header's defines."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    structs = [N.lss_config, N.lss_tensor, N.lss_policy, N.lss_stats]
    defines = sorted(set(re.findall(r"#define\s+(LSS_[A-Z_0-9]+)\s+\d+", open(HEADER).read())))
    lines = ['#include <stdio.h>', '#include "lss.h"', "int main(void) {"]
    for st in structs:
        nm = st.__name__
        lines.append(f'  printf("{nm} size %zu\\n", sizeof({nm}));')
        for f in st._fields_:
            lines.append(f'  printf("{nm}.{f[0]} %zu\\n", offsetof({nm}, {f[0]}));')
    for d in defines:
        lines.append(f'  printf("{d} %ld\\n", (long)({d}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c11", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = dict(l.rsplit(" ", 1) for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                          check=True).stdout.splitlines())
    for st in structs:
        nm = st.__name__
        assert int(got[f"{nm} size"]) == C.sizeof(st), nm
        for f in st._fields_:
            assert int(got[f"{nm}.{f[0]}"]) == getattr(st, f[0]).offset, (nm, f[0])
    mirrored = [d for d in defines if hasattr(N, d)]
    assert {"LSS_STOP_MAX", "LSS_LEVELS_MAX", "LSS_TREE_NODES_MAX", "LSS_WINDOW_MAX"} <= set(mirrored)
    for d in mirrored:
        assert int(got[d]) == getattr(N, d), d


def test_null_engine_calls_are_rejected():
    lib = N.load()
    assert lib.lss_set_gemv_grid(None, 1) == N.LSS_EINVAL
    assert lib.lss_set_sampling(None, 1.0, 0) == N.LSS_EINVAL


def test_workspace_size_and_invalid_configs():
    sh = lss_synth.SHAPES["llama3_8b"]
    nb = lss.workspace_bytes(sh, max_seq=1600, max_rows=16)
    kv = 2 * 32 * 8 * 1600 * 128 * 4          # float32 KV cache (default)
    assert kv < nb < kv + 200 * 2**20
    assert lss.workspace_bytes(sh, max_seq=1600, max_rows=16, kv_dtype="bf16") == nb - kv // 2
    lib = N.load()
    for field, bad in [("head_dim", 96), ("max_rows", 65), ("max_rows", 0), ("d_model", 8208),
                       ("n_kv_heads", 5), ("dtype", 7), ("max_seq", 1), ("kv_dtype", 3), ("max_seqs", 65),
                       ("max_seqs", -1)]:
        cfg = lss.make_config(sh, 1600, 16)
        setattr(cfg, field, bad)
        assert lib.lss_workspace_bytes(C.byref(cfg)) == 0, field
        h = C.c_void_p()
        rc = lib.lss_create(C.byref(cfg), None, 0, None, 0, None, C.byref(h))
        assert rc == N.LSS_EINVAL and not h.value


def test_create_rejects_bad_pointers_without_gpu():
    sh = lss_synth.SHAPES["tiny"]
    lib = N.load()
    cfg = lss.make_config(sh, 64, 8)
    h = C.c_void_p()
    n = 3 + 9 * sh.n_layers
    ptrs = (C.c_void_p * n)(*([0x1000] * n))
    assert lib.lss_create(C.byref(cfg), ptrs, n - 1, C.c_void_p(0x100000), 1 << 30, None, C.byref(h)) == N.LSS_EINVAL
    ptrs[5] = 0x1001                      # misaligned tensor
    assert lib.lss_create(C.byref(cfg), ptrs, n, C.c_void_p(0x100000), 1 << 30, None, C.byref(h)) == N.LSS_EINVAL
    ptrs[5] = 0x1000
    assert lib.lss_create(C.byref(cfg), ptrs, n, C.c_void_p(0x100000), 16, None, C.byref(h)) == N.LSS_ECAPACITY
    assert lib.lss_seq_len(None) == -1


def test_router_plan_matches_oracle():
    rng = np.random.default_rng(7)
    for _ in range(200):
        nl = int(rng.integers(1, 4))
        a = list(rng.uniform(0, 1, nl))
        if rng.uniform() < 0.2:
            a = [float(round(x, 1)) for x in a]
        t = list(rng.uniform(0.05, 1.0, nl))
        tv = float(rng.uniform(0.5, 2.0))
        k = int(rng.integers(0, 9))
        assert lss.router_plan(a, t, tv, k) == oracle.plan_cascade(a, t, tv, k)


def test_router_update_matches_oracle_bitwise():
    rng = np.random.default_rng(8)
    for _ in range(200):
        nl = 3
        a = list(rng.uniform(0, 1, nl))
        k = int(rng.integers(0, 9))
        levels = sorted((int(x) for x in rng.integers(0, nl, k)), reverse=True)
        n = int(rng.integers(0, k + 1))
        assert lss.router_update(a, levels, n) == oracle.update_cascade(a, levels, n)


def test_router_plan_tree_matches_oracle():
    """The tree router of the library against the oracle's, with and without
    row costs (random, rounded and extreme rates; several node budgets)."""
    rng = np.random.default_rng(17)
    for i in range(300):
        nl = int(rng.integers(1, 4))
        a = list(rng.uniform(0, 1, nl))
        if rng.uniform() < 0.2:
            a = [float(round(x, 1)) for x in a]
        t = list(rng.uniform(0.05, 1.0, nl))
        tv = float(rng.uniform(0.5, 2.0))
        k = int(rng.integers(0, 9))
        bmax = int(rng.integers(1, 9))
        nodes = int(rng.integers(1, 16))
        rc = None if i % 2 else [1.0 + float(rng.uniform(0, 0.2)) * r for r in range(16)]
        assert lss.router_plan_tree(a, t, tv, rc, k, bmax, nodes) == oracle.plan_tree(a, t, tv, rc, k, bmax, nodes)


def test_router_update_tree_matches_oracle_bitwise():
    rng = np.random.default_rng(18)
    for _ in range(300):
        nl = 3
        a = list(rng.uniform(0, 1, nl))
        D = int(rng.integers(0, 9))
        levels = sorted((int(x) for x in rng.integers(0, nl, D)), reverse=True)
        n = int(rng.integers(0, D + 1))
        branch = int(rng.integers(0, 4)) if n else -1
        assert lss.router_update_tree(a, levels, n, branch) == oracle.update_tree(a, levels, n, branch)
    with pytest.raises(lss.LssError):
        lss.router_update_tree([0.5], [0, 0], 1, -1)          # n > 0 needs the branch followed
    with pytest.raises(lss.LssError):
        lss.router_plan_tree([0.5], [0.1], 1.0, None, 8, 9)   # width above 8


def test_latency_fit_matches_oracle():
    rng = np.random.default_rng(9)
    samples = [(s, d, 0.3 + 2e-4 * s + 0.04 * d + rng.normal(0, 0.01))
               for s in (128, 512, 1024, 2048) for d in (10, 22, 32)]
    np.testing.assert_allclose(lss.latency_fit(samples), oracle.fit_latency(samples), rtol=1e-9, atol=1e-12)


def test_router_rejects_bad_arguments():
    with pytest.raises(lss.LssError):
        lss.router_plan([0.5] * 5, [1.0] * 5, 1.0, 8)
    with pytest.raises(lss.LssError):
        lss.router_update([0.5, 0.5], [0, 3], 1)


def test_load_weights_checks_names_and_sizes_without_gpu():
    """lss_load_weights validates every tensor's canonical name and element
    count before touching a device, and reports why through
    lss_last_error(NULL)."""
    sh = lss_synth.SHAPES["tiny"]
    lib = N.load()
    cfg = lss.make_config(sh, 64, 8)
    names = lss_synth.shapes.tensor_names(sh)
    numel = [int(np.prod(lss_synth.shapes.tensor_shape(sh, nm))) for nm in names]
    keep = [nm.encode() for nm in names]

    def tensors(nms, sizes):
        return (N.lss_tensor * len(nms))(*[N.lss_tensor(nm, 0x1000, sz) for nm, sz in zip(nms, sizes)])

    h = C.c_void_p()
    n = len(names)
    # correct names and sizes, fake aligned pointers: only the workspace size fails
    rc = lib.lss_load_weights(C.byref(cfg), tensors(keep, numel), n, C.c_void_p(0x100000), 16, None, C.byref(h))
    assert rc == N.LSS_ECAPACITY and not h.value
    bad = list(keep)
    bad[7] = b"layers.0.wx"
    rc = lib.lss_load_weights(C.byref(cfg), tensors(bad, numel), n, C.c_void_p(0x100000), 1 << 30, None, C.byref(h))
    assert rc == N.LSS_EINVAL
    assert b"layers.0.wo" in lib.lss_last_error(None)
    sizes = list(numel)
    sizes[2] -= 1                             # lm_head one element short
    rc = lib.lss_load_weights(C.byref(cfg), tensors(keep, sizes), n, C.c_void_p(0x100000), 1 << 30, None, C.byref(h))
    assert rc == N.LSS_EINVAL
    assert b"lm_head" in lib.lss_last_error(None)
    rc = lib.lss_load_weights(C.byref(cfg), tensors(keep, numel), n - 1, C.c_void_p(0x100000), 1 << 30, None,
                              C.byref(h))
    assert rc == N.LSS_EINVAL


def test_workspace_grows_by_one_cache_per_sequence():
    """max_seqs sequences: one KV cache (keys and values), layer-selection
    target, token slots and result block each, plus a few partials blocks."""
    sh = lss_synth.SHAPES["llama3_8b"]
    one = lss.workspace_bytes(sh, max_seq=1600, max_rows=64)
    four = lss.workspace_bytes(sh, max_seq=1600, max_rows=64, max_seqs=4)
    kv = 2 * 32 * 8 * 1600 * 128 * 4
    assert one == lss.workspace_bytes(sh, max_seq=1600, max_rows=64, max_seqs=0)
    assert 3 * kv < four - one < 3 * kv + 16 * 2**20
