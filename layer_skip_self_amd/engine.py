"""Python face of the engine: the C-ABI calls of include/lss.h with the same
names, plus device-memory plumbing (torch allocates the workspace, the stream
comes from torch).  Every decoding step runs in liblss.so."""
import ctypes as C

import numpy as np

from . import _native as N


class LssError(RuntimeError):
    def __init__(self, what, rc, msg=""):
        super().__init__(f"{what}: {N.STATUS_NAMES.get(rc, rc)} {msg}".strip())
        self.rc = rc


def _i32(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return a, a.ctypes.data_as(C.POINTER(C.c_int32))


def _u8(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.uint8))
    return a, a.ctypes.data_as(C.POINTER(C.c_uint8))


def make_config(shape, max_seq, max_rows=16, kv_dtype="f32", max_seqs=1):
    """``kv_dtype``: "f32" (default) or "bf16".  A bf16 KV cache moves the
    Llama-3-8B-shaped logits ~8e-2 away from the exact result, a float32 one
    ~2e-4, for ~2% more bytes per decoded token at 1.5K context.
    ``max_seqs``: independent sequences the engine holds (each its own KV
    cache of ``max_seq`` positions)."""
    wdt = N.LSS_BF16 if shape.dtype == "bf16" else N.LSS_F32
    kdt = N.LSS_BF16 if kv_dtype == "bf16" else N.LSS_F32
    return N.lss_config(shape.n_layers, shape.d_model, shape.n_heads, shape.n_kv_heads, shape.head_dim,
                        shape.ffn_dim, shape.vocab, float(shape.rope_theta), float(shape.rms_eps),
                        wdt, int(max_seq), int(max_rows), kdt, int(max_seqs))


def workspace_bytes(shape, max_seq, max_rows=16, kv_dtype="f32", max_seqs=1):
    cfg = make_config(shape, max_seq, max_rows, kv_dtype, max_seqs)
    return int(N.load().lss_workspace_bytes(C.byref(cfg)))


class Engine:
    """One GPU engine holding ``max_seqs`` independent sequences (one by
    default).  ``weights``: ``[(name, tensor)]`` in the canonical order on
    the CUDA device (they are borrowed, not copied)."""

    def __init__(self, shape, weights, max_seq, max_rows=16, stream=None, device="cuda", kv_dtype="f32",
                 max_seqs=1):
        import torch
        self.lib = N.load()
        self.shape = shape
        self.cfg = make_config(shape, max_seq, max_rows, kv_dtype, max_seqs)
        self._tensors = [t for _, t in weights]
        n = len(self._tensors)
        nbytes = self.lib.lss_workspace_bytes(C.byref(self.cfg))
        if nbytes == 0:
            raise LssError("lss_workspace_bytes", N.LSS_EINVAL, "invalid config")
        self._ws = torch.empty(int(nbytes), dtype=torch.uint8, device=device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self._ws.device)
        self._names = [name.encode() for name, _ in weights]
        tens = (N.lss_tensor * n)(*[N.lss_tensor(nm, t.data_ptr(), t.numel())
                                    for nm, t in zip(self._names, self._tensors)])
        h = C.c_void_p()
        rc = self.lib.lss_load_weights(C.byref(self.cfg), tens, n, C.c_void_p(self._ws.data_ptr()), nbytes,
                                       C.c_void_p(self.stream.cuda_stream), C.byref(h))
        if rc != 0:
            msg = self.lib.lss_last_error(None)
            raise LssError("lss_load_weights", rc, msg.decode() if msg else "")
        self.h = h

    # -------------------------------------------------------------- helpers
    def _check(self, rc, what):
        if rc != 0:
            msg = self.lib.lss_last_error(self.h)
            raise LssError(what, rc, msg.decode() if msg else "")

    def close(self):
        if getattr(self, "h", None):
            self.lib.lss_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def seq_len(self):
        return int(self.lib.lss_seq_len(self.h))

    # -------------------------------------------------------------- hot path
    def attach_w8(self):
        """int8 copy of every layer's weights for the W8A8 draft (quant = 2),
        in a device buffer this object owns."""
        import torch
        nbytes = int(self.lib.lss_w8_bytes(C.byref(self.cfg)))
        self._w8 = torch.empty(nbytes, dtype=torch.uint8, device=self._ws.device)
        self._check(self.lib.lss_attach_w8(self.h, C.c_void_p(self._w8.data_ptr()), nbytes), "lss_attach_w8")

    def set_sampling(self, temperature, seed=0):
        """Speculative sampling at ``temperature`` with ``seed`` (0: greedy)."""
        self._check(self.lib.lss_set_sampling(self.h, float(temperature), int(seed) % 2**64), "lss_set_sampling")

    def set_gemv_grid(self, wgs_per_cu):
        """Decode-GEMV grid: 0 = one workgroup per weight tile, n > 0 = at
        most n workgroups per compute unit walking tile ranges (same bits)."""
        self._check(self.lib.lss_set_gemv_grid(self.h, int(wgs_per_cu)), "lss_set_gemv_grid")

    DECODE_KERNELS = {"vector": 0, "mfma": 1, "mfma_verify": 2}

    def set_decode_kernel(self, kind):
        """Decode rows with bf16 weights: "vector" (the vector-ALU GEMV, the
        default), "mfma" (one MFMA GEMM launch for up to 16 rows) or
        "mfma_verify" (MFMA for verify and greedy rows, vector for drafts)."""
        self._check(self.lib.lss_set_decode_kernel(self.h, self.DECODE_KERNELS[kind]), "lss_set_decode_kernel")

    def prefill(self, tokens):
        a, p = _i32(tokens)
        t0 = C.c_int32()
        self._check(self.lib.lss_prefill(self.h, p, len(a), C.byref(t0)), "lss_prefill")
        return int(t0.value)

    def draft(self, skip_mask, quant=0, k=1, exit_tau=0.0):
        """quant: 0 / False full precision, 1 / True int8 activations, 2 int8
        activations and int8 weights (``attach_w8`` first)."""
        m, mp = _u8(skip_mask)
        out = np.zeros(max(k, 1), np.int32)
        done = C.c_int32()
        self._check(self.lib.lss_draft(self.h, mp, int(quant), int(k), float(exit_tau),
                                       out.ctypes.data_as(C.POINTER(C.c_int32)), C.byref(done)), "lss_draft")
        return out[:done.value].tolist()

    def draft_tree(self, skip_mask, quant=0, B=2, D=1, levels=None):
        """Token tree of width B and depth D: the draft's B most likely next
        tokens, each extended greedily by D - 1 more.  ``levels``: D pairs
        (skip mask, quant), the draft level of each depth (then
        ``skip_mask`` and ``quant`` are ignored).  Returns the branches
        ([B][D] token lists)."""
        out = np.zeros(max(B * D, 1), np.int32)
        op = out.ctypes.data_as(C.POINTER(C.c_int32))
        if levels is None:
            m, mp = _u8(skip_mask)
            self._check(self.lib.lss_draft_tree(self.h, mp, int(quant), int(B), int(D), op), "lss_draft_tree")
        else:
            m, mp = _u8(np.asarray([lv[0] for lv in levels], np.uint8).reshape(-1))
            q, qp = _i32([int(lv[1]) for lv in levels])
            self._check(self.lib.lss_draft_tree_levels(self.h, mp, qp, int(B), int(D), op), "lss_draft_tree_levels")
        return [out[b * D:(b + 1) * D].tolist() for b in range(B)]

    def verify(self, drafts=None, k=None):
        if drafts is None:
            self._check(self.lib.lss_verify(self.h, None, int(k)), "lss_verify")
        else:
            a, p = _i32(drafts)
            self._check(self.lib.lss_verify(self.h, p, len(a)), "lss_verify")

    def accept(self):
        n, b = C.c_int32(), C.c_int32()
        out = np.zeros(N.LSS_ROWS_MAX, np.int32)
        self._check(self.lib.lss_accept_and_rollback(self.h, C.byref(n), C.byref(b),
                                                     out.ctypes.data_as(C.POINTER(C.c_int32))),
                    "lss_accept_and_rollback")
        return int(n.value), int(b.value), out[:n.value + 1].tolist()

    def select_layers_dp(self, n_skip, n_layers_eff=None):
        L = self.shape.n_layers
        mask = np.zeros(L, np.uint8)
        score = C.c_float()
        mp = mask.ctypes.data_as(C.POINTER(C.c_uint8))
        if n_layers_eff is None:
            self._check(self.lib.lss_select_layers_dp(self.h, int(n_skip), mp, C.byref(score)), "lss_select_layers_dp")
        else:
            self._check(self.lib.lss_select_layers_dp_exit(self.h, int(n_skip), int(n_layers_eff), mp, C.byref(score)),
                        "lss_select_layers_dp_exit")
        return mask.tolist(), float(score.value)

    def calibrate_latency(self, prompt, seq_lens, depths, reps=5):
        """Fit the DyTC latency model t = b0 + b1 * seq_len + b2 * depth
        (CAS-Spec blog, latency prediction section) to timed one-token draft
        steps: for every seq_len, prefill ``prompt[:seq_len]``, then for every
        depth draft one token with the first ``depth`` layers executed, verify
        it and accept.  Each draft is timed with HIP events recorded on the
        engine stream around ``lss_draft``; the first repetition per
        (seq_len, depth) is not timed and the median of the other ``reps``
        is one sample.  Returns (beta, samples [(seq_len, depth, seconds)],
        max relative error of the fit over the samples)."""
        import torch
        L = self.shape.n_layers
        samples = []
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for s in seq_lens:
            self.prefill(list(prompt[:s]))
            for depth in depths:
                mask = [0] * int(depth) + [1] * (L - int(depth))
                times, ps = [], []
                for r in range(reps + 1):
                    p = self.seq_len
                    ev0.record(self.stream)
                    self.draft(mask, k=1)
                    ev1.record(self.stream)
                    ev1.synchronize()
                    dt = ev0.elapsed_time(ev1) * 1e-3
                    self.verify(k=1)
                    self.accept()
                    if r:
                        times.append(dt)
                        ps.append(p)
                samples.append((int(np.median(ps)), int(depth), float(np.median(times))))
        beta = latency_fit(samples)
        err = max(abs(beta[0] + beta[1] * s + beta[2] * d - t) / t for s, d, t in samples)
        return beta, samples, err

    def calibrate_row_cost(self, prompt, max_rows=16, reps=5, seed=0):
        """Cost factors of a pass over r rows for the tree router
        (``row_cost`` of a cascade tree policy): the median time of a
        teacher-forced verify of r rows (the pending token and r - 1 seeded
        random drafts) over the median one-row verify, r = 1 .. max_rows,
        each timed with HIP events recorded on the engine stream after one
        untimed repetition.  Returns the list of max_rows factors."""
        import torch
        rng = np.random.default_rng(seed)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        med = []
        for r in range(1, max_rows + 1):
            self.prefill(list(prompt))
            times = []
            for i in range(reps + 1):
                drafts = rng.integers(0, self.shape.vocab, r - 1).astype(np.int32)
                ev0.record(self.stream)
                self.verify(drafts=drafts)
                ev1.record(self.stream)
                ev1.synchronize()
                if i:
                    times.append(ev0.elapsed_time(ev1))
                self.accept()
            med.append(float(np.median(times)))
        return [m / med[0] for m in med]

    def generate(self, prompt, n_gen, policy):
        """Prefill + decoding of n_gen tokens under ``policy`` (``make_policy``;
        its ``temperature`` / ``seed`` select greedy decoding or sampling,
        ``stop`` a tuple of token ids that end it early).  Returns (the
        emitted tokens, stats)."""
        self.set_sampling(policy.get("temperature", 0.0), policy.get("seed", 0))
        if "decode_kernel" in policy:
            self.set_decode_kernel(policy["decode_kernel"])
        a, p = _i32(prompt)
        pol = make_policy(policy, self.shape.n_layers)
        out = np.zeros(n_gen, np.int32)
        st = N.lss_stats()
        self._check(self.lib.lss_generate(self.h, p, len(a), int(n_gen), C.byref(pol),
                                          out.ctypes.data_as(C.POINTER(C.c_int32)), C.byref(st)), "lss_generate")
        return out[:st.emitted].tolist(), {f: getattr(st, f) for f, _ in N.lss_stats._fields_}

    # -------------------------------------------------------------- several sequences
    def select(self, seq):
        """Make sequence ``seq`` the one every single-sequence call acts on."""
        self._check(self.lib.lss_seq_select(self.h, int(seq)), "lss_seq_select")

    def batch_draft(self, seqs, masks, k, quant=0, exit_tau=0.0):
        """Draft up to ``k[i]`` tokens for each sequence ``seqs[i]`` with
        skip mask ``masks[i]``; returns the drafted token lists."""
        n = len(seqs)
        s, sp = _i32(seqs)
        kk, kp = _i32(k)
        m, mp = _u8(np.asarray(masks, dtype=np.uint8).reshape(n, self.shape.n_layers))
        out = np.zeros((n, N.LSS_WINDOW_MAX), np.int32)
        done = np.zeros(n, np.int32)
        self._check(self.lib.lss_batch_draft(self.h, n, sp, mp, int(quant), kp, float(exit_tau),
                                             out.ctypes.data_as(C.POINTER(C.c_int32)),
                                             done.ctypes.data_as(C.POINTER(C.c_int32))), "lss_batch_draft")
        return [out[i, :done[i]].tolist() for i in range(n)]

    def batch_verify(self, seqs):
        s, sp = _i32(seqs)
        self._check(self.lib.lss_batch_verify(self.h, len(seqs), sp), "lss_batch_verify")

    def batch_accept(self, seqs):
        """Returns [(n_accepted, bonus, emitted tokens)] per sequence."""
        n = len(seqs)
        s, sp = _i32(seqs)
        na = np.zeros(n, np.int32)
        bo = np.zeros(n, np.int32)
        acc = np.zeros((n, N.LSS_WINDOW_MAX + 1), np.int32)
        self._check(self.lib.lss_batch_accept(self.h, n, sp, na.ctypes.data_as(C.POINTER(C.c_int32)),
                                              bo.ctypes.data_as(C.POINTER(C.c_int32)),
                                              acc.ctypes.data_as(C.POINTER(C.c_int32))), "lss_batch_accept")
        return [(int(na[i]), int(bo[i]), acc[i, :na[i] + 1].tolist()) for i in range(n)]

    def generate_batch(self, prompts, n_gen, policy):
        """Decode every prompt (sequences 0 .. len(prompts) - 1) to ``n_gen``
        tokens with ``policy`` applied per sequence; returns (token lists,
        per-sequence stats dicts)."""
        n = len(prompts)
        lens = np.asarray([len(p) for p in prompts], np.int32)
        flat, fp = _i32(np.concatenate([np.asarray(p, np.int32) for p in prompts]))
        _, lp = _i32(lens)
        self.set_sampling(policy.get("temperature", 0.0), policy.get("seed", 0))   # batches refuse sampling
        if "decode_kernel" in policy:
            self.set_decode_kernel(policy["decode_kernel"])
        pol = make_policy(policy, self.shape.n_layers)
        out = np.zeros((n, n_gen), np.int32)
        st = (N.lss_stats * n)()
        self._check(self.lib.lss_generate_batch(self.h, n, fp, lp, int(n_gen), C.byref(pol),
                                                out.ctypes.data_as(C.POINTER(C.c_int32)), st),
                    "lss_generate_batch")
        stats = [{f: getattr(st[i], f) for f, _ in N.lss_stats._fields_} for i in range(n)]
        return [out[i, :st[i].emitted].tolist() for i in range(n)], stats

    # -------------------------------------------------------------- measurement
    EPILOGUES = {"qkv": 0, "resid": 1, "gate_up": 2, "lm_head": 3,
                 "qkv_int8": 16, "resid_int8": 17, "gate_up_int8": 18}

    def profile_kernel(self, epilogue, rows=0, enable=True):
        self._check(self.lib.lss_profile_kernel(self.h, self.EPILOGUES[epilogue], int(rows), int(enable)),
                    "lss_profile_kernel")

    def profile_read(self):
        ms, n, b = C.c_double(), C.c_int64(), C.c_int64()
        self._check(self.lib.lss_profile_read(self.h, C.byref(ms), C.byref(n), C.byref(b)), "lss_profile_read")
        return float(ms.value), int(n.value), int(b.value)

    # -------------------------------------------------------------- parity helpers
    def read_logits(self, rows=1):
        out = np.zeros((rows, self.shape.vocab), np.float32)
        self._check(self.lib.lss_read_logits(self.h, rows, out.ctypes.data_as(C.POINTER(C.c_float))),
                    "lss_read_logits")
        return out

    def read_states(self, row=0):
        out = np.zeros((self.shape.n_layers + 1, self.shape.d_model), np.float32)
        self._check(self.lib.lss_read_states(self.h, row, out.ctypes.data_as(C.POINTER(C.c_float))),
                    "lss_read_states")
        return out

    def read_dp_decisions(self):
        L = self.shape.n_layers
        out = np.zeros((L + 1, L + 1, 3), np.float32)
        self._check(self.lib.lss_read_dp_decisions(self.h, out.ctypes.data_as(C.POINTER(C.c_float))),
                    "lss_read_dp_decisions")
        return out


def make_policy(policy, n_layers):
    """``policy``: dict with ``mode`` in {"ar", "static", "dp", "cascade"} and
    the matching fields of ``lss_policy`` (``temperature`` and ``seed`` are
    applied by ``Engine.generate`` through ``lss_set_sampling``)."""
    pol = N.lss_policy()
    mode = policy.get("mode", "ar")
    pol.mode = {"ar": N.LSS_MODE_AR, "static": N.LSS_MODE_STATIC, "dp": N.LSS_MODE_DP,
                "cascade": N.LSS_MODE_CASCADE}[mode]
    pol.k_max = int(policy.get("k_max", 0))
    pol.exit_tau = float(policy.get("exit_tau", 0.0))
    pol.quant = int(policy.get("quant", 0))
    if mode == "static":
        mask = np.zeros(n_layers, np.uint8)
        for l in policy["skip"]:
            mask[l] = 1
        pol._mask_keepalive = mask
        pol.static_mask = mask.ctypes.data_as(C.POINTER(C.c_uint8))
    pol.n_skip = int(policy.get("n_skip", 0))
    pol.interval = int(policy.get("interval", 1))
    levels = policy.get("levels", [])
    pol.n_levels = len(levels)
    for i, (skip, exit_, quant) in enumerate(levels):
        pol.level_skip[i] = int(skip)
        pol.level_exit[i] = int(exit_)
        pol.level_quant[i] = int(quant)
    beta = policy.get("beta", (0.0, 0.0, 0.0))
    for i in range(3):
        pol.beta[i] = float(beta[i])
    pol.tree_width = int(policy.get("tree_width", 0))
    pol.tree_depth = int(policy.get("tree_depth", 1))
    rc = policy.get("row_cost")
    if rc is not None:
        for i, v in enumerate(rc):
            pol.row_cost[i] = float(v)
    stop = list(policy.get("stop", ()))
    if len(stop) > N.LSS_STOP_MAX:
        raise ValueError(f"at most {N.LSS_STOP_MAX} stop tokens")
    pol.n_stop = len(stop)
    for i, t in enumerate(stop):
        pol.stop_tokens[i] = int(t)
    return pol


# ------------------------------------------------------------------ host-only entry points
def router_plan(accept_rate, t_hat, t_verify, k_max):
    lib = N.load()
    nl = len(accept_rate)
    a = (C.c_double * nl)(*accept_rate)
    t = (C.c_double * nl)(*t_hat)
    out = (C.c_int32 * nl)()
    rc = lib.lss_router_plan(a, t, nl, float(t_verify), int(k_max), out)
    if rc != 0:
        raise LssError("lss_router_plan", rc)
    return list(out)


def router_update(accept_rate, slot_levels, n_accepted):
    lib = N.load()
    nl = len(accept_rate)
    a = (C.c_double * nl)(*accept_rate)
    lv = (C.c_int32 * max(1, len(slot_levels)))(*slot_levels)
    rc = lib.lss_router_update(a, nl, lv, len(slot_levels), int(n_accepted))
    if rc != 0:
        raise LssError("lss_router_update", rc)
    return list(a)


def router_plan_tree(accept_rate, t_hat, t_verify, row_cost, k_max, b_max, nodes_max=N.LSS_TREE_NODES_MAX):
    """(width, draft length per level) of the next tree round
    (``lss_router_plan_tree``); row_cost None: 1 for every row count."""
    lib = N.load()
    nl = len(accept_rate)
    a = (C.c_double * nl)(*accept_rate)
    t = (C.c_double * nl)(*t_hat)
    rcp = None if row_cost is None else (C.c_double * (N.LSS_TREE_NODES_MAX + 1))(*row_cost)
    out = (C.c_int32 * nl)()
    width = C.c_int32()
    rc = lib.lss_router_plan_tree(a, t, nl, float(t_verify), rcp, int(k_max), int(b_max), int(nodes_max),
                                  C.byref(width), out)
    if rc != 0:
        raise LssError("lss_router_plan_tree", rc)
    return int(width.value), list(out)


def router_update_tree(accept_rate, depth_levels, n_accepted, branch):
    lib = N.load()
    nl = len(accept_rate)
    a = (C.c_double * nl)(*accept_rate)
    lv = (C.c_int32 * max(1, len(depth_levels)))(*depth_levels)
    rc = lib.lss_router_update_tree(a, nl, lv, len(depth_levels), int(n_accepted), int(branch))
    if rc != 0:
        raise LssError("lss_router_update_tree", rc)
    return list(a)


def latency_fit(samples):
    lib = N.load()
    flat = [float(v) for s in samples for v in s]
    arr = (C.c_double * len(flat))(*flat)
    beta = (C.c_double * 3)()
    rc = lib.lss_latency_fit(arr, len(samples), beta)
    if rc != 0:
        raise LssError("lss_latency_fit", rc)
    return tuple(beta)


def w8_quantize(w):
    """int8 codes and row scales of a CUDA weight matrix (float32 or bf16)."""
    import torch
    lib = N.load()
    w = w.contiguous()
    rows, k = w.shape
    dt = {torch.float32: N.LSS_F32, torch.bfloat16: N.LSS_BF16}[w.dtype]
    q = torch.empty((rows, k), dtype=torch.int8, device=w.device)
    s = torch.empty((rows,), dtype=torch.float32, device=w.device)
    rc = lib.lss_op_w8_quantize(C.c_void_p(w.data_ptr()), dt, rows, k, C.c_void_p(q.data_ptr()),
                                C.c_void_p(s.data_ptr()), C.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise LssError("lss_op_w8_quantize", rc)
    return q, s


def w8a8_gemv(wq, wscale, xq, xscale):
    """y = fl32(fl32(wq @ xq) * fl32(wscale * xscale)) for CUDA int8 tensors
    wq [n][k], xq [k] and float32 wscale [n], xscale [1]."""
    import torch
    lib = N.load()
    wq, wscale, xq, xscale = (t.contiguous() for t in (wq, wscale, xq, xscale))
    n, k = wq.shape
    y = torch.empty((n,), dtype=torch.float32, device=wq.device)
    rc = lib.lss_op_w8a8_gemv(C.c_void_p(wq.data_ptr()), C.c_void_p(wscale.data_ptr()), n, k,
                              C.c_void_p(xq.data_ptr()), C.c_void_p(xscale.data_ptr()), C.c_void_p(y.data_ptr()),
                              C.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise LssError("lss_op_w8a8_gemv", rc)
    return y


def w8a8_gemv_f32(wq, wscale, x):
    """The W8A8 projection of a float32 CUDA row x [k] (quantized in the
    kernel) against int8 wq [n][k] with row scales wscale [n]."""
    import torch
    lib = N.load()
    wq, wscale, x = (t.contiguous() for t in (wq, wscale, x))
    n, k = wq.shape
    y = torch.empty((n,), dtype=torch.float32, device=wq.device)
    rc = lib.lss_op_w8a8_gemv_f32(C.c_void_p(wq.data_ptr()), C.c_void_p(wscale.data_ptr()), n, k,
                                  C.c_void_p(x.data_ptr()), C.c_void_p(y.data_ptr()),
                                  C.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise LssError("lss_op_w8a8_gemv_f32", rc)
    return y


def quantize_rows(x):
    """int8 codes and per-row scales of a CUDA float32 tensor [rows][n]."""
    import torch
    lib = N.load()
    x = x.contiguous()
    rows, n = x.shape
    q = torch.empty((rows, n), dtype=torch.int8, device=x.device)
    s = torch.empty((rows,), dtype=torch.float32, device=x.device)
    rc = lib.lss_op_quantize_rows(C.c_void_p(x.data_ptr()), rows, n, C.c_void_p(q.data_ptr()),
                                  C.c_void_p(s.data_ptr()), C.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise LssError("lss_op_quantize_rows", rc)
    return q, s


def _op_error(what, rc):
    msg = N.load().lss_last_error(None)
    return LssError(what, rc, msg.decode() if msg else "")


def accept_greedy(logits, drafts, noalloc=False):
    """Greedy acceptance on CUDA logits [rows][vocab] (float32) and drafts
    [rows - 1] (int32): returns the device result [2 + rows] = {n, bonus,
    argmax of every row}.  ``noalloc`` runs the allocation-free entry point
    (library-owned scratch); otherwise a workspace tensor is allocated here."""
    import torch
    lib = N.load()
    logits = logits.contiguous()
    rows, vocab = logits.shape
    drafts = drafts.to(torch.int32).contiguous() if drafts is not None and len(drafts) else None
    res = torch.empty((2 + rows,), dtype=torch.int32, device=logits.device)
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    dp = C.c_void_p(drafts.data_ptr()) if drafts is not None else None
    if noalloc:
        rc = lib.lss_op_accept_greedy_noalloc(C.c_void_p(logits.data_ptr()), rows, vocab, dp,
                                              C.c_void_p(res.data_ptr()), stream)
        if rc != 0:
            raise _op_error("lss_op_accept_greedy_noalloc", rc)
    else:
        nb = int(lib.lss_op_accept_greedy_workspace_bytes(rows, vocab))
        if nb == 0:
            raise LssError("lss_op_accept_greedy_workspace_bytes", N.LSS_EINVAL, "bad sizes")
        ws = torch.empty((nb,), dtype=torch.uint8, device=logits.device)
        rc = lib.lss_op_accept_greedy(C.c_void_p(logits.data_ptr()), rows, vocab, dp, C.c_void_p(res.data_ptr()),
                                      C.c_void_p(ws.data_ptr()), nb, stream)
        if rc != 0:
            raise _op_error("lss_op_accept_greedy", rc)
    return res
