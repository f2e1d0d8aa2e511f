"""Oracle draft -> verify -> accept loop, greedy autoregressive decoding.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What it follows:
  * CLaSp article, section 三 (three stages): the draft runs the model with
    some intermediate layers skipped and produces candidate tokens; the full
    model checks all of them in one forward pass; at the first rejected draft
    token the full model's own prediction replaces it and drafting restarts
    from there.  Section 一: autoregressive decoding emits one token per full
    forward (the baseline).
  * CAS-Spec blog, section 2.1: layer sparsity and early exit (an early exit
    after layer e is the same as skipping layers e..L-1), 8-bit dynamic
    activation quantization; section 2.2: several draft levels in one window.
  * CLaSp article, section 四: a draft exit threshold (readings below).

Readings where the pages are silent (each listed in the design doc):
  * greedy decoding, argmax ties to the lowest index;
  * a skipped layer is the identity on the residual stream and writes no KV;
  * draft rows attend to the committed prefix plus those window positions
    whose KV this layer wrote during drafting (per-layer valid bits);
  * verify rows are [t0, d1..dk] at positions p..p+k, row i predicts d_{i+1},
    row k yields the bonus token; verify overwrites the window's KV;
  * the exit threshold compares the draft's top-1 softmax probability with
    tau; the low-confidence token is kept, then drafting stops;
  * the quantized draft quantizes the inputs of all seven projections of an
    executed layer (q/k/v share one input), never the LM head.

Every decode row goes through ``forward_row`` one row at a time, so verify
row i and the autoregressive step at the same position are the same
computation; only the prompt prefill runs as a block.

Pins (tests/test_oracle_decode.py): greedy prefix property, incremental
decode equal to full recompute, speculative output equal to greedy output
for every policy, accepted length in [0, k], forced wrong drafts, empty-mask
drafts accepted in full, all-skipped draft closed form.
"""
from dataclasses import dataclass, field

import numpy as np

from .model import rms_norm, rope, silu, attend, fake_quant, argmax_first, w8a8_project
from . import sampling as smp

WINDOW_MAX = 32


class DecodeState:
    """KV cache and committed length of one sequence."""

    def __init__(self, model, max_seq):
        L, Hkv, hd = model.L, model.Hkv, model.hd
        self.max_seq = max_seq
        self.k = np.zeros((L, max_seq, Hkv, hd), model.dt)
        self.v = np.zeros((L, max_seq, Hkv, hd), model.dt)
        self.p = 0                 # committed length (KV rows [0, p) are final)
        self.t0 = None             # pending token, input of the row at position p
        self.window = []           # drafted tokens d1..dk (positions p+1..p+k as inputs)
        self.valid = [0] * L       # per layer: bit j set = KV at p+j written by a draft
        self.target_states = None  # full states H*[0..L] of the last accepted token
        self.target_pos = None     # its position t*
        self.window_logits = []    # sampling: draft logits that produced each window token
        self.tree = False          # (B, D) while the window holds a token tree (draft_tree)
        self.margins = []          # sampling: slack of every random decision taken


def _project(W, x):
    return W @ x


def layer_row(model, l, h, pos, st, mode, quant=False):
    """One decoder layer on one residual row ``h`` at position ``pos``.

    mode "full":  writes its k, v at ``pos``; attends to cache rows [0, pos].
    mode "draft": writes its k, v at ``pos`` (a window slot) and sets the
                  layer's valid bit; attends to [0, p) plus valid window slots.
    mode "dp":    writes nothing; attends to [0, pos) plus its own k, v.
    With a bf16 KV cache (``model.kv``) the stored keys and values are
    rounded, and so are the row's own in modes "full" and "draft"; the own
    k, v of a "dp" row enter unrounded, since they are never stored.

    quant: 0 full precision; 1 (or True) int8 activations (codes times
    scale) into the full-precision weights; 2 int8 activations and the
    layer's int8 weight copy (``w8a8_project``).  The same four points are
    quantized either way: the attention input (shared by q/k/v), the
    attention output, the FFN input (shared by gate/up) and the SwiGLU output.
    """
    m = model
    lw = m.layer(l)
    dt = m.dt
    w8 = m.layer_w8(l) if quant == 2 else None

    def proj(name, x):
        if w8 is not None:
            return w8a8_project(*w8[name], x).astype(dt)
        return _project(lw[name], x)

    def qz(x):
        return fake_quant(x, dt) if quant == 1 else x

    x = qz(rms_norm(h, lw["attn_norm"], m.eps))
    q = proj("wq", x).reshape(m.Hq, m.hd)
    k = proj("wk", x).reshape(m.Hkv, m.hd)
    v = proj("wv", x).reshape(m.Hkv, m.hd)
    q = rope(q, pos, m.theta)
    k = rope(k, pos, m.theta)
    if mode in ("full", "draft"):       # the cache's values, used by the row itself too
        k, v = m.kv(k), m.kv(v)
    if mode == "full":
        st.k[l, pos], st.v[l, pos] = k, v
        keys, vals = st.k[l, :pos + 1], st.v[l, :pos + 1]
    elif mode == "draft":
        st.k[l, pos], st.v[l, pos] = k, v
        slot = pos - st.p
        assert 0 <= slot < WINDOW_MAX
        st.valid[l] |= 1 << slot
        idx = list(range(st.p)) + [st.p + j for j in range(WINDOW_MAX) if (st.valid[l] >> j) & 1]
        keys, vals = st.k[l, idx], st.v[l, idx]
    elif mode == "dp":
        keys = np.concatenate([st.k[l, :pos], k[None]], axis=0)
        vals = np.concatenate([st.v[l, :pos], v[None]], axis=0)
    else:
        raise ValueError(mode)
    group = m.Hq // m.Hkv
    o = np.concatenate([attend(q[hh], keys[:, hh // group], vals[:, hh // group])
                        for hh in range(m.Hq)])
    h = h + proj("wo", qz(o))
    x = qz(rms_norm(h, lw["ffn_norm"], m.eps))
    a = silu(proj("w_gate", x)) * proj("w_up", x)
    return h + proj("w_down", qz(a))


def forward_row(model, st, tok, pos, mode, skip=None, quant=False):
    """Embed ``tok`` and run every layer not in ``skip``; returns (logits, states).

    ``states[0]`` is the embedding, ``states[l+1]`` the residual after layer l
    (a skipped layer repeats its input).
    """
    h = model.embed_row(tok)
    states = [h]
    for l in range(model.L):
        if skip is None or not skip[l]:
            h = layer_row(model, l, h, pos, st, mode, quant)
        states.append(h)
    return model.head(h), states


def layer_block(model, l, H, st=None):
    """Decoder layer l over a block of causal rows at positions 0..P-1
    (residual rows H [P][d], every row seeing itself and the rows before it):
    RMSNorm, q/k/v, rotary embedding, softmax attention, output projection
    and residual, RMSNorm, SwiGLU FFN and residual (CLaSp article, LLaMA
    family; shapes from the model).  Writes the block's keys and values into
    ``st`` when given.  Returns the layer's output rows."""
    m = model
    P = H.shape[0]
    pos = np.arange(P)
    group = m.Hq // m.Hkv
    causal = pos[None, :] <= pos[:, None]
    lw = m.layer(l)
    X = np.stack([rms_norm(h, lw["attn_norm"], m.eps) for h in H])
    Q = (X @ lw["wq"].T).reshape(P, m.Hq, m.hd)
    K = (X @ lw["wk"].T).reshape(P, m.Hkv, m.hd)
    Vv = (X @ lw["wv"].T).reshape(P, m.Hkv, m.hd)
    Q = np.stack([rope(Q[t], t, m.theta) for t in range(P)])
    K = np.stack([rope(K[t], t, m.theta) for t in range(P)])
    K, Vv = m.kv(K), m.kv(Vv)           # the cache's values, used by the block's own rows too
    if st is not None:
        st.k[l, :P], st.v[l, :P] = K, Vv
    O = np.empty((P, m.Hq, m.hd), m.dt)
    for hh in range(m.Hq):
        kh = hh // group
        S = (Q[:, hh] @ K[:, kh].T) / m.dt.type(np.sqrt(m.hd))
        S = np.where(causal, S, -np.inf)
        S = S - S.max(axis=1, keepdims=True)
        Pm = np.exp(S)
        Pm = Pm / Pm.sum(axis=1, keepdims=True)
        O[:, hh] = Pm @ Vv[:, kh]
    H = H + O.reshape(P, -1) @ lw["wo"].T
    X = np.stack([rms_norm(h, lw["ffn_norm"], m.eps) for h in H])
    A = silu(X @ lw["w_gate"].T) * (X @ lw["w_up"].T)
    return H + A @ lw["w_down"].T


def _pick(st, z, sampling, purpose, pos):
    """Greedy argmax (sampling None) or a draw from softmax(z / T) with the
    (seed, purpose, pos) stream of ``oracle.sampling``."""
    if sampling is None:
        return argmax_first(z)
    T, seed = sampling
    t, m = smp.sample(z, T, seed, purpose, pos)
    st.margins.append(m)
    return t


def prefill(model, tokens, max_seq, progress=None, sampling=None):
    """Causal full-model pass over the prompt, as one block of rows.

    Returns (state, logits of the last row, states of the last row).  The
    pending token t0 is the argmax of the last row (with ``sampling`` =
    (T, seed): its TARGET draw at position P-1); the last prompt row is the
    first layer-selection target (its own KV stays committed at P-1).
    """
    m = model
    tokens = np.asarray(tokens)
    P = len(tokens)
    assert 1 <= P <= max_seq
    st = DecodeState(m, max_seq)
    H = np.stack([m.embed_row(t) for t in tokens])
    last_states = [H[-1].copy()]
    for l in range(m.L):
        H = layer_block(m, l, H, st)
        last_states.append(H[-1].copy())
        if progress is not None:
            progress(l)
    z = m.head(H[-1])
    st.p = P
    st.t0 = _pick(st, z, sampling, smp.TARGET, P - 1)
    st.target_states = last_states
    st.target_pos = P - 1
    return st, z, last_states


def draft(model, st, skip, quant, k, tau=0.0, sampling=None):
    """Draft up to ``k`` tokens into the window with a skip mask.

    Returns (tokens drafted by this call, top-1 probabilities).  Appends to
    any tokens already in the window (several draft levels may share one
    window).  With ``tau > 0`` drafting stops after the first token whose
    top-1 softmax probability is below ``tau``.  With ``sampling`` =
    (T, seed) each token is the DRAFT draw of its row's position, the top-1
    probability is taken at temperature T, and the logits are kept for the
    acceptance test.
    """
    out, pmax = [], []
    for _ in range(k):
        if len(st.window) >= WINDOW_MAX - 1:
            break
        tok = st.t0 if not st.window else st.window[-1]
        pos = st.p + len(st.window)
        z, _ = forward_row(model, st, tok, pos, "draft", skip, quant)
        d = _pick(st, z, sampling, smp.DRAFT, pos)
        st.window.append(d)
        st.window_logits.append(z)
        out.append(d)
        if sampling is None:
            zs = z - np.max(z)
            pm = 1.0 / float(np.sum(np.exp(zs)))
        else:
            pm = smp.top1_prob(z, sampling[0])
        pmax.append(pm)
        if tau > 0 and pm < tau:
            break
    return out, pmax


def verify(model, st, drafts=None):
    """Full model over rows [t0, d1..dk] at positions p..p+k, row by row.

    ``drafts`` overrides the window (a host-forced draft).  Returns (logits
    [k+1][V], states [k+1][L+1][d], the draft tokens verified).
    """
    d = list(st.window if drafts is None else drafts)
    rows = [st.t0] + d
    logits, states = [], []
    for i, tok in enumerate(rows):
        z, s = forward_row(model, st, tok, st.p + i, "full")
        logits.append(z)
        states.append(s)
    return np.stack(logits), states, d


def accept(st, logits, states, drafts, sampling=None):
    """Greedy acceptance and rollback.

    a_i = argmax of verify row i; n = length of the longest prefix of the
    drafts that equals a_0..a_{n-1}; bonus = a_n.  With ``sampling`` =
    (T, seed) the speculative-sampling rule of ``oracle.sampling`` decides n
    and the bonus (the replacement draw at a rejection).  The committed
    length moves to p + n + 1 (rows past it are stale and never read); the
    window is cleared; row n becomes the next layer-selection target.
    Returns (n, bonus, emitted tokens d_1..d_n + [bonus]).
    """
    k = len(drafts)
    if sampling is None:
        a = [argmax_first(z) for z in logits]
        n = 0
        while n < k and a[n] == drafts[n]:
            n += 1
        bonus = a[n]
    else:
        if k and len(st.window_logits) != k:
            raise ValueError("sampling acceptance needs the draft logits of every window token")
        T, seed = sampling
        n, bonus, mg = smp.accept_sampling(logits, st.window_logits, drafts, T, seed, st.p)
        st.margins.extend(mg)
    emitted = list(drafts[:n]) + [bonus]
    st.target_states = states[n]
    st.target_pos = st.p + n
    st.p = st.p + n + 1
    st.t0 = bonus
    st.window = []
    st.window_logits = []
    st.valid = [0] * len(st.valid)
    return n, bonus, emitted


def top_b(z, B):
    """Indices of the B largest logits, largest first; equal logits keep the
    lowest index first (so top_b(z, 1) == [argmax_first(z)])."""
    z = np.asarray(z, np.float64)
    order = np.lexsort((np.arange(len(z)), -z))
    return [int(i) for i in order[:B]]


def draft_tree(model, st, skip, quant, B, D=1, levels=None):
    """Token tree of width B and depth D, drafted by the skipped-layer model.

    The draft runs the pending token's row (position p) and proposes its B
    most likely tokens for position p + 1 (the first nodes of B branches);
    the draft then extends every branch greedily by D - 1 more tokens, the
    row of node j of a branch (position p + j) seeing the committed prefix,
    the pending token and that branch's earlier nodes only.  Returns (the
    branches [B][D], the draft's top-1 probability at the pending row); the
    window holds the branches one after the other.

    levels: None (every depth drafted with ``skip``, ``quant``) or D pairs
    (skip, quant): the draft level whose pass proposes the nodes of depth j
    is levels[j - 1] (the pending token's row for j = 1, the rows of the
    depth j - 1 nodes otherwise), a cascade routed into the tree.  A layer
    sees the pending token and a branch's earlier nodes only where the
    level of the pass over them ran that layer (the per-layer valid bits of
    a chain window, by depth)."""
    lv = [(skip, quant)] * D if levels is None else list(levels)
    assert len(lv) == D
    z, _ = forward_row(model, st, st.t0, st.p, "draft", lv[0][0], lv[0][1])
    firsts = top_b(z, B)
    root_valid = list(st.valid)                      # window slot 0: the pending token
    branches = []
    for c in firsts:
        st.valid = list(root_valid)                  # another branch's nodes are invisible
        br = [c]
        for j in range(1, D):
            zz, _ = forward_row(model, st, br[-1], st.p + j, "draft", lv[j][0], lv[j][1])
            br.append(argmax_first(zz))
        branches.append(br)
    st.valid = list(root_valid)
    st.window = [t for br in branches for t in br]
    st.tree = (B, D)
    zs = z - np.max(z)
    return branches, 1.0 / float(np.sum(np.exp(zs)))


def verify_tree(model, st):
    """Tree verify in one pass over rows [pending token, branch 1 nodes 1..D,
    branch 2 nodes, ...]: row 0 is the pending token at position p; the row
    of node j of branch b is at position p + j and sees the committed
    prefix, the pending token and nodes 1..j of its own branch (a tree
    mask), so it is the full model's step at p + j after that branch's
    first j tokens.  Returns (logits [1 + B D][V], states, branches, the
    keys/values each branch's nodes give positions p + 1 .. p + D)."""
    B, D = st.tree
    branches = [list(st.window[b * D:(b + 1) * D]) for b in range(B)]
    z0, s0 = forward_row(model, st, st.t0, st.p, "full")
    logits, states, kv = [z0], [s0], []
    for br in branches:
        bkv = []
        for j, c in enumerate(br, start=1):
            z, s = forward_row(model, st, c, st.p + j, "full")    # writes and sees its branch's positions
            logits.append(z)
            states.append(s)
            bkv.append((st.k[:, st.p + j].copy(), st.v[:, st.p + j].copy()))
        kv.append(bkv)
    return np.stack(logits), states, branches, kv


def accept_tree(st, logits, states, branches, kv):
    """Greedy acceptance of a tree: a_0 = argmax of row 0; the branch whose
    first node equals a_0 (at most one: the first nodes are distinct) is
    followed while its next node equals the full model's token after the
    last accepted one; n = accepted nodes, bonus = the full model's token
    after them, and their keys/values become positions p + 1 .. p + n.
    With no such branch n = 0 and the bonus is a_0.  Returns (n, bonus,
    emitted tokens)."""
    B, D = st.tree
    a0 = argmax_first(logits[0])
    hit = [b for b, br in enumerate(branches) if br[0] == a0]
    if hit:
        b = hit[0]
        n, row = 1, 1 + b * D
        while n < D and branches[b][n] == argmax_first(logits[row]):
            n += 1
            row += 1
        bonus = argmax_first(logits[row])
        for j in range(n):
            st.k[:, st.p + 1 + j], st.v[:, st.p + 1 + j] = kv[b][j]
        emitted = list(branches[b][:n]) + [bonus]
    else:
        n, row, bonus, emitted = 0, 0, a0, [a0]
    st.target_states = states[row]
    st.target_pos = st.p + n
    st.p = st.p + n + 1
    st.t0 = bonus
    st.window = []
    st.window_logits = []
    st.tree = False
    st.valid = [0] * len(st.valid)
    return n, bonus, emitted


def _stopped(out, start, stop):
    """Stop tokens: cut ``out`` right after the first stop token among
    out[start:] (in place); True if there was one."""
    for i in range(start, len(out)):
        if out[i] in stop:
            del out[i + 1:]
            return True
    return False


def ar_generate(model, prompt, G, max_seq=None, sampling=None, state_out=None, stop=()):
    """Autoregressive decoding of G tokens (t0 included): greedy, or with
    ``sampling`` = (T, seed) the TARGET draw of every row's position.
    ``state_out`` (a list) receives the decode state (its ``margins``).
    ``stop``: token ids that end the decoding right after their first
    occurrence (kept)."""
    max_seq = max_seq or len(prompt) + G + 1
    st, z, _ = prefill(model, prompt, max_seq, sampling=sampling)
    if state_out is not None:
        state_out.append(st)
    out = [st.t0]
    if _stopped(out, 0, stop):
        return out
    while len(out) < G:
        zz, s = forward_row(model, st, st.t0, st.p, "full")
        st.target_states, st.target_pos = s, st.p
        st.t0 = _pick(st, zz, sampling, smp.TARGET, st.p)
        st.p += 1
        out.append(st.t0)
        if _stopped(out, len(out) - 1, stop):
            break
    return out


@dataclass
class Policy:
    """Draft policy of one speculative run.

    skip: static skip set (layer indices); dp_skip: number of layers the
    CLaSp DP chooses (overrides ``skip``), re-run every ``interval`` verify
    rounds; tau: draft exit threshold (0 = off); quant: 0 full precision, 1
    int8 activations, 2 int8 activations and int8 weights (``layer_row``);
    cascade: a list of levels
    ``[(n_skip_by_dp, exit_layers, quant)]`` ordered fast -> precise, routed
    by the DyTC heuristics with at most ``K`` drafts per round;
    temperature > 0: speculative sampling with that temperature and seed
    (``oracle.sampling``), 0: greedy; tree_width B > 0 (greedy, static or
    DP mask): every round drafts a token tree of width B and depth
    min(tree_depth, tokens still to emit) (``draft_tree``) instead of a
    chain; with ``cascade``, tree_width is the largest width the router may
    choose (``dytc.plan_tree``, row_cost its per-row-count cost factors,
    None: 1), its levels drafting the tree's depths.  stop: token ids that
    end the decoding right after the first one emitted (kept).
    """
    K: int = 4
    skip: tuple = ()
    dp_skip: int = None
    interval: int = 32
    tau: float = 0.0
    quant: int = 0
    cascade: list = None
    latency_beta: tuple = (1.0, 0.0, 1.0)
    forced_drafts: dict = field(default_factory=dict)
    temperature: float = 0.0
    seed: int = 0
    tree_width: int = 0
    tree_depth: int = 1
    row_cost: tuple = None
    stop: tuple = ()

    @property
    def sampling(self):
        """(T, seed) for speculative sampling, None for greedy decoding."""
        return (self.temperature, self.seed) if self.temperature > 0 else None


def _mask_from_set(L, s):
    m = [0] * L
    for l in s:
        m[l] = 1
    return m


def speculative_generate(model, prompt, G, policy, max_seq=None, log=None, state_out=None):
    """Self-speculative decoding of G tokens (t0 included): greedy, or
    speculative sampling when ``policy.temperature`` > 0.

    Returns (tokens, per-round records).  The DP (if any) runs once after the
    prefill and again after every ``interval``-th verify round.
    """
    from .clasp import clasp_dp
    from .dytc import A_INIT, plan_cascade, update_cascade, predict_latency, plan_tree, update_tree
    L = model.L
    max_seq = max_seq or len(prompt) + G + WINDOW_MAX + 1
    sam = policy.sampling
    st, _, _ = prefill(model, prompt, max_seq, sampling=sam)
    if state_out is not None:
        state_out.append(st)
    out = [st.t0]
    records = []
    if _stopped(out, 0, policy.stop):
        return out, records

    def select_masks():
        if policy.cascade is not None:
            ms = []
            for n_skip, exit_layers, _q in policy.cascade:
                le = L - exit_layers
                mask, _, _ = clasp_dp(model, st, n_skip - exit_layers, n_layers=le)
                ms.append(mask)
            return ms
        if policy.dp_skip is not None:
            return [clasp_dp(model, st, policy.dp_skip)[0]]
        return [_mask_from_set(L, policy.skip)]

    masks = select_masks()
    a = [A_INIT] * (len(policy.cascade) if policy.cascade else 0)
    rounds = 0
    while len(out) < G:
        budget = G - len(out) - 1
        if policy.cascade is not None and policy.tree_width:
            depth = [L - sum(mk) for mk in masks]
            t_hat = [predict_latency(policy.latency_beta, st.p, dp) for dp in depth]
            t_ver = predict_latency(policy.latency_beta, st.p, L)
            B, plan = plan_tree(a, t_hat, t_ver, policy.row_cost, policy.K, policy.tree_width)
            levels = []         # depth order: most precise level first
            for lev in reversed(range(len(masks))):
                levels += [lev] * plan[lev]
            levels = levels[:budget]
            if levels:
                draft_tree(model, st, None, None, B, len(levels),
                           levels=[(masks[lev], policy.cascade[lev][2]) for lev in levels])
                logits, states, branches, kv = verify_tree(model, st)
                n, bonus, emitted = accept_tree(st, logits, states, branches, kv)
                firsts = [br[0] for br in branches]
                branch = firsts.index(emitted[0]) if n else -1
            else:
                logits, states, d = verify(model, st)
                n, bonus, emitted = accept(st, logits, states, d, sam)
                branch = -1
            a = update_tree(a, levels, n, branch)
            start = len(out)
            out += emitted
            rounds += 1
            rec = {"k": B * len(levels), "n": n, "bonus": bonus, "tree": True, "width": B,
                   "levels": levels, "branch": branch, "a": list(a)}
            records.append(rec)
            if log is not None:
                log.append(rec)
            if _stopped(out, start, policy.stop):
                break
            if rounds % policy.interval == 0:
                masks = select_masks()
            continue
        if policy.cascade is not None:
            depth = [L - sum(mk) for mk in masks]
            t_hat = [predict_latency(policy.latency_beta, st.p, dp) for dp in depth]
            t_ver = predict_latency(policy.latency_beta, st.p, L)
            plan = plan_cascade(a, t_hat, t_ver, policy.K)
            steps = []          # window order: most precise level first
            for lev in reversed(range(len(masks))):
                kk = min(plan[lev], budget - sum(s[2] for s in steps))
                steps.append((lev, masks[lev], kk))
            drafted_levels = []
            for lev, mk, kk in steps:
                toks, _ = draft(model, st, mk, policy.cascade[lev][2], kk, 0.0, sam)
                drafted_levels += [lev] * len(toks)
        elif policy.tree_width and budget > 0:
            depth = min(policy.tree_depth, budget)
            draft_tree(model, st, masks[0], policy.quant, policy.tree_width, depth)
            logits, states, branches, kv = verify_tree(model, st)
            n, bonus, emitted = accept_tree(st, logits, states, branches, kv)
            start = len(out)
            out += emitted
            rounds += 1
            firsts = [br[0] for br in branches]
            rec = {"k": len(branches) * depth, "n": n, "bonus": bonus, "tree": True,
                   "branch": firsts.index(emitted[0]) if n else -1}
            records.append(rec)
            if log is not None:
                log.append(rec)
            if _stopped(out, start, policy.stop):
                break
            if policy.dp_skip is not None and rounds % policy.interval == 0:
                masks = select_masks()
            continue
        else:
            kk = min(policy.K, budget)
            if rounds in policy.forced_drafts:
                d = list(policy.forced_drafts[rounds])[:kk]
                st.window = d
            else:
                draft(model, st, masks[0], policy.quant, kk, policy.tau, sam)
            drafted_levels = None
        logits, states, d = verify(model, st)
        n, bonus, emitted = accept(st, logits, states, d, sam)
        start = len(out)
        out += emitted
        rounds += 1
        rec = {"k": len(d), "n": n, "bonus": bonus}
        if drafted_levels is not None:
            a = update_cascade(a, drafted_levels, n)
            rec["levels"] = drafted_levels
            rec["a"] = list(a)
        records.append(rec)
        if log is not None:
            log.append(rec)
        if _stopped(out, start, policy.stop):
            break
        if (policy.dp_skip is not None or policy.cascade is not None) and rounds % policy.interval == 0:
            masks = select_masks()
    return out[:G], records


def batch_generate(model, prompts, G, policy):
    """Several independent sequences decoded together (batch > 1): neither
    page batches requests, so a batch is read as a set of sequences each
    decoded exactly as on its own -- its own prompt, cache, drafts, layer
    selection (CLaSp article, section 3, per sequence) and acceptance -- and
    batching only shares the passes over the weights.  The oracle therefore
    runs ``speculative_generate`` on every prompt in turn.  Returns
    [(tokens, per-round records)] in prompt order."""
    return [speculative_generate(model, np.asarray(p), G, policy) for p in prompts]
