"""Oracle of distribution-preserving speculative sampling -- TEST INFRASTRUCTURE ONLY.

Used only by ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg; the engine shares no code with it.

What it follows:
  * The pages call the method lossless and say the draft/verify scheme keeps
    the full model's output distribution (CAS blog, section 1; CAS abs,
    abstract; CLaSp article, section 四 results), and that verification
    predicts a probability distribution for every draft token and checks the
    drafts against it (CLaSp article, section 三, verification stage).  They
    print no sampling rule.  Reading: the standard speculative-sampling rule
    that preserves the target distribution exactly -- accept draft d with
    probability min(1, p(d) / q(d)); at the first rejection draw the
    replacement from the normalised positive part of p - q; if every draft
    is accepted draw the bonus token from the full model's last row.
  * Temperature T > 0: p = softmax(z_full / T), q = softmax(z_draft / T).
    T = 0 is greedy decoding (``oracle.decode``).
  * Random numbers come from one counter-based generator, Philox-4x64 with
    10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
    easy as 1, 2, 3", SC 2011).  Every draw is a pure function of
    (seed, purpose, position, index), so a run is reproducible and the GPU
    engine draws the same numbers:
        key     = (seed, purpose)
        counter = (j, position, 0, 0)     block j gives entries 4j .. 4j+3
        u       = ((x >> 41) + 1/2) / 2**23      23-bit uniform in (0, 1), exact
                                                 in float32 as well
    Purposes: DRAFT (the draft's sample at a draft row), TARGET (the full
    model's sample: prefill token, sampled AR step, bonus token), ACCEPT
    (the uniform of the acceptance test of the draft a row checks), RESIDUAL
    (the replacement after a rejection).  "position" is always the position
    of the row whose output distribution is sampled or tested.
  * Categorical draws use the Gumbel-max identity: argmax_v(log w_v + G_v)
    with G_v = -log(-log u_v) is distributed as w / sum(w).  Ties go to the
    lowest index.

Each committed position draws its DRAFT noise possibly several times (a
re-draft after an earlier rejection) but its ACCEPT, RESIDUAL and TARGET
noise at most once; no committed outcome depends on the DRAFT noise of a
position past the first rejection, so the reuse keeps every draw fresh given
the history, and the emitted sequence has the full model's distribution.

Floating point: float64.  The GPU engine takes the same decisions in
float32 from its own logits; parity tests compare decisions whose margin
exceeds the logits' tolerance.

Pins (tests/test_oracle_sampling.py): Philox against numpy's Philox bit
generator; the Gumbel-max frequencies against softmax (chi-square); the
acceptance probability against its closed form sum_v min(p_v, q_v); the
first emitted token's frequencies against p (chi-square); q = p accepts
everything; a vanishing temperature reduces to greedy.
"""
import numpy as np

DRAFT, TARGET, ACCEPT, RESIDUAL = 1, 2, 3, 4

_M0 = np.uint64(0xD2E7470EE14C6C93)
_M1 = np.uint64(0xCA5A826395121157)
_W0 = np.uint64(0x9E3779B97F4A7C15)
_W1 = np.uint64(0xBB67AE8584CAA73B)
_LO32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo(a, b):
    """(high, low) 64-bit halves of the 128-bit product of uint64 arrays."""
    a0, a1 = a & _LO32, a >> _S32
    b0, b1 = b & _LO32, b >> _S32
    p00, p01, p10, p11 = a0 * b0, a0 * b1, a1 * b0, a1 * b1
    mid = (p00 >> _S32) + (p01 & _LO32) + (p10 & _LO32)
    hi = p11 + (p01 >> _S32) + (p10 >> _S32) + (mid >> _S32)
    lo = a * b
    return hi, lo


def philox4x64_int(ctr, key, rounds=10):
    """Philox-4x64 of one counter (4 Python ints) under a 2-word key.

    One round: (hi0, lo0) = M0 * c0 and (hi1, lo1) = M1 * c2 as 128-bit
    products; the new counter is (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0).
    The key gains the Weyl constants (W0, W1) between rounds.
    """
    mask = (1 << 64) - 1
    c0, c1, c2, c3 = (int(x) & mask for x in ctr)
    k0, k1 = int(key[0]) & mask, int(key[1]) & mask
    for r in range(rounds):
        if r > 0:
            k0, k1 = (k0 + int(_W0)) & mask, (k1 + int(_W1)) & mask
        p0, p1 = int(_M0) * c0, int(_M1) * c2
        c0, c1, c2, c3 = (p1 >> 64) ^ c1 ^ k0, p1 & mask, (p0 >> 64) ^ c3 ^ k1, p0 & mask
    return [c0, c1, c2, c3]


def philox4x64(ctr, key, rounds=10):
    """Philox-4x64 (the rounds of ``philox4x64_int``) of counters ``ctr``
    [..., 4], vectorised over uint64 arrays."""
    c = np.array(ctr, dtype=np.uint64)
    c0, c1, c2, c3 = c[..., 0].copy(), c[..., 1].copy(), c[..., 2].copy(), c[..., 3].copy()
    k0, k1 = np.uint64(key[0]), np.uint64(key[1])
    with np.errstate(over="ignore"):
        for r in range(rounds):
            if r > 0:
                k0, k1 = k0 + _W0, k1 + _W1
            hi0, lo0 = _mulhilo(np.full_like(c0, _M0), c0)
            hi1, lo1 = _mulhilo(np.full_like(c2, _M1), c2)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1)


def uniforms(seed, purpose, pos, n):
    """Entries 0 .. n-1 of the uniform stream (seed, purpose, position)."""
    nb = (n + 3) // 4
    if nb <= 4:                      # short streams: plain integers
        words = [w for j in range(nb) for w in philox4x64_int((j, pos, 0, 0), (seed, purpose))][:n]
        return (np.array([w >> 41 for w in words], np.float64) + 0.5) / float(1 << 23)
    ctr = np.zeros((nb, 4), np.uint64)
    ctr[:, 0] = np.arange(nb, dtype=np.uint64)
    ctr[:, 1] = np.uint64(pos)
    x = philox4x64(ctr, (np.uint64(seed), np.uint64(purpose))).reshape(-1)[:n]
    return ((x >> np.uint64(41)).astype(np.float64) + 0.5) / float(1 << 23)


def gumbel(seed, purpose, pos, n):
    """G_v = -log(-log u_v) for the first n entries of a stream."""
    return -np.log(-np.log(uniforms(seed, purpose, pos, n)))


def softmax(z, T):
    """softmax(z / T) in float64."""
    s = np.asarray(z, np.float64) / T
    s = s - np.max(s)
    e = np.exp(s)
    return e / np.sum(e)


def sample(z, T, seed, purpose, pos):
    """A draw from softmax(z / T): argmax of z / T plus Gumbel noise.

    Returns (token, margin): margin is the gap between the best and the
    second-best perturbed value, the slack of the decision.
    """
    v = np.asarray(z, np.float64) / T + gumbel(seed, purpose, pos, len(z))
    t = int(np.argmax(v))
    second = np.max(np.delete(v, t)) if len(v) > 1 else -np.inf
    return t, float(v[t] - second)


def top1_prob(z, T):
    """Largest probability of softmax(z / T) (the draft exit test)."""
    return float(np.max(softmax(z, T)))


def residual_sample(zp, zq, T, seed, pos):
    """Replacement token after a rejection: a draw from max(0, p - q)
    (normalised), with the RESIDUAL stream of the row's position.

    If rounding leaves no positive entry the draw comes from p with the same
    noise (p = q exactly accepts every draft, so this never decides an exact
    computation).  Returns (token, margin).
    """
    p, q = softmax(zp, T), softmax(zq, T)
    w = np.maximum(p - q, 0.0)
    g = gumbel(seed, RESIDUAL, pos, len(w))
    if np.any(w > 0):
        with np.errstate(divide="ignore"):
            v = np.log(w) + g
    else:
        v = np.asarray(zp, np.float64) / T + g
    t = int(np.argmax(v))
    rest = np.delete(v, t)
    second = np.max(rest) if rest.size else -np.inf
    return t, float(v[t] - second)


def accept_sampling(zp, zq, drafts, T, seed, pos0):
    """Speculative-sampling acceptance of one verify round.

    zp: full-model logits of the verify rows [k+1][V] (row i at position
    pos0 + i); zq: draft logits [k][V] (row i produced drafts[i] at position
    pos0 + i).  Draft i is accepted iff r_i * q_i(d) < p_i(d) with
    r_i = U(ACCEPT, pos0 + i); the first rejection at i emits a residual
    draw and ends the round; with all k accepted the bonus is a TARGET draw
    from row k.  Returns (n accepted, replacement/bonus token, margins):
    margins holds, per decision taken, the relative slack of the acceptance
    test or the gap of the final draw.
    """
    k = len(drafts)
    margins = []
    for i in range(k):
        p = softmax(zp[i], T)
        q = softmax(zq[i], T)
        d = int(drafts[i])
        r = uniforms(seed, ACCEPT, pos0 + i, 1)[0]
        lhs, rhs = r * q[d], p[d]
        margins.append(abs(lhs - rhs) / max(rhs, 1e-300))
        if not lhs < rhs:
            t, m = residual_sample(zp[i], zq[i], T, seed, pos0 + i)
            margins.append(m)
            return i, t, margins
    t, m = sample(zp[k], T, seed, TARGET, pos0 + k)
    margins.append(m)
    return k, t, margins
