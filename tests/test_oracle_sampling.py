"""Pins of the oracle's speculative sampling (CPU only).

What fixes the expected values:
  * Philox-4x64-10 is checked bit for bit against numpy's own Philox bit
    generator (a library implementation of the same published function).
  * Gumbel-max: argmax(z/T + G) is distributed as softmax(z/T); checked by a
    chi-square test of draw frequencies.
  * Speculative sampling (the reading of the pages' "keeps the output
    distribution", CLaSp article section 三 and CAS abs abstract): a draft
    drawn from q is accepted with probability sum_v min(p_v, q_v) (closed
    form), and the first emitted token is distributed as p; q = p accepts
    everything; a vanishing temperature is greedy decoding.
A plausible slip (ratio q/p instead of p/q, a residual without max(0, .), a
draft and an acceptance sharing one stream, an off-by-one position) fails
at least one of these.
"""
import copy

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle import sampling as smp


@pytest.mark.parametrize("key", [(1, 2), (0, 0), (2**64 - 1, 12345), (0x0123456789ABCDEF, 7)])
@pytest.mark.parametrize("ctr", [(5, 7, 9, 11), (0, 0, 0, 0), (2**64 - 2, 3, 2**63, 1), (2**64 - 1, 0, 0, 0)])
def test_philox_matches_numpy_bit_generator(key, ctr):
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(ctr, dtype=np.uint64))
    ref = bg.random_raw(4)           # numpy advances the counter first, then generates
    nxt = list(ctr)
    nxt[0] = (nxt[0] + 1) % 2**64
    if nxt[0] == 0:                  # carry into the next word
        nxt[1] = (nxt[1] + 1) % 2**64
    got = smp.philox4x64(np.array([nxt, nxt], dtype=np.uint64), key)[1]
    assert [int(x) for x in got] == [int(x) for x in ref]
    assert smp.philox4x64_int(nxt, key) == [int(x) for x in ref]


def test_uniforms_are_23_bit_and_open():
    u = smp.uniforms(11, smp.TARGET, 5, 4000)
    codes = u * 2**23 - 0.5
    assert np.all(u.astype(np.float32).astype(np.float64) == u)   # exact in float32
    assert np.all(codes == np.round(codes))
    assert np.all((u > 0) & (u < 1))
    # streams differ by purpose and by position
    assert not np.array_equal(u[:16], smp.uniforms(11, smp.DRAFT, 5, 16))
    assert not np.array_equal(u[:16], smp.uniforms(11, smp.TARGET, 6, 16))
    # entry v of a long stream equals entry v of a short one (block layout;
    # the short one takes the plain-integer generator)
    assert np.array_equal(smp.uniforms(11, smp.TARGET, 5, 7), u[:7])
    assert np.array_equal(smp.uniforms(11, smp.TARGET, 5, 16), u[:16])
    ks = stats.kstest(u, "uniform")
    assert ks.pvalue > 1e-4


Z = np.array([1.0, 0.2, -0.5, 2.0, 0.0, -1.5, 0.7, 1.2])


def test_gumbel_max_frequencies_match_softmax():
    T, N = 0.8, 8000
    counts = np.zeros(len(Z))
    for pos in range(N):
        t, _ = smp.sample(Z, T, 3, smp.TARGET, pos)
        counts[t] += 1
    p = smp.softmax(Z, T)
    chi = stats.chisquare(counts, p * N)
    assert chi.pvalue > 1e-4, (counts, p * N)


def _toy_round(zp, zq, T, seed, pos0):
    d, _ = smp.sample(zq, T, seed, smp.DRAFT, pos0)
    n, t, _ = smp.accept_sampling(np.stack([zp, zp]), [zq], [d], T, seed, pos0)
    return d, n, t


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_speculative_sampling_preserves_the_target_distribution(T):
    zp = Z
    zq = np.array([0.2, 1.1, -0.3, 1.0, 0.9, -1.0, 0.1, 0.4])
    N = 8000
    first = np.zeros(len(Z))
    acc = 0
    for pos0 in range(N):
        d, n, t = _toy_round(zp, zq, T, 5, pos0)
        acc += n
        first[d if n == 1 else t] += 1
    p, q = smp.softmax(zp, T), smp.softmax(zq, T)
    a = float(np.sum(np.minimum(p, q)))
    sd = np.sqrt(a * (1 - a) / N)
    assert abs(acc / N - a) < 5 * sd, (acc / N, a)
    chi = stats.chisquare(first, p * N)
    assert chi.pvalue > 1e-4, (first, p * N)


def test_equal_distributions_accept_every_draft():
    for pos0 in range(500):
        d, n, t = _toy_round(Z, Z, 0.9, 2, pos0)
        assert n == 1


def test_vanishing_temperature_is_greedy():
    rng = np.random.default_rng(0)
    for pos in range(50):
        z = rng.normal(size=64)
        t, _ = smp.sample(z, 1e-6, 9, smp.DRAFT, pos)
        assert t == int(np.argmax(z))


def test_residual_draw_never_picks_a_token_with_p_below_q():
    zp = Z
    zq = np.array([3.0, 0.2, -0.5, 2.0, 0.0, -1.5, 0.7, 1.2])   # q moves mass onto token 0
    p, q = smp.softmax(zp, 1.0), smp.softmax(zq, 1.0)
    for pos in range(300):
        t, _ = smp.residual_sample(zp, zq, 1.0, 4, pos)
        assert p[t] > q[t]


# ---------------------------------------------------------------- the whole loop on the tiny model

G = 24


def test_loop_draws_each_target_accept_residual_stream_once(tiny_model, tiny_prompt, monkeypatch):
    """Over a whole speculative-sampling run, the ACCEPT, RESIDUAL and TARGET
    streams of a position are each drawn at most once (DRAFT streams may be
    redrawn after a rejection), and every decision's position is a row
    position of the run."""
    log = []
    real = smp.uniforms

    def spy(seed, purpose, pos, n):
        log.append((purpose, pos))
        return real(seed, purpose, pos, n)

    monkeypatch.setattr(smp, "uniforms", spy)
    pol = oracle.Policy(K=4, skip=(1, 2), temperature=1.0, seed=77)
    toks, recs = oracle.speculative_generate(tiny_model, tiny_prompt, G, pol)
    assert len(toks) == G
    once = [e for e in log if e[0] != smp.DRAFT]
    assert len(once) == len(set(once))
    P = len(tiny_prompt)
    assert all(P - 1 <= pos < P + G + 4 for _, pos in log)
    # one TARGET or RESIDUAL draw per round plus t0
    assert sum(1 for e in log if e[0] in (smp.TARGET, smp.RESIDUAL)) == len(recs) + 1


def test_loop_with_empty_mask_accepts_everything(tiny_model, tiny_prompt):
    pol = oracle.Policy(K=5, skip=(), temperature=0.9, seed=3)
    toks, recs = oracle.speculative_generate(tiny_model, tiny_prompt, G, pol)
    assert all(r["n"] == r["k"] for r in recs)


def test_loop_is_reproducible_and_seed_dependent(tiny_model, tiny_prompt):
    pol = oracle.Policy(K=4, skip=(2,), temperature=1.0, seed=1)
    a, _ = oracle.speculative_generate(tiny_model, tiny_prompt, G, pol)
    b, _ = oracle.speculative_generate(tiny_model, tiny_prompt, G, pol)
    c, _ = oracle.speculative_generate(tiny_model, tiny_prompt, G, oracle.Policy(K=4, skip=(2,), temperature=1.0,
                                                                               seed=2))
    assert a == b and a != c


def test_ar_sampling_at_vanishing_temperature_is_greedy(tiny_model, tiny_prompt):
    greedy = oracle.ar_generate(tiny_model, tiny_prompt, G)
    cold = oracle.ar_generate(tiny_model, tiny_prompt, G, sampling=(1e-7, 5))
    assert cold == greedy


def test_first_round_of_the_loop_matches_the_target_distribution(tiny_model, tiny_prompt):
    """Whole-loop check of the first drafted position: over many seeds, the
    token emitted after t0 is distributed as the full model's softmax at that
    position given t0.  t0 is fixed by a vanishing-temperature prefill so
    that every seed continues the same prefix; the rows then sample at T."""
    T = 1.5
    P = len(tiny_prompt)
    st0, _, _ = oracle.prefill(tiny_model, tiny_prompt, P + 8)
    zfull, _ = oracle.forward_row(tiny_model, st0, st0.t0, P, "full")
    p = smp.softmax(zfull, T)
    top = np.argsort(p)[::-1][:6]
    N = 800
    counts = np.zeros(len(top) + 1)
    for seed in range(N):
        st = copy.deepcopy(st0)
        oracle.draft(tiny_model, st, [0, 1, 1, 0], False, 1, 0.0, (T, seed))
        logits, states, d = oracle.verify(tiny_model, st)
        _, _, emitted = oracle.accept(st, logits, states, d, (T, seed))
        t = emitted[0]
        hit = np.nonzero(top == t)[0]
        counts[hit[0] if hit.size else len(top)] += 1
    exp = np.append(p[top], 1 - p[top].sum()) * N
    chi = stats.chisquare(counts, exp)
    assert chi.pvalue > 1e-4, (counts, exp)
