"""Pins for the CPU oracle: facts fixed by the pages and by the mathematics.

Each test ties the oracle to something other than itself: numbers printed in a
worked example (fixtures under tests/golden/ carry their citation), closed
forms, library routines, invariants, and brute force on tiny inputs. A
plausible slip in the oracle (a dropped max, a wrong comparison, a swapped
operand, an off-by-one in the walk) breaks at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special

from oracle import spec_oracle as O
from tests.conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _logits(p):
    p = np.asarray(p, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.log(p)


# --------------------------------------------------------------------------
# softmax with temperature: library routine, invariants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T", [0.3, 0.7, 1.0, 2.5])
def test_softmax_matches_scipy(T):
    rng = np.random.default_rng(1)
    for V in (1, 3, 16, 1000):
        x = rng.normal(0, 3, V)
        p = O.softmax_t(x, T)
        ref = scipy.special.softmax(x / T)
        assert np.allclose(p, ref, rtol=1e-13, atol=1e-300)
        assert abs(p.sum() - 1.0) < 1e-12


def test_softmax_uniform_and_masked():
    p = O.softmax_t(np.full(7, 3.25), 0.8)
    assert np.allclose(p, 1 / 7, rtol=1e-15)
    x = np.array([0.0, -np.inf, 1.0, -np.inf])
    p = O.softmax_t(x, 1.0)
    assert p[1] == 0.0 and p[3] == 0.0
    assert np.isclose(p[2] / p[0], math.e, rtol=1e-14)


def test_softmax_temperature_scales_logit_gaps():
    x = np.array([0.0, 1.0, 2.0])
    p = O.softmax_t(x, 0.5)
    # ratio of neighbouring probabilities is exp(gap / T)
    assert np.isclose(p[1] / p[0], math.exp(2.0), rtol=1e-14)
    assert np.isclose(p[2] / p[1], math.exp(2.0), rtol=1e-14)


def test_argmax_lowest_index_on_ties():
    assert O.argmax_lowest([1.0, 3.0, 3.0, 2.0]) == 1
    assert O.argmax_lowest([-0.0, 0.0]) == 0
    assert O.argmax_lowest([-np.inf, -np.inf, 5.0]) == 2


# --------------------------------------------------------------------------
# the worked examples on the pages
# --------------------------------------------------------------------------

@pytest.mark.parametrize("fixture", ["worked_example_dvc.json", "worked_example_rnr.json"])
def test_worked_example_mass_accounting(fixture):
    g = _golden(fixture)
    p, q = np.array(g["p"]), np.array(g["q"])
    a = O.acceptance_probability(p, q)
    assert np.allclose(a, g["acceptance"], atol=1e-15)
    m = O.accepted_mass(p, q)
    assert np.allclose(m, g["accepted_mass"], atol=1e-15)
    assert math.isclose(m.sum(), g["accepted_mass_total"], abs_tol=1e-15)
    r_unnorm, Z = O.positive_residual(p, q)
    if "positive_residual" in g:
        assert np.allclose(r_unnorm, g["positive_residual"], atol=1e-15)
    if "Z" in g:
        assert math.isclose(Z, g["Z"], abs_tol=1e-15)
    assert math.isclose(Z, 1.0 - g["accepted_mass_total"], abs_tol=1e-15)
    r = O.residual_distribution(p, q)
    assert np.allclose(r, g["residual"], atol=1e-15)
    assert np.allclose(m + Z * r, g["recovered"], atol=1e-15)


def test_counterexample_restart_from_p_is_wrong():
    g = _golden("worked_example_rnr.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    m = O.accepted_mass(p, q)
    _, Z = O.positive_residual(p, q)
    naive = m + Z * p
    assert np.allclose(naive, g["naive_restart_from_p"], atol=1e-15)
    assert math.isclose(abs(naive[0] - p[0]), g["naive_tv_at_first_symbol"], abs_tol=1e-15)
    # the correct rule recovers p, the naive one does not
    assert np.allclose(m + Z * O.residual_distribution(p, q), p, atol=1e-15)
    assert not np.allclose(naive, p, atol=1e-3)


def test_one_step_law_identity_random():
    rng = np.random.default_rng(7)
    for V in (2, 3, 16, 257):
        for _ in range(20):
            p = rng.dirichlet(np.full(V, 0.5))
            q = rng.dirichlet(np.full(V, 0.5))
            q[rng.random(V) < 0.2] = 0.0
            if q.sum() == 0:
                continue
            q /= q.sum()
            m = O.accepted_mass(p, q)
            r_unnorm, Z = O.positive_residual(p, q)
            assert np.allclose(m + r_unnorm, p, atol=1e-14)
            assert math.isclose(Z, 1.0 - np.minimum(p, q).sum(), abs_tol=1e-14)


def test_p_equals_q_gives_exact_zero_residual():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 2, 50)
    p = O.softmax_t(x, 0.9)
    r, Z = O.positive_residual(p, p.copy())
    assert Z == 0.0 and not r.any()
    with pytest.raises(ZeroDivisionError):
        O.residual_distribution(p, p.copy())


# --------------------------------------------------------------------------
# inverse CDF: exhaustive interval enumeration
# --------------------------------------------------------------------------

def test_inverse_cdf_intervals_exhaustive():
    rng = np.random.default_rng(11)
    for V in (1, 2, 3, 5, 16):
        for _ in range(30):
            w = rng.random(V)
            w[rng.random(V) < 0.3] = 0.0
            if not w.any():
                w[rng.integers(V)] = 0.5
            C = np.cumsum(w) / w.sum()
            lo = 0.0
            for v in range(V):
                hi = C[v]
                if w[v] > 0:
                    eps = 1e-9 if hi - lo > 2e-9 else 0.0
                    for u in (lo + eps, 0.5 * (lo + hi), hi - eps):
                        tok, dist = O.inverse_cdf(w, u)
                        assert tok == v, (w, u, tok, v)
                        assert dist >= 0.0
                lo = hi
            # u = 0 selects the first token with positive weight
            assert O.inverse_cdf(w, 0.0)[0] == int(np.flatnonzero(w > 0)[0])
            # zero-weight tokens are never drawn
            for u in np.linspace(0, 1, 101, endpoint=False):
                assert w[O.inverse_cdf(w, u)[0]] > 0


def test_inverse_cdf_rounding_clamp_picks_last_positive():
    w = np.array([0.25, 0.5, 0.25, 0.0])
    tok, _ = O.inverse_cdf(w, 1.0)   # t = total: no C_v > t
    assert tok == 2


# --------------------------------------------------------------------------
# the block walk: brute force and closed forms
# --------------------------------------------------------------------------

def _cells(breaks):
    """Midpoints and widths of the cells [0,1) is cut into by `breaks`."""
    pts = sorted({0.0, 1.0, *[min(max(b, 0.0), 1.0) for b in breaks]})
    return [(0.5 * (a + b), b - a) for a, b in zip(pts[:-1], pts[1:]) if b > a]


def test_block_walk_exact_law_bruteforce_V3_K2():
    """Enumerate drafts and uniform cells exactly; every emitted token has the
    target law of its position (marginally, given the position is reached)."""
    rng = np.random.default_rng(5)
    V, K, T = 3, 2, 1.0
    for trial in range(4):
        P = [rng.dirichlet(np.ones(V)) for _ in range(K + 1)]
        Q = [rng.dirichlet(np.ones(V)) for _ in range(K)]
        if trial == 3:
            Q[0] = np.array([0.0, 0.6, 0.4])      # zero-q token
        target = np.stack([_logits(p) for p in P])
        draft = np.stack([_logits(q) for q in Q])
        law = {}
        for d0 in range(V):
            for d1 in range(V):
                wq = Q[0][d0] * Q[1][d1]
                if wq == 0:
                    continue
                d = np.array([d0, d1])
                a = [min(1.0, P[i][d[i]] / Q[i][d[i]]) for i in range(K)]
                # cells of u0, u1 decide acceptance; u2's cells come from every
                # weight vector the final draw may use
                ws = [np.maximum(P[i] - Q[i], 0) for i in range(K)] + [P[K]]
                br = [c for w in ws for c in (np.cumsum(w) / w.sum()).tolist()]
                for u0, w0 in _cells([a[0]]):
                    for u1, w1 in _cells([a[1]]):
                        for u2, w2 in _cells(br):
                            res = O.verify_sequence(target, draft, d,
                                                    [u0, u1, u2], T, O.MODE_STOCHASTIC)
                            key = tuple(int(t) for t in res.tokens if t >= 0)
                            law[key] = law.get(key, 0.0) + wq * w0 * w1 * w2
        assert math.isclose(sum(law.values()), 1.0, abs_tol=1e-12)
        # first token: law p_0
        first = np.zeros(V)
        for k, w in law.items():
            first[k[0]] += w
        assert np.allclose(first, P[0], atol=1e-12)
        # token at position 1, given it is emitted: law p_1
        second = np.zeros(V)
        for k, w in law.items():
            if len(k) >= 2:
                second[k[1]] += w
        assert np.allclose(second / second.sum(), P[1], atol=1e-12)
        # bonus token, given all drafts kept: law p_2
        third = np.zeros(V)
        for k, w in law.items():
            if len(k) == 3:
                third[k[2]] += w
        assert np.allclose(third / third.sum(), P[2], atol=1e-12)
        # emitted count 1..K+1; the probability of emitting >= i+1 tokens is
        # the product of per-position accepted mass (independent rows here)
        alpha = [np.minimum(P[i], Q[i]).sum() for i in range(K)]
        n1 = sum(w for k, w in law.items() if len(k) >= 2)
        n2 = sum(w for k, w in law.items() if len(k) >= 3)
        assert math.isclose(n1, alpha[0], abs_tol=1e-12)
        assert math.isclose(n2, alpha[0] * alpha[1], abs_tol=1e-12)
        if trial == 3:
            # token 0 has q = 0: never kept as a draft at position 0, but still
            # emitted there with its full target probability via the residual
            assert not any(len(k) >= 2 and k[0] == 0 for k in law)
            assert math.isclose(first[0], P[0][0], abs_tol=1e-12)


def _const_alpha_batch(alpha, K, B, seed):
    """V = 2 with q = (1, 0) and p = (alpha, 1 - alpha) at every position: the
    draft is always token 0 and is kept with probability exactly alpha."""
    rng = np.random.default_rng(seed)
    t_row = _logits([alpha, 1 - alpha])
    d_row = _logits([1.0, 0.0])
    target = np.broadcast_to(t_row, (B, K + 1, 2))
    draft = np.broadcast_to(d_row, (B, K, 2))
    tokens = np.zeros((B, K), dtype=np.int64)
    u = rng.random((B, K + 1))
    return target, draft, tokens, u


def test_block_walk_constant_alpha_closed_form():
    alpha, K, B = 0.6, 4, 20000
    target, draft, tokens, u = _const_alpha_batch(alpha, K, B, 21)
    res = O.verify_batch(target, draft, tokens, u, 1.0, O.MODE_STOCHASTIC)
    E = (1 - alpha ** (K + 1)) / (1 - alpha)
    emitted = res.accept_len + 1
    se = emitted.std() / math.sqrt(B)
    assert abs(emitted.mean() - E) < 5 * se
    probs = np.array([alpha ** j * (1 - alpha) for j in range(K)] + [alpha ** K])
    exp = probs * B
    chi2 = ((res.hist - exp) ** 2 / exp).sum()
    assert chi2 < scipy.stats.chi2.ppf(0.9999, K)
    # rejection at i always corrects to token 1 (the only positive residual)
    rej = res.accept_len < K
    assert np.all(res.tokens[rej, res.accept_len[rej]] == 1)
    assert np.all(res.z[rej] > 0) and np.allclose(res.z[rej], 1 - alpha)
    # histogram invariants
    assert res.hist.sum() == B
    assert (np.arange(K + 1) * res.hist).sum() == res.accept_len.sum()


def test_closed_form_matches_printed_cost_model():
    """The pin used above, E = sum_{i=0}^{gamma} alpha^i, reproduces the
    printed cost-model sweep."""
    g = _golden("cost_model_rnr.json")

    def E(a, k):
        return sum(a ** i for i in range(k + 1))

    def best(a, c):
        vals = [(E(a, k) / (1 + c * k), k) for k in range(1, 17)]
        return max(vals)

    s, k = best(0.7, 0.05)
    assert k == g["alpha_0.7_c_0.05"]["best_gamma"]
    assert round(E(0.7, 6), 6) == g["alpha_0.7_c_0.05"]["E"]
    assert round(s, 3) == g["alpha_0.7_c_0.05"]["S"]
    s, k = best(0.7, 0.20)
    assert k == g["alpha_0.7_c_0.20"]["best_gamma"]
    assert round(s, 3) == g["alpha_0.7_c_0.20"]["S"]
    assert round(E(0.7, 6) / (3 + 0.05 * 6), 3) == g["alpha_0.7_gamma_6_c_0.05_g_3"]["ratio"]
    # geometric closed form equals the partial sum
    assert math.isclose(E(0.7, 6), (1 - 0.7 ** 7) / 0.3, rel_tol=1e-14)


# --------------------------------------------------------------------------
# Monte Carlo: the sampler recovers p; the naive correction does not
# --------------------------------------------------------------------------

def _mc_batch(p, q, N, seed):
    rng = np.random.default_rng(seed)
    V = len(p)
    d = rng.choice(V, size=N, p=q)
    u = rng.random((N, 2))
    target = np.broadcast_to(_logits(p), (N, 2, V))
    draft = np.broadcast_to(_logits(q), (N, 1, V))
    return target, draft, d.reshape(N, 1), u


def _mc_freq_ok(p, freq, N):
    se = np.sqrt(p * (1 - p) / N)
    return bool(np.all(np.abs(freq - p) <= 5 * se + 1e-12))


def _mc_cases():
    g = _golden("worked_example_dvc.json")
    rng = np.random.default_rng(16)
    p16 = rng.dirichlet(np.ones(16))
    q16 = rng.dirichlet(np.ones(16))
    q16[[2, 5, 11]] = 0.0           # zero-q subset: reachable only by the residual
    q16 /= q16.sum()
    return [("V3", np.array(g["p"]), np.array(g["q"])), ("V16", p16, q16)]


@pytest.mark.parametrize("name,p,q", _mc_cases())
def test_monte_carlo_recovers_target(name, p, q):
    N = 200_000
    target, draft, d, u = _mc_batch(p, q, N, 20260923)
    res = O.verify_batch(target, draft, d, u, 1.0, O.MODE_STOCHASTIC)
    first = res.tokens[:, 0]
    freq = np.bincount(first, minlength=len(p)) / N
    assert _mc_freq_ok(p, freq, N), (freq, p)
    # zero-q tokens never arrive as kept drafts
    zq = np.flatnonzero(q == 0)
    kept = res.accept_len == 1
    assert not np.isin(first[kept], zq).any()
    if len(zq):
        assert np.isin(first, zq).any()


def test_monte_carlo_detects_naive_correction(monkeypatch):
    """Plant the 'restart from p' mistake in the oracle: the same Monte Carlo
    check must reject it."""
    g = _golden("worked_example_rnr.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    N = 200_000
    target, draft, d, u = _mc_batch(p, q, N, 20260923)

    def naive_residual(pp, qq):
        pp = np.asarray(pp, dtype=np.float64)
        return pp.copy(), float(pp.sum())

    monkeypatch.setattr(O, "positive_residual", naive_residual)
    res = O.verify_batch(target, draft, d, u, 1.0, O.MODE_STOCHASTIC)
    freq = np.bincount(res.tokens[:, 0], minlength=3) / N
    assert not _mc_freq_ok(p, freq, N)
    assert np.allclose(freq, g["naive_restart_from_p"], atol=0.01)


# --------------------------------------------------------------------------
# p = q, zero-q, invalid input
# --------------------------------------------------------------------------

def test_p_equals_q_accepts_everything_and_skips_residual():
    rng = np.random.default_rng(8)
    B, K, V = 50, 5, 40
    target = rng.normal(0, 2, (B, K + 1, V))
    draft = target[:, :K].copy()
    tokens = rng.integers(0, V, (B, K))
    u = rng.random((B, K + 1))
    res = O.verify_batch(target, draft, tokens, u, 0.7, O.MODE_STOCHASTIC)
    assert np.all(res.accept_len == K)
    assert np.all(res.z == -1.0) and res.z0_fallbacks == 0
    assert np.array_equal(res.p_d, res.q_d)
    assert np.array_equal(res.tokens[:, :K], tokens)


def test_zero_q_draft_is_accepted_and_counted():
    target = np.log(np.array([[0.2, 0.8], [0.5, 0.5]]))
    draft = np.array([[-np.inf, 0.0]])
    res = O.verify_sequence(target, draft, [0], [0.99, 0.5], 1.0, O.MODE_STOCHASTIC)
    assert res.accept_len == 1 and res.zero_q_accepts == 1


def test_invalid_sequences_are_flagged():
    rng = np.random.default_rng(2)
    B, K, V = 4, 3, 10
    target = rng.normal(0, 1, (B, K + 1, V))
    draft = rng.normal(0, 1, (B, K, V))
    tokens = rng.integers(0, V, (B, K))
    u = rng.random((B, K + 1))
    tokens[0, 1] = V                  # out of range
    target[1, 2, 3] = np.nan          # NaN row
    draft[2, 0, :] = -np.inf          # no finite maximum
    res = O.verify_batch(target, draft, tokens, u, 1.0, O.MODE_STOCHASTIC)
    assert list(res.accept_len[:3]) == [-1, -1, -1] and res.accept_len[3] >= 0
    assert np.all(res.tokens[:3] == -1)
    assert res.hist.sum() == 1 and res.invalid == 3
    g = O.verify_batch(target, draft, tokens, u, 1.0, O.MODE_GREEDY)
    # greedy reads target rows only: the all -inf draft row does not matter
    assert g.accept_len[0] == -1 and g.accept_len[1] == -1 and g.accept_len[2] >= 0


# --------------------------------------------------------------------------
# greedy and margin modes
# --------------------------------------------------------------------------

def test_greedy_hand_example_with_bonus():
    # argmax per row: 2, 0, 1, 3 (row 3 is the bonus row)
    target = np.array([[0, 1, 5, 2],
                       [9, 1, 1, 9],      # tie: lowest index 0
                       [0, 4, 1, 1],
                       [0, 0, 0, 7]], dtype=np.float64)
    r = O.verify_sequence(target, None, [2, 0, 1], None, 1.0, O.MODE_GREEDY)
    assert r.accept_len == 3 and list(r.tokens) == [2, 0, 1, 3]
    r = O.verify_sequence(target, None, [2, 3, 1], None, 1.0, O.MODE_GREEDY)
    assert r.accept_len == 1 and list(r.tokens) == [2, 0, -1, -1]
    r = O.verify_sequence(target, None, [0, 0, 1], None, 1.0, O.MODE_GREEDY)
    assert r.accept_len == 0 and list(r.tokens) == [2, -1, -1, -1]


def test_greedy_bruteforce_all_drafts():
    rng = np.random.default_rng(4)
    V, K = 3, 3
    target = rng.integers(0, 3, (K + 1, V)).astype(np.float64)   # many ties
    A = [int(np.flatnonzero(row == row.max())[0]) for row in target]
    for code in range(V ** K):
        d = [(code // V ** i) % V for i in range(K)]
        n = 0
        while n < K and d[n] == A[n]:
            n += 1
        r = O.verify_sequence(target, None, d, None, 1.0, O.MODE_GREEDY)
        assert r.accept_len == n
        assert list(r.tokens[:n]) == d[:n] and r.tokens[n] == A[n]


def test_margin_hand_example():
    # p = (0.5, 0.3, 0.2) at T = 1: ratios to the top-1 are (1, 0.6, 0.4)
    row = np.log([0.5, 0.3, 0.2])
    target = np.stack([row, row, row])
    r = O.verify_sequence(target, None, [1, 2], None, 1.0, O.MODE_MARGIN, tau=0.3)
    assert r.accept_len == 2 and list(r.tokens) == [1, 2, 0]
    assert np.allclose(r.p_d, [0.6, 0.4], atol=1e-14)
    r = O.verify_sequence(target, None, [1, 2], None, 1.0, O.MODE_MARGIN, tau=0.5)
    assert r.accept_len == 1 and list(r.tokens) == [1, 0, -1]
    r = O.verify_sequence(target, None, [2, 0], None, 1.0, O.MODE_MARGIN, tau=0.4)
    assert r.accept_len == 0 and list(r.tokens) == [0, -1, -1]   # strict '>'


def test_margin_limits_and_monotonicity():
    rng = np.random.default_rng(9)
    B, K, V = 60, 5, 12
    target = rng.normal(0, 2, (B, K + 1, V))
    target[:, :, 7] = -np.inf
    tokens = rng.integers(0, V, (B, K))
    g = O.verify_batch(target, None, tokens, None, 1.0, O.MODE_GREEDY)
    for tau in (1.0, 1.5):
        m = O.verify_batch(target, None, tokens, None, 1.0, O.MODE_MARGIN, tau=tau)
        assert np.array_equal(m.tokens, g.tokens)
    m0 = O.verify_batch(target, None, tokens, None, 1.0, O.MODE_MARGIN, tau=0.0)
    for k in range(B):
        first_zero = next((i for i in range(K) if tokens[k, i] == 7), K)
        assert m0.accept_len[k] == first_zero
    prev = None
    for tau in (0.0, 0.1, 0.3, 0.6, 0.9, 1.0):
        m = O.verify_batch(target, None, tokens, None, 0.8, O.MODE_MARGIN, tau=tau)
        if prev is not None:
            assert np.all(m.accept_len <= prev)
        prev = m.accept_len


# --------------------------------------------------------------------------
# EMA
# --------------------------------------------------------------------------

def test_ema_hand_values():
    s = O.EmaState(2, 0.99)
    s.observe(0, 1.0)
    assert s.ema[0] == 1.0
    s.observe(0, 0.0)
    assert math.isclose(s.ema[0], 0.99, rel_tol=1e-15)
    s.observe(0, 0.5)
    assert math.isclose(s.ema[0], 0.99 * 0.99 + 0.01 * 0.5, rel_tol=1e-15)
    for _ in range(100):
        s.observe(1, 0.25)
    assert s.ema[1] == 0.25 and s.steps[1] == 100


def test_ema_stationary_mean_under_constant_alpha():
    alpha, K, B, steps = 0.5, 3, 64, 400
    ema = O.EmaState(B, 0.95)
    for st in range(steps):
        target, draft, tokens, u = _const_alpha_batch(alpha, K, B, 1000 + st)
        O.verify_batch(target, draft, tokens, u, 1.0, O.MODE_STOCHASTIC, ema=ema)
    E = (1 - alpha ** (K + 1)) / (1 - alpha)
    assert abs(ema.ema.mean() - (E - 1) / K) < 0.02
