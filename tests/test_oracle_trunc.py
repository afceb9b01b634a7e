"""Pins for the oracle's top-k / top-p truncation of p and q.

The pages only say that p and q are the distributions the samplers really
use, after temperature, masks and truncation, and that a mask applied only
after the correction breaks the guarantee ([RNR] s.1 and s.2). The top-k and
top-p rules themselves are the usual ones; the readings (ties at a cut keep
the whole value level, top-k before top-p, greedy and margin modes untouched)
are pinned here against computations that do not share the oracle's code:

  * top-k keep sets against rank counting: a token is kept iff fewer than k
    tokens have a strictly larger logit;
  * top-p keep sets against a brute-force search for the shortest run of
    whole value levels from the top whose mass reaches top_p, and, for
    distinct values, against the textbook rule (sort ascending, drop the
    tokens whose inclusive cumulative mass is at most 1 - top_p);
  * no truncation reproduces the plain cycle bit for bit;
  * top_k = 1 with drafts at the draft argmax reduces stochastic verification
    to greedy verification;
  * by exact enumeration on V = 4, K = 2 the emitted tokens have the law of
    the truncated target, with drafts drawn from the truncated draft.
"""

import math

import numpy as np
import pytest

from oracle import spec_oracle as O


def _softmax(x, T):
    e = np.exp((x - x.max()) / T)
    return e / e.sum()


def _keep_topk_by_rank(x, k):
    V = x.size
    if not (1 <= k < V):
        return np.ones(V, dtype=bool)
    return np.array([(x > x[v]).sum() < k for v in range(V)])


def _keep_topp_by_prefix_search(x, T, base_keep, top_p):
    """Shortest run of whole value levels (largest first) of the base-kept
    tokens whose renormalised mass reaches top_p, by trying every run."""
    p = np.where(base_keep, _softmax(x, T), 0.0)
    p = p / p.sum()
    levels = sorted(set(x[base_keep].tolist()), reverse=True)
    for m in range(1, len(levels) + 1):
        sel = base_keep & (x >= levels[m - 1])
        if p[sel].sum() >= top_p:
            return sel, p
    return base_keep.copy(), p


def _tied_row(rng, V, levels=7):
    # logits on a coarse grid, so that ties at the cuts are common
    return np.round(rng.normal(0, 1.5, V) * levels) / levels


@pytest.mark.parametrize("V", [5, 17, 64])
def test_top_k_keep_set_is_rank_counting(V):
    rng = np.random.default_rng(100 + V)
    for _ in range(40):
        x = _tied_row(rng, V)
        for k in [-1, 0, 1, 2, 3, V // 2, V - 1, V, V + 3]:
            keep, dist = O.truncation_keep(x, 1.0, k, 1.0)
            assert np.array_equal(keep, _keep_topk_by_rank(x, k)), (k, x)
            assert dist == math.inf


@pytest.mark.parametrize("V", [6, 20, 80])
def test_top_p_keep_set_is_the_shortest_level_run(V):
    rng = np.random.default_rng(200 + V)
    checked = 0
    for _ in range(40):
        x = _tied_row(rng, V)
        T = float(rng.choice([0.5, 1.0, 1.7]))
        for k in [0, 3, V // 2]:
            base = _keep_topk_by_rank(x, k)
            for top_p in [1e-9, 0.3, 0.5, 0.8, 0.95, 0.999]:
                keep, dist = O.truncation_keep(x, T, k, top_p)
                want, _ = _keep_topp_by_prefix_search(x, T, base, top_p)
                if dist < 1e-12:
                    continue        # a level mass within rounding of top_p
                assert np.array_equal(keep, want), (k, top_p, x)
                assert keep[np.argmax(x)]
                checked += 1
    assert checked > 500


def test_top_p_distinct_values_follow_the_sorted_cumsum_rule():
    rng = np.random.default_rng(7)
    for _ in range(200):
        V = int(rng.integers(2, 60))
        x = rng.normal(0, 2.0, V)                     # distinct almost surely
        top_p = float(rng.uniform(0.05, 0.99))
        keep, dist = O.truncation_keep(x, 1.0, 0, top_p)
        if dist < 1e-12:
            continue
        p = _softmax(x, 1.0)
        order = np.argsort(p)                         # ascending
        cum = np.cumsum(p[order])
        drop = np.zeros(V, dtype=bool)
        drop[order[cum <= 1.0 - top_p]] = True
        assert np.array_equal(keep, ~drop)


def test_truncated_softmax_is_renormalised_and_zero_outside():
    rng = np.random.default_rng(3)
    for _ in range(50):
        x = _tied_row(rng, 40)
        p, _ = O.truncated_softmax(x, 0.8, 10, 0.7)
        keep, _ = O.truncation_keep(x, 0.8, 10, 0.7)
        assert math.isclose(p.sum(), 1.0, rel_tol=1e-12)
        assert np.all(p[~keep] == 0.0) and np.all(p[keep] > 0.0)
        full = _softmax(x, 0.8)
        assert np.allclose(p[keep], full[keep] / full[keep].sum(), rtol=1e-12)


MODES = [O.MODE_STOCHASTIC, O.MODE_GREEDY, O.MODE_MARGIN]


@pytest.mark.parametrize("mode", MODES)
def test_no_truncation_is_the_plain_cycle(mode):
    rng = np.random.default_rng(30 + mode)
    V, K = 25, 4
    for _ in range(60):
        target = rng.normal(0, 1.5, (K + 1, V))
        draft = target[:K] + rng.normal(0, 1.0, (K, V))
        toks = rng.integers(0, V, K)
        u = rng.random(K + 1)
        plain = O.verify_sequence(target, draft, toks, u, 0.9, mode, 0.3)
        for k, tp in [(0, 1.0), (V, 1.0), (V + 4, 2.0), (-2, 1.0)]:
            res = O.verify_sequence(target, draft, toks, u, 0.9, mode, 0.3, top_k=k, top_p=tp)
            assert np.array_equal(res.tokens, plain.tokens)
            assert res.accept_len == plain.accept_len
            assert np.array_equal(res.p_d, plain.p_d, equal_nan=True)
            assert np.array_equal(res.q_d, plain.q_d, equal_nan=True)
            assert res.z == plain.z


def test_greedy_and_margin_ignore_truncation():
    rng = np.random.default_rng(41)
    V, K = 30, 5
    for mode in (O.MODE_GREEDY, O.MODE_MARGIN):
        for _ in range(40):
            target = rng.normal(0, 1.5, (K + 1, V))
            toks = np.argmax(target[:K] + rng.normal(0, 0.7, (K, V)), axis=1)
            a = O.verify_sequence(target, None, toks, None, 1.0, mode, 0.2)
            b = O.verify_sequence(target, None, toks, None, 1.0, mode, 0.2, top_k=2, top_p=0.3)
            assert np.array_equal(a.tokens, b.tokens) and a.accept_len == b.accept_len


def test_top_k_one_is_greedy_verification():
    """top_k = 1: p and q are point masses on the argmaxes, so a draft at the
    draft argmax is kept iff it is the target argmax, and the correction or
    bonus is the target argmax: the greedy rule, whatever the uniforms."""
    rng = np.random.default_rng(5)
    V, K = 40, 6
    for _ in range(200):
        target = rng.normal(0, 1.0, (K + 1, V))
        draft = target[:K] + rng.normal(0, 0.8, (K, V))
        toks = np.argmax(draft, axis=1)
        u = rng.random(K + 1)
        st = O.verify_sequence(target, draft, toks, u, 1.0, O.MODE_STOCHASTIC, top_k=1)
        gr = O.verify_sequence(target, None, toks, None, 1.0, O.MODE_GREEDY)
        assert np.array_equal(st.tokens, gr.tokens)
        assert st.accept_len == gr.accept_len
        # a vanishing nucleus keeps only the top level as well
        tp = O.verify_sequence(target, draft, toks, u, 1.0, O.MODE_STOCHASTIC, top_p=1e-12)
        assert np.array_equal(tp.tokens, gr.tokens)


@pytest.mark.parametrize("top_p", [0.0, -0.5, float("nan")])
def test_non_positive_top_p_is_invalid(top_p):
    rng = np.random.default_rng(9)
    V, K = 12, 3
    target = rng.normal(0, 1, (K + 1, V))
    draft = rng.normal(0, 1, (K, V))
    res = O.verify_sequence(target, draft, [0, 1, 2], rng.random(K + 1), 1.0,
                            O.MODE_STOCHASTIC, top_p=top_p)
    assert not res.valid and res.accept_len == -1 and np.all(res.tokens == -1)


def _cells(breaks):
    pts = sorted({0.0, 1.0, *[min(max(b, 0.0), 1.0) for b in breaks]})
    return [(0.5 * (a + b), b - a) for a, b in zip(pts[:-1], pts[1:]) if b > a]


def _trunc_law(x, T, k, top_p):
    base = _keep_topk_by_rank(x, k)
    if top_p < 1.0:
        keep, _ = _keep_topp_by_prefix_search(x, T, base, top_p)
    else:
        keep = base
    p = np.where(keep, _softmax(x, T), 0.0)
    return p / p.sum()


@pytest.mark.parametrize("k,top_p", [(2, 1.0), (0, 0.7), (3, 0.8), (1, 1.0), (0, 0.35)])
def test_exact_law_with_truncation_bruteforce_V4_K2(k, top_p):
    rng = np.random.default_rng(23)
    V, K = 4, 2
    overlap = 0
    for _ in range(6):
        target = rng.normal(0, 1.2, (K + 1, V))
        draft = target[:K] + rng.normal(0, 0.8, (K, V))
        Pt = [_trunc_law(target[i], 1.0, k, top_p) for i in range(K + 1)]
        Qt = [_trunc_law(draft[i], 1.0, k, top_p) for i in range(K)]
        law = {}
        for d0 in range(V):
            for d1 in range(V):
                wq = Qt[0][d0] * Qt[1][d1]
                if wq == 0.0:
                    continue                  # never proposed by the truncated draft
                d = np.array([d0, d1])
                a = [min(1.0, Pt[i][d[i]] / Qt[i][d[i]]) for i in range(K)]
                ws = [np.maximum(Pt[i] - Qt[i], 0) for i in range(K)] + [Pt[K]]
                br = [c for w in ws if w.sum() > 0 for c in (np.cumsum(w) / w.sum()).tolist()]
                for u0, w0 in _cells([a[0]]):
                    for u1, w1 in _cells([a[1]]):
                        for u2, w2 in _cells(br):
                            res = O.verify_sequence(target, draft, d, [u0, u1, u2], 1.0,
                                                    O.MODE_STOCHASTIC, top_k=k, top_p=top_p)
                            key = tuple(int(t) for t in res.tokens if t >= 0)
                            law[key] = law.get(key, 0.0) + wq * w0 * w1 * w2
        assert math.isclose(sum(law.values()), 1.0, abs_tol=1e-12)
        first = np.zeros(V)
        second = np.zeros(V)
        for key, w in law.items():
            first[key[0]] += w
            if len(key) >= 2:
                second[key[1]] += w
        assert np.allclose(first, Pt[0], atol=1e-12)
        n2 = sum(w for key, w in law.items() if len(key) >= 2)
        assert math.isclose(n2, float(np.minimum(Pt[0], Qt[0]).sum()), abs_tol=1e-12)
        if n2 > 0.0:
            assert np.allclose(second / second.sum(), Pt[1], atol=1e-12)
            overlap += 1
    assert overlap >= 2


def test_batch_passes_per_sequence_truncation():
    rng = np.random.default_rng(12)
    B, V, K = 12, 30, 3
    target = rng.normal(0, 1.5, (B, K + 1, V))
    draft = target[:, :K] + rng.normal(0, 1.0, (B, K, V))
    toks = rng.integers(0, V, (B, K))
    u = rng.random((B, K + 1))
    tk = rng.integers(0, V + 2, B)
    tp = rng.uniform(0.2, 1.2, B).astype(np.float32)
    res = O.verify_batch(target, draft, toks, u, 1.0, O.MODE_STOCHASTIC, top_k=tk, top_p=tp)
    for b in range(B):
        one = O.verify_sequence(target[b], draft[b], toks[b], u[b], 1.0, O.MODE_STOCHASTIC,
                                top_k=int(tk[b]), top_p=float(tp[b]))
        assert np.array_equal(res.tokens[b], one.tokens)
        assert res.accept_len[b] == one.accept_len


def test_signed_zeros_are_one_level():
    """-0 and +0 compare equal, so they are one value level: top_k = 1 on a
    row whose maximum is zero keeps both zeros (counted with multiplicity),
    and top-p keeps or drops them together (fp32 rows hold both)."""
    x = np.array([-1.0, 0.0, -3.0, -0.0, -2.0])
    keep, _ = O.truncation_keep(x, 1.0, 1, 1.0)
    assert keep.tolist() == [False, True, False, True, False]
    # mass of the zero level is 2 / (2 + e^-1 + e^-2 + e^-3) ~ 0.783: a top_p
    # below that keeps exactly the two zeros, above it the next level too
    keep, _ = O.truncation_keep(x, 1.0, 0, 0.5)
    assert keep.tolist() == [False, True, False, True, False]
    keep, _ = O.truncation_keep(x, 1.0, 0, 0.8)
    assert keep.tolist() == [True, True, False, True, False]
    p, _ = O.truncated_softmax(x, 1.0, 1, 1.0)
    assert p[1] == p[3] == 0.5 and p.sum() == 1.0
