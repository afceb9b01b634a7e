"""Pins for the oracle's stopping rules: end-of-sequence token, per-sequence
draft count k_b and emission budget m_b.

The pages only say that end-of-sequence and length limits can end a cycle
before its draft block is used up, and that the returned tokens must agree with
them ([DVC] "Verify several proposed tokens in one target pass", "Speculation
needs cache rollback"; [RNR] s.5 on early stops). The readings (cut after the
first eos, then to m_b tokens; k_b drafts tested; the draw only when emitted)
are pinned here against things other than the stop-rule code itself:

  * pathwise, with the same uniforms, the output is the plain cycle's output
    truncated by an independent list operation (a correction never equals the
    rejected draft, so truncation cannot change which tokens are drafts);
  * k_b < K is the plain cycle of a K = k_b block on the sliced inputs;
  * by exact enumeration on V = 3, K = 2 the first token has law p_0 under any
    budget, a later token has law p_i given it is emitted, nothing follows an
    eos, and P(two or more tokens) = sum over x != eos of min(p_0, q_0)(x).
"""

import math

import numpy as np
import pytest

from oracle import spec_oracle as O

MODES = [O.MODE_STOCHASTIC, O.MODE_GREEDY, O.MODE_MARGIN]


def _logits(p):
    p = np.asarray(p, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.log(p)


def _case(rng, V, K, mode):
    target = rng.normal(0, 1.5, (K + 1, V))
    draft = target[:K] + rng.normal(0, 1.0, (K, V))
    if mode == O.MODE_STOCHASTIC:
        q = [O.softmax_t(draft[i], 1.0) for i in range(K)]
        toks = np.array([rng.choice(V, p=q[i]) for i in range(K)])
    else:
        # mostly the draft argmax, so that greedy/margin walks run long
        toks = np.argmax(draft, axis=1)
        flip = rng.random(K) < 0.2
        toks[flip] = rng.integers(0, V, flip.sum())
    u = rng.random(K + 1)
    return target, draft, toks, u


def _truncate(tokens, eos, m):
    e = [int(t) for t in tokens if t >= 0]
    if eos in e:
        e = e[:e.index(eos) + 1]
    return e[:m]


@pytest.mark.parametrize("mode", MODES)
def test_stop_rules_truncate_the_plain_cycle(mode):
    rng = np.random.default_rng(11 + mode)
    V, K = 12, 5
    hits = 0
    for _ in range(300):
        target, draft, toks, u = _case(rng, V, K, mode)
        plain = O.verify_sequence(target, draft, toks, u, 1.0, mode, 0.3)
        # eos: often one of the drafted tokens, sometimes any token or none
        r = rng.random()
        eos = int(toks[rng.integers(0, K)]) if r < 0.6 else int(rng.integers(-1, V))
        m = int(rng.integers(1, K + 3))
        res = O.verify_sequence(target, draft, toks, u, 1.0, mode, 0.3, eos=eos, max_emit=m)
        want = _truncate(plain.tokens, eos, m)
        got = [int(t) for t in res.tokens if t >= 0]
        assert got == want
        assert np.all(res.tokens[len(got):] == -1)
        assert res.accept_len == min(plain.accept_len, len(want))
        # the correction/bonus is evaluated only when it is emitted
        emitted_c = len(want) > plain.accept_len
        if mode == O.MODE_STOCHASTIC and not emitted_c:
            assert res.z == -1.0
        if mode == O.MODE_STOCHASTIC and emitted_c:
            assert res.z == plain.z
        hits += len(want) < len([t for t in plain.tokens if t >= 0])
    assert hits > 50          # the rules did cut many cycles


@pytest.mark.parametrize("mode", MODES)
def test_draft_count_is_a_shorter_block(mode):
    rng = np.random.default_rng(21 + mode)
    V, K = 10, 6
    for _ in range(200):
        target, draft, toks, u = _case(rng, V, K, mode)
        kb = int(rng.integers(0, K + 1))
        res = O.verify_sequence(target, draft, toks, u, 1.0, mode, 0.3, draft_len=kb)
        ref = O.verify_sequence(target[:kb + 1], draft[:kb], toks[:kb],
                                np.concatenate([u[:kb], u[K:]]), 1.0, mode, 0.3)
        assert np.array_equal(res.tokens[:kb + 1], ref.tokens)
        assert np.all(res.tokens[kb + 1:] == -1)
        assert res.accept_len == ref.accept_len
        assert res.draft_len == kb


def test_rows_past_the_draft_count_are_not_needed():
    rng = np.random.default_rng(3)
    V, K = 8, 4
    target, draft, toks, u = _case(rng, V, K, O.MODE_STOCHASTIC)
    target[3, 2] = np.nan
    draft[2, :] = -np.inf
    toks[3] = V + 5
    res = O.verify_sequence(target, draft, toks, u, 1.0, O.MODE_STOCHASTIC, draft_len=2)
    assert res.valid and 0 <= res.accept_len <= 2
    assert not O.verify_sequence(target, draft, toks, u, 1.0, O.MODE_STOCHASTIC,
                                 draft_len=3).valid
    for kb, m in [(-1, 3), (K + 1, 3), (2, 0)]:
        assert not O.verify_sequence(target, draft, toks, u, 1.0, O.MODE_STOCHASTIC,
                                     draft_len=kb, max_emit=m).valid


def _cells(breaks):
    pts = sorted({0.0, 1.0, *[min(max(b, 0.0), 1.0) for b in breaks]})
    return [(0.5 * (a + b), b - a) for a, b in zip(pts[:-1], pts[1:]) if b > a]


@pytest.mark.parametrize("eos,m", [(1, 3), (0, 3), (1, 2), (2, 1), (-1, 2)])
def test_exact_law_with_stop_rules_bruteforce_V3_K2(eos, m):
    rng = np.random.default_rng(17)
    V, K = 3, 2
    for trial in range(3):
        P = [rng.dirichlet(np.ones(V)) for _ in range(K + 1)]
        Q = [rng.dirichlet(np.ones(V)) for _ in range(K)]
        target = np.stack([_logits(p) for p in P])
        draft = np.stack([_logits(q) for q in Q])
        law = {}
        for d0 in range(V):
            for d1 in range(V):
                wq = Q[0][d0] * Q[1][d1]
                d = np.array([d0, d1])
                a = [min(1.0, P[i][d[i]] / Q[i][d[i]]) for i in range(K)]
                ws = [np.maximum(P[i] - Q[i], 0) for i in range(K)] + [P[K]]
                br = [c for w in ws for c in (np.cumsum(w) / w.sum()).tolist()]
                for u0, w0 in _cells([a[0]]):
                    for u1, w1 in _cells([a[1]]):
                        for u2, w2 in _cells(br):
                            res = O.verify_sequence(target, draft, d, [u0, u1, u2], 1.0,
                                                    O.MODE_STOCHASTIC, eos=eos, max_emit=m)
                            key = tuple(int(t) for t in res.tokens if t >= 0)
                            law[key] = law.get(key, 0.0) + wq * w0 * w1 * w2
        assert math.isclose(sum(law.values()), 1.0, abs_tol=1e-12)
        for k in law:
            assert 1 <= len(k) <= m
            if eos in k:
                assert k.index(eos) == len(k) - 1      # nothing after an eos
        first = np.zeros(V)
        for k, w in law.items():
            first[k[0]] += w
        assert np.allclose(first, P[0], atol=1e-12)
        if m >= 2:
            second = np.zeros(V)
            for k, w in law.items():
                if len(k) >= 2:
                    second[k[1]] += w
            assert np.allclose(second / second.sum(), P[1], atol=1e-12)
            # two or more tokens: draft 0 kept and not the eos
            n2 = sum(w for k, w in law.items() if len(k) >= 2)
            want = sum(min(P[0][x], Q[0][x]) for x in range(V) if x != eos)
            assert math.isclose(n2, want, abs_tol=1e-12)


def test_histogram_and_ema_with_draft_counts():
    rng = np.random.default_rng(8)
    B, V, K = 40, 9, 4
    target = rng.normal(0, 1.5, (B, K + 1, V))
    draft = target[:, :K] + rng.normal(0, 1.0, (B, K, V))
    toks = np.array([[rng.choice(V, p=O.softmax_t(draft[b, i], 1.0)) for i in range(K)]
                     for b in range(B)])
    u = rng.random((B, K + 1))
    kb = rng.integers(0, K + 1, B)
    m = rng.integers(1, K + 2, B)
    ema = O.EmaState(B, 0.9)
    res = O.verify_batch(target, draft, toks, u, 1.0, O.MODE_STOCHASTIC, ema=ema,
                         eos=2, draft_len=kb, max_emit=m)
    assert np.array_equal(res.hist, np.bincount(res.accept_len, minlength=K + 1))
    for b in range(B):
        if kb[b] == 0:
            assert ema.steps[b] == 0 and res.accept_len[b] == 0
        else:
            assert ema.steps[b] == 1
            assert ema.ema[b] == res.accept_len[b] / kb[b]
        n = int((res.tokens[b] >= 0).sum())
        assert 1 <= n <= m[b] and n <= kb[b] + 1
