"""Pins for the oracle's draft residual side output ([DRIFT] "The update rule
and its objective"; support width m = 32 in "Ablations").

The page fixes the quantity (target log-probability minus draft
log-probability, both restricted to a shared top-m support) but not which top
m: the reading is the draft's top m, ties to the lower token index. Pinned
here against computations that do not share the oracle's code: the support
against rank counting, the residual against closed forms (p = q gives 0; the
restricted laws sum to one; with m >= V it is the difference of the full log
softmaxes; a shift of either row's logits by a constant leaves it unchanged).
"""

import math

import numpy as np
import pytest

from oracle import spec_oracle as O


def _tied_row(rng, V):
    return np.round(rng.normal(0, 1.5, V) * 4) / 4


@pytest.mark.parametrize("V,m", [(5, 3), (40, 7), (40, 40), (64, 32), (7, 12)])
def test_support_is_rank_counting(V, m):
    rng = np.random.default_rng(V * 100 + m)
    for _ in range(30):
        x = _tied_row(rng, V)
        S = O.draft_topm_support(x, m)
        rank = np.array([np.sum(x > x[v]) + np.sum((x == x[v]) & (np.arange(V) < v))
                         for v in range(V)])
        want = np.argsort(rank)[:min(m, V)]     # ranks are distinct
        assert np.array_equal(S, want)
        assert len(set(S.tolist())) == len(S)


def test_equal_rows_give_zero_residual():
    rng = np.random.default_rng(1)
    for _ in range(20):
        x = rng.normal(0, 2, 50)
        S, r = O.drift_residual(x, x.copy(), 0.8, 16)
        assert np.all(r == 0.0)


def test_restricted_laws_are_normalised():
    rng = np.random.default_rng(2)
    for _ in range(50):
        xt, xd = rng.normal(0, 2, 80), rng.normal(0, 2, 80)
        T = float(rng.uniform(0.3, 2.0))
        S, r = O.drift_residual(xt, xd, T, 32)
        qS = np.exp(xd[S] / T) / np.exp(xd[S] / T).sum()
        assert math.isclose(float(np.sum(qS * np.exp(r))), 1.0, rel_tol=1e-12)   # sum p_S = 1


def test_full_support_is_log_softmax_difference():
    rng = np.random.default_rng(3)
    for _ in range(20):
        xt, xd = rng.normal(0, 2, 30), rng.normal(0, 2, 30)
        S, r = O.drift_residual(xt, xd, 1.3, 64)
        lp = np.log(O.softmax_t(xt, 1.3))[S]
        lq = np.log(O.softmax_t(xd, 1.3))[S]
        assert np.allclose(r, lp - lq, atol=1e-12)


def test_shift_invariance():
    rng = np.random.default_rng(4)
    xt, xd = rng.normal(0, 2, 60), rng.normal(0, 2, 60)
    S, r = O.drift_residual(xt, xd, 0.7, 32)
    S2, r2 = O.drift_residual(xt + 11.0, xd - 3.0, 0.7, 32)
    assert np.array_equal(S, S2) and np.allclose(r, r2, atol=1e-12)


def test_batch_respects_draft_counts_and_validity():
    rng = np.random.default_rng(5)
    B, K, V, m = 4, 3, 20, 8
    target = rng.normal(0, 1, (B, K + 1, V))
    draft = rng.normal(0, 1, (B, K, V))
    sup, res = O.drift_batch(target, draft, 1.0, m, np.array([1, -1, 0, 2]), np.array([3, 3, 1, 0]))
    assert np.all(sup[1] == -1) and np.all(np.isnan(res[1]))      # invalid sequence
    assert np.all(sup[2, 1:] == -1) and np.all(sup[2, 0] >= 0)    # k_b = 1
    assert np.all(sup[3] == -1)                                   # k_b = 0
    assert np.all(sup[0] >= 0)
