"""Pins for the oracle's tree-shape policy epilogue ([MNW] s.3, dynamic draft
tree-shaping).

What the page fixes, and is pinned here: the rolling acceptance is an EMA
with alpha = 0.3 (decay 0.7 on the old value); the shape range runs from
(3, 4, 4) to (7, 1, 8) as the confidence score goes from 0 to 1, depth
growing with the score and branching with one minus it; five consecutive
zero-accept steps restore the starting configuration. What the page leaves
open (how the draft's top-1 probability and the acceptance combine into the
score, and the divisor d) is a reading, min(1, conf * acc / d): that part is
parity unpinned, and only its saturation and monotonicity are checked.
"""

import math

import numpy as np
import pytest

from oracle import spec_oracle as O


def test_shape_endpoints_and_interpolation():
    assert O.shape_for(0.0) == (3, 4, 4)
    assert O.shape_for(1.0) == (7, 1, 8)
    assert O.shape_for(0.5) == (5, 3, 6)          # top-k 2.5 rounds half up
    assert O.shape_for(0.25) == (4, 3, 5)         # 4.0, 3.25, 5.0
    prev = O.shape_for(0.0)
    for dcs in np.linspace(0.0, 1.0, 401):
        s = O.shape_for(float(dcs))
        assert s[0] >= prev[0] and s[2] >= prev[2] and s[1] <= prev[1]   # deeper, narrower
        assert 3 <= s[0] <= 7 and 1 <= s[1] <= 4 and 4 <= s[2] <= 8
        prev = s


def test_alpha_0_3_is_decay_0_7():
    ema = O.EmaState(1, 0.7)
    ema.observe(0, 1.0)
    ema.observe(0, 0.0)
    assert ema.ema[0] == pytest.approx(0.7)       # new observation weighted 0.3
    ema.observe(0, 1.0)
    assert ema.ema[0] == pytest.approx(0.7 * 0.7 + 0.3)


def _step(pol, ema, a, k=4, conf=0.9):
    if k > 0:
        ema.observe(0, a / k)
    return pol.step(ema, 0, True, a, k, conf)


def test_circuit_breaker_after_five_zero_accept_steps():
    ema = O.EmaState(1, 0.7)
    pol = O.TreePolicy(1, 0.5)
    shape, dcs = _step(pol, ema, 4)                # full acceptance: confident
    assert shape == (7, 1, 8) and dcs == 1.0
    for i in range(4):                            # four misses: not yet
        shape, _ = _step(pol, ema, 0)
        assert pol.streak[0] == i + 1
    shape, dcs = _step(pol, ema, 0)                # the fifth restores the start
    assert shape == (3, 4, 4) and dcs == 0.0
    assert pol.streak[0] == 0 and ema.steps[0] == 0
    shape, _ = _step(pol, ema, 2)                  # the EMA restarts from this step
    assert ema.ema[0] == 0.5 and ema.steps[0] == 1


def test_breaker_counts_only_consecutive_tested_steps():
    ema = O.EmaState(1, 0.7)
    pol = O.TreePolicy(1, 0.5)
    for _ in range(4):
        _step(pol, ema, 0)
    _step(pol, ema, 0, k=0)                        # no drafts tested: no observation
    assert pol.streak[0] == 4
    _step(pol, ema, 1)                             # one kept draft resets the streak
    assert pol.streak[0] == 0
    for _ in range(4):
        _step(pol, ema, 0)
    assert pol.streak[0] == 4 and ema.steps[0] > 0


def test_score_saturates_and_is_monotone():
    pol = O.TreePolicy(1, 0.4)
    ema = O.EmaState(1, 0.7)
    ema.observe(0, 0.5)
    shapes = [pol.step(ema, 0, True, 2, 4, c)[0] for c in np.linspace(0, 1, 21)]
    depth = [s[0] for s in shapes]
    assert depth == sorted(depth)
    assert pol.step(ema, 0, True, 2, 4, 1.0)[1] == 1.0    # 1 * 0.5 / 0.4 saturates
    assert pol.step(ema, 0, True, 2, 4, 0.0) == ((3, 4, 4), 0.0)


@pytest.mark.parametrize("conf", [-0.1, 1.5, float("nan")])
def test_invalid_inputs_leave_the_state(conf):
    pol = O.TreePolicy(1, 0.5)
    ema = O.EmaState(1, 0.7)
    pol.streak[0] = 3
    assert pol.step(ema, 0, True, 0, 4, conf)[0] == (-1, -1, -1)
    assert pol.step(ema, 0, False, 0, 4, 0.5)[0] == (-1, -1, -1)
    assert pol.streak[0] == 3


def test_batch_policy_matches_stepwise():
    rng = np.random.default_rng(2)
    B, V, K = 6, 20, 4
    ema_a, ema_b = O.EmaState(B, 0.7), O.EmaState(B, 0.7)
    pol_a, pol_b = O.TreePolicy(B, 0.45), O.TreePolicy(B, 0.45)
    for step in range(12):
        target = rng.normal(0, 1.5, (B, K + 1, V))
        # mostly mismatching drafts in the first sequences, so breakers fire
        toks = np.argmax(target[:, :K], axis=2)
        toks[: step % 3 + 1] = (toks[: step % 3 + 1] + 1) % V
        conf = rng.uniform(0, 1, B).astype(np.float32)
        res = O.verify_batch(target, None, toks, None, 1.0, O.MODE_GREEDY, ema=ema_a,
                             policy=pol_a, conf=conf)
        for b in range(B):
            r = O.verify_sequence(target[b], None, toks[b], None, 1.0, O.MODE_GREEDY)
            if r.valid and r.draft_len > 0:
                ema_b.observe(b, r.accept_len / r.draft_len)
            shape, dcs = pol_b.step(ema_b, b, r.valid, r.accept_len, r.draft_len, conf[b])
            assert tuple(res.shape[b]) == shape
            assert res.dcs[b] == dcs or (math.isnan(dcs) and math.isnan(res.dcs[b]))
    assert np.array_equal(pol_a.streak, pol_b.streak)
