"""Value pins for the oracle's boundary distances and the margin temperature.

The parity tests excuse a GPU/oracle difference only when the oracle says a
decision lay within 1e-6 of its boundary, so the distances themselves must be
right: a distance computed too small would silently widen the excused band
("Speculative decoding: why correcting a rejection is not resampling from the
target", section 4, on checking a sampler against its exact law). Every value
below is worked out by hand from the definitions:

  * acceptance test at position i: |u_i - p(d)/q(d)|, the distance of the
    uniform from the point where the keep/reject decision flips;
  * inverse-CDF draw: the distance of u from the nearer edge of the chosen
    token's interval [C_{v-1}/C_end, C_v/C_end);
  * margin test: |p(d)/p(top1) - tau|, with p at the call's temperature
    ("Margins, Not Windows", section 3, the margin rule);
  * top-p cut: the smallest |mass above a value level - top_p| over the levels
    of the kept top-k set.

The last tests plant mistakes in the oracle (distances halved; the margin
ratio taken without its temperature) and check that the pins catch them.
"""

import builtins
import math

import numpy as np
import pytest

from oracle import spec_oracle as O

TOL = 1e-12


def _logits(p):
    p = np.asarray(p, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.log(p)


# --------------------------------------------------------------------------
# inverse CDF
# --------------------------------------------------------------------------

def check_inverse_cdf_distances():
    w = np.array([0.25, 0.5, 0.25])          # intervals [0,.25) [.25,.75) [.75,1)
    for u, tok, dist in ((0.3, 1, 0.05), (0.1, 0, 0.1), (0.8, 2, 0.05), (0.0, 0, 0.0),
                         (0.5, 1, 0.25), (0.74, 1, 0.01)):
        t, d = O.inverse_cdf(w, u)
        assert t == tok, (u, t, tok)
        assert abs(d - dist) <= TOL, (u, d, dist)
    # zero-weight tokens own no interval: (0, .5, 0, .5) -> [0,.5) and [.5,1)
    w = np.array([0.0, 0.5, 0.0, 0.5])
    for u, tok, dist in ((0.4, 1, 0.1), (0.55, 3, 0.05), (0.9, 3, 0.1)):
        t, d = O.inverse_cdf(w, u)
        assert t == tok and abs(d - dist) <= TOL, (u, t, d)
    # unnormalised weights: the same intervals after dividing by the total
    t, d = O.inverse_cdf(np.array([2.0, 6.0]), 0.2)
    assert t == 0 and abs(d - 0.05) <= TOL


def test_inverse_cdf_distance_values():
    check_inverse_cdf_distances()


# --------------------------------------------------------------------------
# acceptance tests and the draw inside verify_sequence
# --------------------------------------------------------------------------

# "Speculative Decoding: Draft, Verify, and Correct", "Three possible next
# tokens": p = (0.6, 0.3, 0.1), q = (0.2, 0.5, 0.3); acceptance (1, 0.6, 1/3),
# positive residual (0.4, 0, 0).
P_DVC = [0.6, 0.3, 0.1]
Q_DVC = [0.2, 0.5, 0.3]
P_BONUS = [0.5, 0.25, 0.25]                 # target row K: intervals [0,.5) [.5,.75) [.75,1)


def _one_draft(p0, q0, p1, tok, u0, uk):
    target = np.stack([_logits(p0), _logits(p1)])
    draft = _logits(q0)[None, :]
    return O.verify_sequence(target, draft, [tok], [u0, uk], 1.0, O.MODE_STOCHASTIC)


def check_acceptance_distances():
    # token 2: p/q = 1/3; u = 0.3 keeps it, 1/30 from the flip; the bonus
    # draw from row K at u = 0.6 lands in [.5, .75): token 1, 0.1 from an edge
    r = _one_draft(P_DVC, Q_DVC, P_BONUS, 2, 0.3, 0.6)
    assert r.accept_len == 1 and list(r.tokens) == [2, 1]
    assert len(r.dists) == 2
    assert abs(r.dists[0] - 1.0 / 30.0) <= TOL and abs(r.dists[1] - 0.1) <= TOL
    assert abs(r.min_dist - 1.0 / 30.0) <= TOL
    # token 1: p/q = 0.6; u = 0.75 rejects it, 0.15 from the flip; the residual
    # (1, 0, 0) gives token 0 on [0, 1): u = 0.2 is 0.2 from its nearer edge
    r = _one_draft(P_DVC, Q_DVC, P_BONUS, 1, 0.75, 0.2)
    assert r.accept_len == 0 and list(r.tokens) == [0, -1]
    assert abs(r.z - 0.4) <= TOL
    assert abs(r.dists[0] - 0.15) <= TOL and abs(r.dists[1] - 0.2) <= TOL
    assert abs(r.min_dist - 0.15) <= TOL
    # token 0: p >= q, kept whatever u is; its flip point p/q = 3 lies 2.7
    # from u = 0.3, so the bonus draw's 0.1 is the nearest boundary
    r = _one_draft(P_DVC, Q_DVC, P_BONUS, 0, 0.3, 0.6)
    assert r.accept_len == 1 and list(r.tokens) == [0, 1]
    assert abs(r.dists[0] - 2.7) <= TOL and abs(r.min_dist - 0.1) <= TOL
    # a residual with two positive entries: p = (.5, .3, .2), q = (.1, .2, .7):
    # [p - q]+ = (.4, .1, 0), Z = 0.5, normalised (.8, .2, 0). Token 2 has
    # p/q = 2/7 and u = 0.5 rejects it, 3/14 from the flip; u_K = 0.85 falls
    # in token 1's interval [.8, 1), 0.05 from its lower edge
    r = _one_draft([0.5, 0.3, 0.2], [0.1, 0.2, 0.7], P_BONUS, 2, 0.5, 0.85)
    assert r.accept_len == 0 and list(r.tokens) == [1, -1]
    assert abs(r.z - 0.5) <= TOL
    assert abs(r.dists[0] - 3.0 / 14.0) <= TOL and abs(r.dists[1] - 0.05) <= TOL
    assert abs(r.min_dist - 0.05) <= TOL


def test_acceptance_and_draw_distance_values():
    check_acceptance_distances()


def test_batch_counts_the_decisions_taken():
    """verify_batch reports how many decisions it took (acceptance tests,
    draws, margin tests, top-p cuts): the denominator of the excuse rate."""
    target = np.stack([np.stack([_logits(P_DVC), _logits(P_BONUS)])] * 3)
    draft = np.stack([_logits(Q_DVC)[None, :]] * 3)
    tokens = np.array([[2], [1], [0]])
    u = np.array([[0.3, 0.6], [0.75, 0.2], [0.3, 0.6]])
    r = O.verify_batch(target, draft, tokens, u, 1.0, O.MODE_STOCHASTIC)
    assert r.n_decisions == 6                 # one test and one draw each
    assert np.allclose(r.min_dist, [1.0 / 30.0, 0.15, 0.1], atol=TOL)
    g = O.verify_batch(target, None, tokens, None, 1.0, O.MODE_GREEDY)
    assert g.n_decisions == 0 and np.all(np.isinf(g.min_dist))   # exact comparisons only


# --------------------------------------------------------------------------
# margin rule
# --------------------------------------------------------------------------

def check_margin_distances():
    # p = (0.5, 0.3, 0.2) at T = 1: ratios to the top-1 (1, 0.6, 0.4)
    row = _logits([0.5, 0.3, 0.2])
    target = np.stack([row, row, row])
    r = O.verify_sequence(target, None, [1, 2], None, 1.0, O.MODE_MARGIN, tau=0.3)
    assert r.accept_len == 2
    assert len(r.dists) == 2
    assert abs(r.dists[0] - 0.3) <= TOL and abs(r.dists[1] - 0.1) <= TOL
    # a draft equal to the argmax takes no margin decision
    r = O.verify_sequence(target, None, [0, 1], None, 1.0, O.MODE_MARGIN, tau=0.3)
    assert r.accept_len == 2 and len(r.dists) == 1 and abs(r.dists[0] - 0.3) <= TOL


def check_margin_temperature():
    # logits (2, 1, 0): the ratio of token 1 to the top-1 is exp(-1 / T)
    row = np.array([2.0, 1.0, 0.0])
    target = np.stack([row, row, row])
    # T = 0.5: exp(-2) = 0.1353 < 0.2, rejected at position 0
    r = O.verify_sequence(target, None, [1, 1], None, 0.5, O.MODE_MARGIN, tau=0.2)
    assert r.accept_len == 0 and list(r.tokens) == [0, -1, -1]
    assert abs(r.p_d[0] - math.exp(-2.0)) <= TOL
    assert abs(r.dists[0] - (0.2 - math.exp(-2.0))) <= TOL
    # T = 1: exp(-1) = 0.3679 > 0.2, both kept, bonus = argmax of row 2
    r = O.verify_sequence(target, None, [1, 1], None, 1.0, O.MODE_MARGIN, tau=0.2)
    assert r.accept_len == 2 and list(r.tokens) == [1, 1, 0]
    assert np.allclose(r.p_d, math.exp(-1.0), atol=TOL)
    # T = 2: exp(-1/2) = 0.6065; tau = 0.6 keeps it by 0.0065
    r = O.verify_sequence(target, None, [1, 1], None, 2.0, O.MODE_MARGIN, tau=0.6)
    assert r.accept_len == 2
    assert np.allclose(r.dists, math.exp(-0.5) - 0.6, atol=TOL)


def test_margin_distance_values():
    check_margin_distances()


def test_margin_ratio_scales_with_temperature():
    check_margin_temperature()


# --------------------------------------------------------------------------
# top-p cut
# --------------------------------------------------------------------------

def check_top_p_distances():
    # distinct levels 0.5, 0.3, 0.2; mass above each: 0, 0.5, 0.8. top_p 0.75
    # keeps the first two levels; the nearest level is 0.8 - 0.75 = 0.05 away
    keep, dist = O.truncation_keep(_logits([0.5, 0.3, 0.2]), 1.0, 0, 0.75)
    assert list(keep) == [True, True, False] and abs(dist - 0.05) <= TOL
    # top-k 3 first: (0.4, 0.3, 0.2)/0.9 -> masses above 0, 4/9, 7/9; top_p 0.7
    keep, dist = O.truncation_keep(_logits([0.4, 0.3, 0.2, 0.1]), 1.0, 3, 0.7)
    assert list(keep) == [True, True, False, False]
    assert abs(dist - (7.0 / 9.0 - 0.7)) <= TOL
    # a level of three tied tokens: masses above 0 and 0.4; top_p 0.5 keeps all
    keep, dist = O.truncation_keep(_logits([0.2, 0.4, 0.2, 0.2]), 1.0, 0, 0.5)
    assert keep.all() and abs(dist - 0.1) <= TOL
    # temperature first: ln(0.5, 0.3, 0.2) at T = 0.5 is (25, 9, 4)/38;
    # masses above 0, 25/38, 34/38; top_p 0.75 keeps two, 0.75 - 25/38 away
    keep, dist = O.truncation_keep(_logits([0.5, 0.3, 0.2]), 0.5, 0, 0.75)
    assert list(keep) == [True, True, False]
    assert abs(dist - (0.75 - 25.0 / 38.0)) <= TOL
    # top-p off: no cut, no decision
    keep, dist = O.truncation_keep(_logits([0.5, 0.3, 0.2]), 1.0, 2, 1.0)
    assert dist == math.inf


def test_top_p_distance_values():
    check_top_p_distances()


def test_top_p_distance_enters_the_sequence():
    """Each truncated row's top-p distance is one of the sequence's decisions."""
    t0 = _logits([0.5, 0.3, 0.2])               # top_p 0.75: 0.05
    t1 = _logits([0.6, 0.25, 0.15])             # masses above 0, .6, .85: 0.1
    d0 = _logits([0.45, 0.3, 0.25])             # masses above 0, .45, .75: 0.0 -> the cut
    r = O.verify_sequence(np.stack([t0, t1]), d0[None, :], [0], [0.5, 0.5], 1.0,
                          O.MODE_STOCHASTIC, top_p=0.75)
    tp_dists = sorted(r.dists[:3])
    assert abs(tp_dists[0] - 0.0) <= TOL
    assert abs(tp_dists[1] - 0.05) <= TOL and abs(tp_dists[2] - 0.1) <= TOL
    assert r.min_dist <= TOL


# --------------------------------------------------------------------------
# planted mistakes: the pins above must catch them
# --------------------------------------------------------------------------

@pytest.mark.parametrize("check", [check_inverse_cdf_distances, check_acceptance_distances,
                                   check_margin_distances, check_top_p_distances])
def test_pins_catch_distances_that_are_too_small(monkeypatch, check):
    """Every distance in the oracle is an absolute difference; halving them all
    (a distance that understates how far a decision was from flipping) must
    fail each pin."""
    monkeypatch.setattr(O, "abs", lambda v: 0.5 * builtins.abs(v), raising=False)
    with pytest.raises(AssertionError):
        check()


def test_pins_catch_a_margin_ratio_without_temperature(monkeypatch):
    real = O.softmax_t
    monkeypatch.setattr(O, "softmax_t", lambda x, T: real(x, 1.0))
    with pytest.raises(AssertionError):
        check_margin_temperature()
