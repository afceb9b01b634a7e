"""Pins for the oracle's walk-order reading: a position's rows are read only
once the walk reaches it, and
the walk reads nothing past its first rejection ([DVC] "Verify several
proposed tokens in one target pass": at the first rejection the correction is
drawn and later proposals are discarded; [SMB] "Seeing It in Code": the walk
stops at the first disagreement).

Pinned against things other than the walk-order code itself:

  * with every row and token usable, the result is the full reading's, field
    by field (the full reading is pinned elsewhere);
  * the boundary of what is read, by construction: the first rejection j is
    forced with the uniforms, then an unusable row or token is planted at
    position j + 1 (must not matter), at j (must invalidate) and below j (must
    invalidate); with every position kept, target row k_b must be usable and
    target rows past k_b are never read;
  * planted-mistake control: a walk that read one position further than its
    first rejection would invalidate the j + 1 case, and one that stopped a
    position early would keep the j case valid; both are caught above;
  * the greedy and margin walks the same way over target rows, with the
    argmax side output -1 past the stop, and a margin mismatch that clears
    tau keeping the walk going;
  * with truncation: the full reading's result on usable rows (each row read
    truncated as there), the same read boundary, the top-p parameter still
    checked, and only the rows read contributing top-p cut decisions (so the
    smallest decision distance is never below the full reading's).
"""

import math

import numpy as np
import pytest

from oracle import spec_oracle as O

S = O.MODE_STOCHASTIC


def _case(rng, V, K):
    target = rng.normal(0, 2.0, (K + 1, V))
    draft = 0.5 * target[:K] + rng.normal(0, 2.0, (K, V))
    q = [O.softmax_t(draft[i], 1.0) for i in range(K)]
    toks = np.array([rng.choice(V, p=q[i]) for i in range(K)])
    return target, draft, toks


def _forced(rng, V, K, j):
    """A case whose walk keeps positions < j and rejects j (j = K: keeps all):
    positions < j get u = 0 (kept whatever the ratio, since p(d) > 0), and
    position j gets a draft token with p < q and u just below 1."""
    while True:
        target, draft, toks = _case(rng, V, K)
        u = np.zeros(K + 1)
        u[K] = rng.random()
        if j == K:
            return target, draft, toks, u
        p = O.softmax_t(target[j], 1.0)
        q = O.softmax_t(draft[j], 1.0)
        cand = np.flatnonzero(p < 0.5 * q)
        if len(cand):
            toks[j] = cand[0]
            u[j] = 0.999999
            return target, draft, toks, u


def _same(a, b):
    assert a.valid == b.valid
    assert np.array_equal(a.tokens, b.tokens)
    assert a.accept_len == b.accept_len
    assert (a.z == b.z) or (math.isnan(a.z) and math.isnan(b.z))


@pytest.mark.parametrize("seed", range(6))
def test_walk_order_equals_full_reading_on_usable_rows(seed):
    rng = np.random.default_rng(400 + seed)
    V, K = 16, 5
    for _ in range(40):
        target, draft, toks = _case(rng, V, K)
        u = rng.random(K + 1)
        full = O.verify_sequence(target, draft, toks, u, 1.0, S)
        walk = O.verify_sequence(target, draft, toks, u, 1.0, S, walk_order=True)
        _same(full, walk)
        j = full.accept_len
        # p(d), q(d): the same where the walk read, NaN past the rejection
        last = j if j < K else K - 1
        assert np.array_equal(full.p_d[:last + 1], walk.p_d[:last + 1])
        assert np.array_equal(full.q_d[:last + 1], walk.q_d[:last + 1])
        assert np.all(np.isnan(walk.p_d[last + 1:])) and np.all(np.isnan(walk.q_d[last + 1:]))


BAD = {
    "nan": lambda row: row.__setitem__(3, np.nan),
    "+inf": lambda row: row.__setitem__(5, np.inf),
    "all -inf": lambda row: row.__setitem__(slice(None), -np.inf),
}


@pytest.mark.parametrize("kind", list(BAD))
@pytest.mark.parametrize("j", [0, 1, 3])
def test_read_boundary_is_the_first_rejection(kind, j):
    rng = np.random.default_rng(17 + j)
    V, K = 12, 5
    target, draft, toks, u = _forced(rng, V, K, j)
    ref = O.verify_sequence(target, draft, toks, u, 1.0, S, walk_order=True)
    assert ref.valid and ref.accept_len == j
    for which in ("target", "draft"):
        # past the rejection: not read
        t2, d2 = target.copy(), draft.copy()
        BAD[kind]((t2 if which == "target" else d2)[j + 1])
        r = O.verify_sequence(t2, d2, toks, u, 1.0, S, walk_order=True)
        _same(r, ref)
        assert not O.verify_sequence(t2, d2, toks, u, 1.0, S).valid   # the full reading reads it
        # at the rejection, and below it: read
        for i in range(j + 1):
            t3, d3 = target.copy(), draft.copy()
            BAD[kind]((t3 if which == "target" else d3)[i])
            r = O.verify_sequence(t3, d3, toks, u, 1.0, S, walk_order=True)
            assert not r.valid and r.accept_len == -1 and np.all(r.tokens == -1)


@pytest.mark.parametrize("j", [0, 2])
def test_token_out_of_range_counts_only_where_read(j):
    rng = np.random.default_rng(90 + j)
    V, K = 10, 4
    target, draft, toks, u = _forced(rng, V, K, j)
    ref = O.verify_sequence(target, draft, toks, u, 1.0, S, walk_order=True)
    t2 = toks.copy()
    t2[j + 1] = V            # past the rejection
    _same(O.verify_sequence(target, draft, t2, u, 1.0, S, walk_order=True), ref)
    t3 = toks.copy()
    t3[j] = -1               # at the rejection
    assert not O.verify_sequence(target, draft, t3, u, 1.0, S, walk_order=True).valid


def test_all_kept_reads_the_bonus_row_and_nothing_past_k_b():
    rng = np.random.default_rng(5)
    V, K = 12, 5
    target, draft, toks, u = _forced(rng, V, K, K)
    ref = O.verify_sequence(target, draft, toks, u, 1.0, S, walk_order=True)
    assert ref.valid and ref.accept_len == K and ref.tokens[K] >= 0
    t2 = target.copy()
    t2[K, 2] = np.nan
    assert not O.verify_sequence(t2, draft, toks, u, 1.0, S, walk_order=True).valid
    # k_b = 3: bonus from target row 3; rows 4.. of either kind are never read
    kb = 3
    r = O.verify_sequence(target, draft, toks, u, 1.0, S, draft_len=kb, walk_order=True)
    t3, d3, tk3 = target.copy(), draft.copy(), toks.copy()
    t3[kb + 1:] = np.nan
    d3[kb:] = np.nan
    tk3[kb:] = -5
    r3 = O.verify_sequence(t3, d3, tk3, u, 1.0, S, draft_len=kb, walk_order=True)
    _same(r3, r)
    assert r3.valid and r3.accept_len == kb


def test_stops_cut_the_emission_not_the_reading():
    """An end-of-sequence draft before the first rejection ends the emission
    there, yet the walk still reads up to the rejection: a bad row at the
    rejection invalidates the sequence, one past it does not."""
    rng = np.random.default_rng(71)
    V, K, j = 12, 5, 3
    target, draft, toks, u = _forced(rng, V, K, j)
    eos = int(toks[1])
    if eos in toks[:1]:
        pytest.skip("needs a first eos at position 1")
    r = O.verify_sequence(target, draft, toks, u, 1.0, S, eos=eos, walk_order=True)
    assert r.valid and r.accept_len == 2 and r.tokens[2] == -1
    d2 = draft.copy()
    d2[j] = np.nan
    assert not O.verify_sequence(target, d2, toks, u, 1.0, S, eos=eos, walk_order=True).valid
    d3 = draft.copy()
    d3[j + 1] = np.nan
    _same(O.verify_sequence(target, d3, toks, u, 1.0, S, eos=eos, walk_order=True), r)


TRUNCS = ((5, 1.0), (0, 0.9), (3, 0.8), (1, 1.0), (0, 0.5))


def _forced_trunc(rng, V, K, j, tk, tp):
    """As _forced, under truncation (top_k tk, top_p tp): positions < j draft
    their target row's argmax (inside any truncation, so p > 0 and u = 0
    keeps them); position j drafts a token the truncated draft row keeps
    with truncated p below half its truncated q, and u just below 1."""
    while True:
        target, draft, toks = _case(rng, V, K)
        u = np.zeros(K + 1)
        u[K] = rng.random()
        toks[:j] = np.argmax(target[:j], axis=1)
        if j == K:
            return target, draft, toks, u
        p = O.truncated_softmax(target[j], 1.0, tk, tp)[0]
        q = O.truncated_softmax(draft[j], 1.0, tk, tp)[0]
        cand = np.flatnonzero((q > 0) & (p < 0.5 * q))
        if len(cand):
            toks[j] = cand[0]
            u[j] = 0.999999
            return target, draft, toks, u


@pytest.mark.parametrize("tk,tp", TRUNCS)
def test_truncated_walk_equals_full_reading_on_usable_rows(tk, tp):
    rng = np.random.default_rng(800 + tk + int(10 * tp))
    V, K = 14, 5
    for _ in range(30):
        target, draft, toks = _case(rng, V, K)
        u = rng.random(K + 1)
        full = O.verify_sequence(target, draft, toks, u, 1.0, S, top_k=tk, top_p=tp)
        walk = O.verify_sequence(target, draft, toks, u, 1.0, S, top_k=tk, top_p=tp,
                                 walk_order=True)
        _same(full, walk)
        j = full.accept_len
        last = j if j < K else K - 1
        assert np.array_equal(full.p_d[:last + 1], walk.p_d[:last + 1])
        assert np.array_equal(full.q_d[:last + 1], walk.q_d[:last + 1])
        assert np.all(np.isnan(walk.p_d[last + 1:])) and np.all(np.isnan(walk.q_d[last + 1:]))
        # the walk's decisions are a subset of the full reading's
        assert walk.min_dist >= full.min_dist


@pytest.mark.parametrize("tk,tp", ((5, 1.0), (0, 0.9)))
@pytest.mark.parametrize("j", [0, 2])
def test_truncated_read_boundary(tk, tp, j):
    rng = np.random.default_rng(60 + j + tk)
    V, K = 12, 5
    target, draft, toks, u = _forced_trunc(rng, V, K, j, tk, tp)
    ref = O.verify_sequence(target, draft, toks, u, 1.0, S, top_k=tk, top_p=tp, walk_order=True)
    assert ref.valid and ref.accept_len == j
    for which in ("target", "draft"):
        t2, d2 = target.copy(), draft.copy()
        (t2 if which == "target" else d2)[j + 1, 1] = np.nan      # past it: not read
        _same(O.verify_sequence(t2, d2, toks, u, 1.0, S, top_k=tk, top_p=tp, walk_order=True),
              ref)
        assert not O.verify_sequence(t2, d2, toks, u, 1.0, S, top_k=tk, top_p=tp).valid
        t3, d3 = target.copy(), draft.copy()
        (t3 if which == "target" else d3)[j, 1] = np.inf          # at it: read
        assert not O.verify_sequence(t3, d3, toks, u, 1.0, S, top_k=tk, top_p=tp,
                                     walk_order=True).valid


def test_truncated_walk_still_checks_top_p():
    rng = np.random.default_rng(8)
    V, K = 12, 4
    target, draft, toks = _case(rng, V, K)
    u = rng.random(K + 1)
    for tp in (0.0, -1.0, float("nan")):
        r = O.verify_sequence(target, draft, toks, u, 1.0, S, top_p=tp, walk_order=True)
        assert not r.valid and r.accept_len == -1
    # greedy ignores the truncation parameters, as in the full reading
    g = O.verify_sequence(target, None, toks, None, 1.0, O.MODE_GREEDY, top_p=0.0,
                          walk_order=True)
    assert g.valid


def test_truncated_walk_cut_decisions_only_from_rows_read():
    """A top-p cut close to moving in a row past the first rejection is not a
    decision of the walk-order reading (it is one of the full reading)."""
    rng = np.random.default_rng(23)
    V, K, j = 12, 4, 0
    tp = 0.9
    target, draft, toks, u = _forced_trunc(rng, V, K, j, 0, tp)
    # put target row j + 1's top-p cut exactly on a level boundary: two
    # levels whose masses after renormalisation are tp and 1 - tp
    t2 = target.copy()
    row = np.full(V, -1e9)
    row[0] = math.log(tp)
    row[1] = math.log(1.0 - tp)
    t2[j + 1] = row
    full = O.verify_sequence(t2, draft, toks, u, 1.0, S, top_p=tp)
    walk = O.verify_sequence(t2, draft, toks, u, 1.0, S, top_p=tp, walk_order=True)
    assert walk.valid and walk.accept_len == j and full.valid and full.accept_len == j
    assert full.min_dist < 1e-9
    assert walk.min_dist > 1e-9
    # the same cut in a row the walk reads (position 0, kept, before a
    # rejection at 1) is a decision of both readings
    target, draft, toks, u = _forced_trunc(rng, V, K, 1, 0, tp)
    t3 = target.copy()
    t3[0] = row
    toks[0] = 0
    full = O.verify_sequence(t3, draft, toks, u, 1.0, S, top_p=tp)
    walk = O.verify_sequence(t3, draft, toks, u, 1.0, S, top_p=tp, walk_order=True)
    assert walk.valid and walk.accept_len == 1 and full.accept_len == 1
    assert walk.min_dist < 1e-9 and full.min_dist < 1e-9


# greedy and margin walks: target rows only, the walk stops at the first
# position that fails its rule

def _argmax_case(rng, V, K, t, mode, tau=0.3):
    """Tokens that keep positions < t and fail position t (t = K: keep all):
    the row argmax below t, at t a token whose margin ratio is below tau."""
    target = rng.normal(0, 2.0, (K + 1, V))
    toks = np.argmax(target[:K], axis=1).astype(np.int64)
    if t < K:
        p = O.softmax_t(target[t], 1.0)
        r = p / p.max()
        cand = np.flatnonzero(r < 0.5 * tau)
        toks[t] = cand[0]
    return target, toks


@pytest.mark.parametrize("mode", [O.MODE_GREEDY, O.MODE_MARGIN])
@pytest.mark.parametrize("t", [0, 2, 4])
def test_argmax_walk_read_boundary(mode, t):
    rng = np.random.default_rng(300 + t + 10 * mode)
    V, K = 12, 4
    target, toks = _argmax_case(rng, V, K, t, mode)
    full = O.verify_sequence(target, None, toks, None, 1.0, mode, tau=0.3)
    ref = O.verify_sequence(target, None, toks, None, 1.0, mode, tau=0.3, walk_order=True)
    _same(full, ref)
    assert ref.valid and ref.accept_len == t
    # the argmax side output: rows the walk reads (0..t), -1 past them
    assert np.array_equal(ref.argmax[:t + 1], full.argmax[:t + 1])
    assert np.all(ref.argmax[t + 1:] == -1)
    if t + 1 <= K:
        t2 = target.copy()
        t2[t + 1, 1] = np.nan                    # past the stop: not read
        _same(O.verify_sequence(t2, None, toks, None, 1.0, mode, tau=0.3, walk_order=True),
              ref)
        assert not O.verify_sequence(t2, None, toks, None, 1.0, mode, tau=0.3).valid
        tk2 = toks.copy()
        if t + 1 < K:
            tk2[t + 1] = V + 1                   # a token past the stop: not read
            _same(O.verify_sequence(target, None, tk2, None, 1.0, mode, tau=0.3,
                                    walk_order=True), ref)
    for i in range(t + 1):                       # at and below the stop: read
        t3 = target.copy()
        t3[i, :] = -np.inf
        assert not O.verify_sequence(t3, None, toks, None, 1.0, mode, tau=0.3,
                                     walk_order=True).valid


def test_margin_walk_goes_on_past_a_kept_mismatch():
    """A drafted token that is not the argmax but clears the margin keeps the
    walk going: the next row is read (a bad row there invalidates)."""
    rng = np.random.default_rng(41)
    V, K = 12, 4
    target = rng.normal(0, 0.3, (K + 1, V))    # flat rows: every ratio near 1
    toks = np.argmax(target[:K], axis=1).astype(np.int64)
    toks[0] = int(np.argsort(target[0])[-2])  # second largest: ratio > 0.3
    r = O.verify_sequence(target, None, toks, None, 1.0, O.MODE_MARGIN, tau=0.3,
                          walk_order=True)
    assert r.valid and r.accept_len == K
    t2 = target.copy()
    t2[1, 3] = np.inf
    assert not O.verify_sequence(t2, None, toks, None, 1.0, O.MODE_MARGIN, tau=0.3,
                                 walk_order=True).valid
    assert O.verify_sequence(t2, None, toks, None, 1.0, O.MODE_GREEDY,
                             walk_order=True).valid   # greedy stops at position 0


@pytest.mark.parametrize("mode", [O.MODE_GREEDY, O.MODE_MARGIN])
def test_argmax_walk_equals_full_reading_on_usable_rows(mode):
    rng = np.random.default_rng(500 + mode)
    V, K = 16, 5
    for _ in range(60):
        target = rng.normal(0, 2.0, (K + 1, V))
        toks = np.argmax(target[:K] + rng.normal(0, 1.5, (K, V)), axis=1)
        kb = int(rng.integers(0, K + 1))
        a = O.verify_sequence(target, None, toks, None, 1.0, mode, tau=0.3, draft_len=kb)
        b = O.verify_sequence(target, None, toks, None, 1.0, mode, tau=0.3, draft_len=kb,
                              walk_order=True)
        _same(a, b)
        stop = a.accept_len if a.accept_len < kb else kb
        assert np.array_equal(a.argmax[:stop + 1], b.argmax[:stop + 1])
        assert np.all(b.argmax[stop + 1:] == -1)


def test_batch_threads_the_reading():
    rng = np.random.default_rng(12)
    B, V, K = 6, 10, 4
    cases = [_forced(rng, V, K, 0) for _ in range(B)]
    tg = np.stack([c[0] for c in cases])
    dr = np.stack([c[1] for c in cases])
    tk = np.stack([c[2] for c in cases])
    uu = np.stack([c[3] for c in cases])
    dr[:, 2, :] = np.nan              # past every sequence's rejection at 0
    full = O.verify_batch(tg, dr, tk, uu, 1.0, S)
    walk = O.verify_batch(tg, dr, tk, uu, 1.0, S, walk_order=True)
    assert full.invalid == B and walk.invalid == 0
    assert np.all(walk.accept_len == 0) and walk.hist[0] == B
