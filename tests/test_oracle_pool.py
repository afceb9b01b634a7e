"""The process-pool runner of the oracle gives exactly what one sequential
verify_batch call gives: same tokens, lengths, side outputs, histogram,
decision count and EMA state, whatever the chunking."""

import numpy as np

from oracle import spec_oracle as O
from oracle.pool import OraclePool


def _batch(B, K, V, seed):
    rng = np.random.default_rng(seed)
    t = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
    d = (0.7 * t[:, :K] + rng.normal(0, 1.5, (B, K, V))).astype(np.float32)
    tok = np.stack([[rng.choice(V, p=O.softmax_t(d[b, i], 0.9)) for i in range(K)]
                    for b in range(B)]).astype(np.int32)
    u = (rng.integers(0, 1 << 24, (B, K + 1)) / float(1 << 24)).astype(np.float32)
    return t, d, tok, u


def _same(a, b):
    for k in ("tokens", "accept_len", "argmax"):
        assert np.array_equal(getattr(a, k), getattr(b, k)), k
    for k in ("p_d", "q_d", "z", "min_dist"):
        assert np.array_equal(getattr(a, k), getattr(b, k), equal_nan=True), k
    assert np.array_equal(a.hist, b.hist)
    assert (a.n_decisions, a.invalid, a.zero_q_accepts, a.z0_fallbacks) == \
        (b.n_decisions, b.invalid, b.zero_q_accepts, b.z0_fallbacks)


def test_pool_matches_sequential_oracle():
    B, K, V = 23, 3, 97
    t, d, tok, u = _batch(B, K, V, 5)
    rng = np.random.default_rng(6)
    kb = rng.integers(0, K + 1, B)
    mx = rng.integers(1, K + 2, B)
    tk = rng.choice([0, 5, 40], B).astype(np.int32)
    tp = rng.choice([1.0, 0.8], B).astype(np.float32)
    rows = np.sort(rng.choice(B, 17, replace=False))
    shapes = dict(target=(t.shape, np.float32), draft=(d.shape, np.float32),
                  tokens=(tok.shape, np.int32), uniforms=(u.shape, np.float32))
    with OraclePool(shapes, nproc=2) as pool:
        pool.load(target=t, draft=d, tokens=tok, uniforms=u)
        for step in range(2):
            e_seq, e_par = O.EmaState(B, 0.9), O.EmaState(B, 0.9)
            for e in (e_seq, e_par):
                e.ema[:] = np.linspace(0, 1, B)
                e.steps[:] = np.arange(B) % 3
            ref = O.verify_batch(t, d, tok, u, 0.9, O.MODE_STOCHASTIC, ema=e_seq, rows=rows,
                                 eos=7, draft_len=kb, max_emit=mx, top_k=tk, top_p=tp)
            got = pool.verify(rows, 0.9, O.MODE_STOCHASTIC, ema=e_par, eos=7, draft_len=kb,
                              max_emit=mx, top_k=tk, top_p=tp, chunk=3 + step)
            _same(ref, got)
            assert np.array_equal(e_seq.ema, e_par.ema) and np.array_equal(e_seq.steps,
                                                                           e_par.steps)
        # greedy reads target rows only
        ref = O.verify_batch(t, None, tok, None, 1.0, O.MODE_GREEDY)
        _same(ref, pool.verify(np.arange(B), 1.0, O.MODE_GREEDY))
