"""GPU parity of the walk-order reading (spec_verify_set_walk_order) against
the oracle's walk_order reading: the streaming pass runs in stages of
positions and a stage's workgroups read their rows only when the walk of
their sequence reaches them.

Checked on both stochastic finish paths (one workgroup per sequence, and the
scan / tile / pick kernels), bf16 and fp32 rows, whole batches (c1, c2, c3),
against the full reading of the same inputs (every output equal, p(d) and
q(d) NaN past the first rejection), with unusable rows and tokens planted
past, at and below each sequence's first rejection and in the bonus row, and
with the stopping rules. The greedy and margin walks (target rows only: the
argmax pass over row 0, then the rows of the sequences that keep position 0)
are checked the same way, with the per-row argmax side output -1 and the
margin ratio NaN past the row the walk stops at. Truncated bf16 calls read
in walk order through both truncation passes (mixed per-sequence top-k /
top-p, rows handed to the full-histogram pass, planted rows, stopping rules,
the c3 shape), and truncated fp32 calls through their three passes (c1, fp32
rows of the c2 shape, planted rows, a c5 sample).
"""

import numpy as np
import pytest
import torch

from oracle import spec_oracle as O
from tests.parity import check_invariants, compare, oracle_for
from workloads import CONFIGS, make_inputs, to_host_f64, window_edge_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


@pytest.fixture(scope="module")
def sv():
    import speculative_decoding_verification_temp_amd as pkg
    pkg.load_library()
    torch.cuda.set_device(DEV)
    return pkg


def _run(sv, x, cfg, walk, stops=None, mode="stochastic", tau=0.3, trunc=None):
    v = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, x["target"].dtype, ema_decay=0.9)
    aux = v.enable_aux()
    if trunc is not None:
        tk, tp = trunc
        v.set_truncation(torch.as_tensor(tk, device=DEV).contiguous(),
                         torch.as_tensor(tp, device=DEV).contiguous())
    if stops is not None:
        eos, kb, mx = stops
        v.set_stops(eos, None if kb is None else torch.as_tensor(kb, device=DEV).contiguous(),
                    None if mx is None else torch.as_tensor(mx, device=DEV).contiguous())
    v.set_walk_order(walk)
    if mode == "stochastic":
        tok, alen, hist = v.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"],
                                   "stochastic")
    else:
        tok, alen, hist = v.verify(x["target"], None, x["tokens"], None, x["T"], mode, tau=tau)
    torch.cuda.synchronize()
    out = (tok.clone(), alen.clone(), hist.clone(), {k: t.clone() for k, t in aux.items()})
    v.close()
    return out


def _pq_pattern(aux, ref, rows, label):
    """p(d), q(d): NaN exactly where the oracle's are (walk-order reading:
    past the first rejection and in invalid sequences)."""
    for key, r in (("p_d", ref.p_d), ("q_d", ref.q_d)):
        g = aux[key].cpu().numpy()[rows]
        assert np.array_equal(np.isnan(g), np.isnan(r)), f"{label}: {key} NaN pattern"


def _same_outputs(a, b):
    """Tokens, lengths and histogram equal; Z close (the staged streaming pass
    may split rows into other segments, whose float32 group sums round
    differently: about 1e-8 relative in a normaliser)."""
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    assert torch.allclose(a[3]["z"], b[3]["z"], rtol=1e-9, atol=1e-15)


@pytest.mark.parametrize("path", ["finish", "multikernel"])
@pytest.mark.parametrize("name", ["c1", "c2"])
def test_walk_matches_oracle_and_full_reading(sv, monkeypatch, name, path):
    monkeypatch.setenv("SPEC_VERIFY_FINISH_SEQ", "1" if path == "finish" else "0")
    cfg = CONFIGS[name]
    x = make_inputs(cfg, 3, DEV)
    rows = np.arange(cfg.B)
    full = _run(sv, x, cfg, False)
    walk = _run(sv, x, cfg, True)
    ref = oracle_for(x, rows, "stochastic", walk=True)
    compare(rows, ref, walk[0], walk[1], "stochastic", walk[3], f"{name}/{path}/walk")
    check_invariants(walk[0], walk[1], walk[2], x["tokens"], cfg.V, cfg.K)
    _pq_pattern(walk[3], ref, rows, f"{name}/{path}")
    _same_outputs(walk, full)
    # where the walk read, p(d) and q(d) are those of the full reading
    for key in ("p_d", "q_d"):
        g, f = walk[3][key].cpu().numpy(), full[3][key].cpu().numpy()
        read = ~np.isnan(g)
        assert np.allclose(g[read], f[read], rtol=1e-6, atol=0)


def test_walk_c3_whole_batch(sv):
    cfg = CONFIGS["c3"]
    x = make_inputs(cfg, 0, DEV)
    rows = np.arange(cfg.B)
    full = _run(sv, x, cfg, False)
    walk = _run(sv, x, cfg, True)
    ref = oracle_for(x, rows, "stochastic", walk=True)
    compare(rows, ref, walk[0], walk[1], "stochastic", walk[3], "c3/walk")
    _pq_pattern(walk[3], ref, rows, "c3")
    _same_outputs(walk, full)


def _plant(x, cfg, j, seed):
    """Unusable rows and tokens placed by each sequence's first rejection j
    (from the full reading): past it (never read by the walk), at it and below
    it (read), and in the bonus row of sequences that keep every draft."""
    rng = np.random.default_rng(seed)
    K, V = cfg.K, cfg.V
    tg, dr, tk = x["target"].clone(), x["draft"].clone(), x["tokens"].clone()
    kinds = ("nan", "inf", "allneg")

    def spoil(row):
        k = kinds[rng.integers(0, 3)]
        if k == "nan":
            row[int(rng.integers(0, V))] = float("nan")
        elif k == "inf":
            row[int(rng.integers(0, V))] = float("inf")
        else:
            row.fill_(float("-inf"))

    for b in range(cfg.B):
        jb = int(j[b])
        case = b % 5
        if case == 0 and jb + 1 < K:             # past the rejection: the draft row
            spoil(dr[b, jb + 1])
        elif case == 1 and jb + 1 <= K and jb < K:   # past it: the target row
            spoil(tg[b, jb + 1])
        elif case == 2 and jb < K:               # at the rejection
            spoil(dr[b, jb] if rng.random() < 0.5 else tg[b, jb])
        elif case == 3 and jb > 0:               # below it
            spoil(tg[b, jb - 1] if rng.random() < 0.5 else dr[b, jb - 1])
        elif case == 4 and jb + 1 < K:           # a drafted token out of range past it
            tk[b, jb + 1] = V + 3
        if jb == K:                              # every draft kept: the bonus row
            spoil(tg[b, K])
    return dict(x, target=tg, draft=dr, tokens=tk)


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_walk_unusable_rows_count_only_where_read(sv, name):
    cfg = CONFIGS[name].scaled(B=CONFIGS[name].B * 4) if name == "c1" else CONFIGS[name]
    x = make_inputs(cfg, 8, DEV)
    j = _run(sv, x, cfg, False)[1].cpu().numpy()
    assert np.all(j >= 0)
    y = _plant(x, cfg, j, 21)
    rows = np.arange(cfg.B)
    walk = _run(sv, y, cfg, True)
    full = _run(sv, y, cfg, False)
    ref = oracle_for(y, rows, "stochastic", walk=True)
    ref_full = oracle_for(y, rows, "stochastic")
    compare(rows, ref, walk[0], walk[1], "stochastic", walk[3], f"{name}/walk/planted")
    compare(rows, ref_full, full[0], full[1], "stochastic", full[3], f"{name}/full/planted")
    _pq_pattern(walk[3], ref, rows, f"{name}/planted")
    a_walk, a_full = walk[1].cpu().numpy(), full[1].cpu().numpy()
    # the walk-order reading keeps valid every sequence whose spoiled row or
    # token lies past its rejection, and only those
    assert (a_walk < 0).sum() < (a_full < 0).sum()
    assert np.array_equal(a_walk < 0, ref.accept_len < 0)
    assert np.array_equal(a_full < 0, ref_full.accept_len < 0)


def test_walk_with_stopping_rules(sv):
    cfg = CONFIGS["c2"]
    x = make_inputs(cfg, 11, DEV)
    rng = np.random.default_rng(5)
    toks = x["tokens"].cpu().numpy()
    eos = int(np.bincount(toks.ravel()).argmax())
    kb = rng.integers(0, cfg.K + 1, cfg.B).astype(np.int32)
    mx = rng.integers(1, cfg.K + 3, cfg.B).astype(np.int32)
    kb[1], kb[2], mx[3] = -1, cfg.K + 1, 0
    stops = (eos, kb, mx)
    rows = np.arange(cfg.B)
    walk = _run(sv, x, cfg, True, stops)
    full = _run(sv, x, cfg, False, stops)
    ref = oracle_for(x, rows, "stochastic", stops=stops, walk=True)
    compare(rows, ref, walk[0], walk[1], "stochastic", walk[3], "c2/walk/stops")
    _pq_pattern(walk[3], ref, rows, "c2/stops")
    _same_outputs(walk, full)


# --------------------------------------------------------------------------
# greedy and margin
# --------------------------------------------------------------------------

TAU = 0.3


def _argmax_checks(res, ref, rows, mode, label):
    """Side outputs of the greedy and margin walks: the argmax -1 exactly
    where the oracle's is on valid sequences (rows past the stop are not
    read), the margin ratio NaN exactly where the oracle's is."""
    valid = ref.accept_len >= 0
    ga = res[3]["argmax"].cpu().numpy()[rows]
    assert np.array_equal(ga[valid], ref.argmax[valid]), f"{label}: argmax"
    if mode == "margin":
        gp = res[3]["p_d"].cpu().numpy()[rows]
        assert np.array_equal(np.isnan(gp), np.isnan(ref.p_d)), f"{label}: ratio NaN pattern"


def _same_argmax_outputs(walk, full, mode):
    """Tokens, lengths and histogram equal; where the walk read a row, its
    argmax and margin ratio are those of the full reading (the same maxima:
    no rounding is involved)."""
    for a, b in zip(walk[:3], full[:3]):
        assert torch.equal(a, b)
    ok = walk[1].cpu().numpy() >= 0
    ga, fa = walk[3]["argmax"].cpu().numpy()[ok], full[3]["argmax"].cpu().numpy()[ok]
    read = ga >= 0
    assert np.array_equal(ga[read], fa[read])
    if mode == "margin":
        g, f = walk[3]["p_d"].cpu().numpy(), full[3]["p_d"].cpu().numpy()
        read = ~np.isnan(g)
        assert np.array_equal(g[read], f[read])


@pytest.mark.parametrize("mode", ["greedy", "margin"])
@pytest.mark.parametrize("name", ["c1", "c2", "c2odd"])
def test_walk_argmax_matches_oracle_and_full_reading(sv, name, mode):
    # c2odd: V not a multiple of the vector width (the one-element load path)
    cfg = CONFIGS["c2"].scaled(V=32003) if name == "c2odd" else CONFIGS[name]
    x = make_inputs(cfg, 4, DEV, "greedy")
    rows = np.arange(cfg.B)
    full = _run(sv, x, cfg, False, mode=mode, tau=TAU)
    walk = _run(sv, x, cfg, True, mode=mode, tau=TAU)
    ref = oracle_for(x, rows, mode, tau=TAU, walk=True)
    compare(rows, ref, walk[0], walk[1], mode, walk[3], f"{name}/{mode}/walk")
    check_invariants(walk[0], walk[1], walk[2], x["tokens"], cfg.V, cfg.K)
    _argmax_checks(walk, ref, rows, mode, f"{name}/{mode}")
    _same_argmax_outputs(walk, full, mode)
    # the walk stops at position 0 in some sequences and goes past it in others
    a = walk[1].cpu().numpy()
    if cfg.B >= 16:
        assert (a == 0).any() and (a >= 1).any()


@pytest.mark.parametrize("name,mode", [("c3", "greedy"), ("c4", "margin"), ("c4", "greedy")])
def test_walk_argmax_whole_batch(sv, name, mode):
    cfg = CONFIGS[name]
    x = make_inputs(cfg, 0, DEV, "greedy")
    rows = np.arange(cfg.B)
    full = _run(sv, x, cfg, False, mode=mode, tau=cfg.tau or TAU)
    walk = _run(sv, x, cfg, True, mode=mode, tau=cfg.tau or TAU)
    ref = oracle_for(x, rows, mode, tau=cfg.tau or TAU, walk=True)
    compare(rows, ref, walk[0], walk[1], mode, walk[3], f"{name}/{mode}/walk")
    _argmax_checks(walk, ref, rows, mode, f"{name}/{mode}")
    _same_argmax_outputs(walk, full, mode)


def _plant_target(x, cfg, j, seed):
    """Unusable target rows and tokens placed by each sequence's stop j
    (from the full reading): past it (never read by the walk), at it and below
    it (read), and in the last row of sequences that keep every draft."""
    rng = np.random.default_rng(seed)
    K, V = cfg.K, cfg.V
    tg, tk = x["target"].clone(), x["tokens"].clone()

    def spoil(row):
        k = int(rng.integers(0, 3))
        if k == 0:
            row[int(rng.integers(0, V))] = float("nan")
        elif k == 1:
            row[int(rng.integers(0, V))] = float("inf")
        else:
            row.fill_(float("-inf"))

    for b in range(cfg.B):
        jb = int(j[b])
        case = b % 4
        if case == 0 and jb < K:                 # past the stop: the next row
            spoil(tg[b, jb + 1])
        elif case == 1 and jb < K:               # at the stop
            spoil(tg[b, jb])
        elif case == 2 and jb > 0:               # below it
            spoil(tg[b, jb - 1])
        elif case == 3 and jb + 1 < K:           # a drafted token out of range past it
            tk[b, jb + 1] = -2
        if jb == K:                              # every draft kept: the last row
            spoil(tg[b, K])
    return dict(x, target=tg, tokens=tk)


@pytest.mark.parametrize("mode", ["greedy", "margin"])
@pytest.mark.parametrize("name", ["c1", "c2"])
def test_walk_argmax_unusable_rows_count_only_where_read(sv, name, mode):
    cfg = CONFIGS[name].scaled(B=CONFIGS[name].B * 8) if name == "c1" else CONFIGS[name]
    x = make_inputs(cfg, 9, DEV, "greedy")
    j = _run(sv, x, cfg, False, mode=mode)[1].cpu().numpy()
    assert np.all(j >= 0)
    y = _plant_target(x, cfg, j, 23)
    rows = np.arange(cfg.B)
    walk = _run(sv, y, cfg, True, mode=mode)
    full = _run(sv, y, cfg, False, mode=mode)
    ref = oracle_for(y, rows, mode, tau=TAU, walk=True)
    ref_full = oracle_for(y, rows, mode, tau=TAU)
    compare(rows, ref, walk[0], walk[1], mode, walk[3], f"{name}/{mode}/walk/planted")
    compare(rows, ref_full, full[0], full[1], mode, full[3], f"{name}/{mode}/full/planted")
    _argmax_checks(walk, ref, rows, mode, f"{name}/{mode}/planted")
    a_walk, a_full = walk[1].cpu().numpy(), full[1].cpu().numpy()
    assert (a_walk < 0).sum() < (a_full < 0).sum()
    assert np.array_equal(a_walk < 0, ref.accept_len < 0)
    assert np.array_equal(a_full < 0, ref_full.accept_len < 0)


@pytest.mark.parametrize("mode", ["greedy", "margin"])
def test_walk_argmax_with_stopping_rules(sv, mode):
    cfg = CONFIGS["c2"]
    x = make_inputs(cfg, 12, DEV, "greedy")
    rng = np.random.default_rng(6)
    toks = x["tokens"].cpu().numpy()
    eos = int(np.bincount(toks.ravel()).argmax())
    kb = rng.integers(0, cfg.K + 1, cfg.B).astype(np.int32)
    mx = rng.integers(1, cfg.K + 3, cfg.B).astype(np.int32)
    kb[1], kb[2], mx[3] = -1, cfg.K + 1, 0
    stops = (eos, kb, mx)
    rows = np.arange(cfg.B)
    walk = _run(sv, x, cfg, True, stops, mode=mode)
    full = _run(sv, x, cfg, False, stops, mode=mode)
    ref = oracle_for(x, rows, mode, tau=TAU, stops=stops, walk=True)
    compare(rows, ref, walk[0], walk[1], mode, walk[3], f"c2/{mode}/walk/stops")
    _argmax_checks(walk, ref, rows, mode, f"c2/{mode}/stops")
    _same_argmax_outputs(walk, full, mode)


# --------------------------------------------------------------------------
# truncated calls
# --------------------------------------------------------------------------

def _trunc_settings(B, V, seed, invalid=False):
    rng = np.random.default_rng(seed)
    tk = rng.choice([0, 1, 2, 20, 50, 1000, V, V + 7, -3], B).astype(np.int32)
    tp = rng.choice([1.0, 0.5, 0.8, 0.9, 0.95, 0.99, 1.5], B).astype(np.float32)
    if invalid:
        tp[1], tp[2] = 0.0, np.nan
    return tk, tp


def _trunc_drafts(x, T, tk, tp, seed):
    """Drafted tokens from each sequence's truncated draft distribution."""
    rng = np.random.default_rng(seed)
    d = to_host_f64(x["draft"])
    B, K, _ = d.shape
    toks = np.zeros((B, K), dtype=np.int32)
    for b in range(B):
        p = float(tp[b]) if np.isfinite(tp[b]) and tp[b] > 0 else 1.0
        for i in range(K):
            q, _ = O.truncated_softmax(d[b, i], T, int(tk[b]), p)
            toks[b, i] = rng.choice(q.size, p=q)
    return dict(x, tokens=torch.as_tensor(toks, device=DEV).contiguous())


def _same_exact(a, b):
    """Tokens, lengths, histogram and Z equal (the truncation passes give
    each row the same partial whichever launch reads it)."""
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    za, zb = a[3]["z"], b[3]["z"]
    assert torch.equal(torch.nan_to_num(za, nan=-9.0), torch.nan_to_num(zb, nan=-9.0))


def _trunc_case(sv, x, cfg, trunc, label, stops=None):
    rows = np.arange(cfg.B)
    walk = _run(sv, x, cfg, True, stops, trunc=trunc)
    full = _run(sv, x, cfg, False, stops, trunc=trunc)
    ref = oracle_for(x, rows, "stochastic", stops=stops, trunc=trunc, walk=True)
    compare(rows, ref, walk[0], walk[1], "stochastic", walk[3], f"{label}/walk")
    _pq_pattern(walk[3], ref, rows, label)
    _same_exact(walk, full)
    return walk, full, ref


def test_walk_truncated_mixed_settings(sv):
    cfg = CONFIGS["c2"]
    x = make_inputs(cfg, 13, DEV)
    tk, tp = _trunc_settings(cfg.B, cfg.V, 14, invalid=True)
    x = _trunc_drafts(x, cfg.T, tk, tp, 15)
    walk, full, ref = _trunc_case(sv, x, cfg, (tk, tp), "c2/trunc")
    a = walk[1].cpu().numpy()
    assert a[1] == -1 and a[2] == -1          # top_p = 0 and NaN
    assert (a == 0).any() and (a >= 1).any()


def test_walk_truncated_rows_handed_over(sv):
    """Rows with values outside the window pass's bins go through the
    full-histogram pass, in both stages of the walk."""
    cfg = CONFIGS["c2"].scaled(B=32)
    x = window_edge_inputs(cfg, 4, DEV)
    tk, tp = _trunc_settings(cfg.B, cfg.V, 5)
    x = _trunc_drafts(x, cfg.T, tk, tp, 6)
    _trunc_case(sv, x, cfg, (tk, tp), "c2/trunc/window edges")


def test_walk_truncated_unusable_rows_count_only_where_read(sv):
    cfg = CONFIGS["c2"]
    x = make_inputs(cfg, 16, DEV)
    tk, tp = _trunc_settings(cfg.B, cfg.V, 17)
    x = _trunc_drafts(x, cfg.T, tk, tp, 18)
    trunc = (tk, tp)
    j = _run(sv, x, cfg, False, trunc=trunc)[1].cpu().numpy()
    assert np.all(j >= 0)
    y = _plant(x, cfg, j, 22)
    rows = np.arange(cfg.B)
    walk = _run(sv, y, cfg, True, trunc=trunc)
    full = _run(sv, y, cfg, False, trunc=trunc)
    ref = oracle_for(y, rows, "stochastic", trunc=trunc, walk=True)
    ref_full = oracle_for(y, rows, "stochastic", trunc=trunc)
    compare(rows, ref, walk[0], walk[1], "stochastic", walk[3], "c2/trunc/walk/planted")
    compare(rows, ref_full, full[0], full[1], "stochastic", full[3], "c2/trunc/full/planted")
    _pq_pattern(walk[3], ref, rows, "c2/trunc/planted")
    a_walk, a_full = walk[1].cpu().numpy(), full[1].cpu().numpy()
    assert (a_walk < 0).sum() < (a_full < 0).sum()
    assert np.array_equal(a_walk < 0, ref.accept_len < 0)
    assert np.array_equal(a_full < 0, ref_full.accept_len < 0)


def test_walk_truncated_with_stopping_rules(sv):
    cfg = CONFIGS["c2"]
    x = make_inputs(cfg, 19, DEV)
    tk, tp = _trunc_settings(cfg.B, cfg.V, 20)
    x = _trunc_drafts(x, cfg.T, tk, tp, 21)
    rng = np.random.default_rng(7)
    toks = x["tokens"].cpu().numpy()
    eos = int(np.bincount(toks.ravel()).argmax())
    kb = rng.integers(0, cfg.K + 1, cfg.B).astype(np.int32)
    mx = rng.integers(1, cfg.K + 3, cfg.B).astype(np.int32)
    kb[3], kb[4], mx[5] = -1, cfg.K + 1, 0
    _trunc_case(sv, x, cfg, (tk, tp), "c2/trunc/stops", stops=(eos, kb, mx))


def test_walk_truncated_c3_whole_batch(sv):
    cfg = CONFIGS["c3"]
    x = make_inputs(cfg, 0, DEV)
    tk = np.full(cfg.B, 50, np.int32)
    tp = np.full(cfg.B, 0.9, np.float32)
    _trunc_case(sv, x, cfg, (tk, tp), "c3/trunc")


@pytest.mark.parametrize("name", ["c1", "c2f32"])
def test_walk_fp32_truncated(sv, name):
    """Truncated fp32 rows through the list, one-read and multi-read passes
    (mixed per-sequence top-k / top-p, invalid top_p included)."""
    cfg = (CONFIGS["c1"].scaled(B=32) if name == "c1"
           else CONFIGS["c2"].scaled(B=32, dtype="f32"))
    x = make_inputs(cfg, 23, DEV)
    tk, tp = _trunc_settings(cfg.B, cfg.V, 24, invalid=True)
    x = _trunc_drafts(x, cfg.T, tk, tp, 25)
    walk, full, ref = _trunc_case(sv, x, cfg, (tk, tp), f"{name}/fp32 trunc")
    a = walk[1].cpu().numpy()
    assert a[1] == -1 and a[2] == -1


def test_walk_fp32_truncated_unusable_rows_count_only_where_read(sv):
    cfg = CONFIGS["c1"].scaled(B=40)
    x = make_inputs(cfg, 26, DEV)
    tk, tp = _trunc_settings(cfg.B, cfg.V, 27)
    x = _trunc_drafts(x, cfg.T, tk, tp, 28)
    trunc = (tk, tp)
    j = _run(sv, x, cfg, False, trunc=trunc)[1].cpu().numpy()
    assert np.all(j >= 0)
    y = _plant(x, cfg, j, 29)
    rows = np.arange(cfg.B)
    walk = _run(sv, y, cfg, True, trunc=trunc)
    full = _run(sv, y, cfg, False, trunc=trunc)
    ref = oracle_for(y, rows, "stochastic", trunc=trunc, walk=True)
    ref_full = oracle_for(y, rows, "stochastic", trunc=trunc)
    compare(rows, ref, walk[0], walk[1], "stochastic", walk[3], "c1/fp32 trunc/walk/planted")
    compare(rows, ref_full, full[0], full[1], "stochastic", full[3],
            "c1/fp32 trunc/full/planted")
    _pq_pattern(walk[3], ref, rows, "c1/fp32 trunc/planted")
    a_walk, a_full = walk[1].cpu().numpy(), full[1].cpu().numpy()
    assert (a_walk < 0).sum() < (a_full < 0).sum()
    assert np.array_equal(a_walk < 0, ref.accept_len < 0)


def test_walk_fp32_truncated_c5_sample(sv):
    """The c5 shape (B = 1024, fp32, p = q and zeroed-mass sequences), top-k
    50 + top-p 0.9: every sequence equal to the full reading, a sample of
    256 against the oracle."""
    cfg = CONFIGS["c5"]
    x = make_inputs(cfg, 0, DEV)
    tk = np.full(cfg.B, 50, np.int32)
    tp = np.full(cfg.B, 0.9, np.float32)
    walk = _run(sv, x, cfg, True, trunc=(tk, tp))
    full = _run(sv, x, cfg, False, trunc=(tk, tp))
    _same_exact(walk, full)
    rows = np.sort(np.random.default_rng(31).choice(cfg.B, 256, replace=False))
    ref = oracle_for(x, rows, "stochastic", trunc=(tk, tp), walk=True)
    compare(rows, ref, walk[0], walk[1], "stochastic", walk[3], "c5/fp32 trunc/walk")


# --------------------------------------------------------------------------
# small shapes: one drafted position, one sequence
# --------------------------------------------------------------------------

@pytest.mark.parametrize("route", ["plain", "trunc-bf16", "trunc-fp32", "greedy", "margin"])
@pytest.mark.parametrize("B,K", [(1, 1), (1, 4), (9, 1)])
def test_walk_small_shapes(sv, route, B, K):
    """Grids of one or two workgroups per stage, a list stage holding only
    the bonus row (K = 1), and a single sequence: every route of the
    walk-order reading against the oracle's and the full reading."""
    dtype = "f32" if route == "trunc-fp32" else "bf16"
    cfg = CONFIGS["c2"].scaled(B=B, K=K, dtype=dtype)
    argmax = route in ("greedy", "margin")
    for step in range(6):
        x = make_inputs(cfg, 40 + step, DEV, "greedy" if argmax else "stochastic")
        trunc = None
        if route.startswith("trunc"):
            tk = np.full(B, 20, np.int32)
            tp = np.full(B, 0.9, np.float32)
            trunc = (tk, tp)
            x = _trunc_drafts(x, cfg.T, tk, tp, 50 + step)
        mode = route if argmax else "stochastic"
        rows = np.arange(B)
        walk = _run(sv, x, cfg, True, mode=mode, trunc=trunc)
        full = _run(sv, x, cfg, False, mode=mode, trunc=trunc)
        ref = oracle_for(x, rows, mode, tau=TAU, trunc=trunc, walk=True)
        compare(rows, ref, walk[0], walk[1], mode, walk[3], f"small/{route}/B{B}K{K}/{step}")
        for a, b in zip(walk[:3], full[:3]):
            assert torch.equal(a, b)
