"""GPU parity of top-k / top-p truncation over fp32 rows against the oracle.

fp32 rows go through their own truncation passes (the row's top-k list from
one read; else the k-th largest order key and the top-p level found digit by
digit, 12 + 10 + 10 bits, with fixed-point masses, or from the few candidate
values sorted in LDS) and then the per-sequence finish, whose draw compares
each value's order key with its row's threshold. The main cases run on each
route (the `route` fixture; SPEC_VERIFY_TRUNC32_LIST=0 skips the list pass,
SPEC_VERIFY_TRUNC32_BUF=0 keeps to the digit reads), and rows a route cannot
settle fall back by themselves. The tests cover:
per-sequence mixes of settings (off, on, invalid), each rule alone, drafts
from the untruncated draft (q(d) = 0 accepted), values that share their
upper key digits, ties, -inf, zeros of both signs, huge magnitudes, rows with
NaN or +inf, low temperatures (the draw's per-term scaled path), the stopping
rules, the residual side output, top_k = 1 against the greedy mode,
vocabularies that are not a multiple of 4 (scalar loads), and the c5 shape
(B = 1024, K = 4, V = 128256) on sampled sequences.
"""

import numpy as np
import pytest
import torch

from oracle import spec_oracle as O
from tests.parity import compare, oracle_for
from tests.test_gpu_trunc import _check, _resample_drafts, _settings
from workloads import CONFIGS, make_inputs, to_host_f64, window_edge_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
SMALL = CONFIGS["c5"].scaled(B=48, V=20000)


@pytest.fixture(params=["list", "list-multi", "buffered", "digits"])
def route(request, monkeypatch):
    """The truncation passes' route, read when a verifier is created: the
    one-read list pass and the one-read top-p pass first (rows they cannot
    settle then take the buffered route), the list pass without the top-p
    pass, the buffered route alone, or the digit reads alone."""
    monkeypatch.setenv("SPEC_VERIFY_TRUNC32_LIST", "1" if request.param.startswith("list") else "0")
    monkeypatch.setenv("SPEC_VERIFY_TRUNC32_ONE", "0" if request.param == "list-multi" else "1")
    monkeypatch.setenv("SPEC_VERIFY_TRUNC32_BUF", "0" if request.param == "digits" else "1")
    return request.param


@pytest.fixture(scope="module")
def sv():
    import speculative_decoding_verification_temp_amd as pkg
    pkg.load_library()
    torch.cuda.set_device(DEV)
    return pkg


def test_trunc32_per_sequence_settings(sv, route):
    cfg = SMALL
    x = make_inputs(cfg, 1, DEV)
    assert x["target"].dtype == torch.float32
    tk, tp = _settings(cfg.B, cfg.V, 21, invalid=True)
    _resample_drafts(x, cfg.T, tk, tp, 22)
    tok, alen, ref = _check(sv, x, cfg, tk, tp, f"trunc32/mixed/{route}")
    a = alen.cpu().numpy()
    assert a[1] == -1 and a[2] == -1          # top_p = 0 and NaN
    assert (a >= 0).sum() == cfg.B - 2


@pytest.mark.parametrize("which", ["top_k", "top_p"])
def test_trunc32_one_rule(sv, which, route):
    cfg = SMALL.scaled(B=32)
    x = make_inputs(cfg, 2, DEV)
    tk, tp = _settings(cfg.B, cfg.V, 23)
    if which == "top_k":
        tp = None
    else:
        tk = None
    _resample_drafts(x, cfg.T, tk if tk is not None else np.zeros(cfg.B, np.int32),
                     tp if tp is not None else np.ones(cfg.B, np.float32), 24)
    _check(sv, x, cfg, tk, tp, f"trunc32/{which}/{route}")


def test_trunc32_untruncated_drafts(sv):
    cfg = SMALL.scaled(B=32)
    x = make_inputs(cfg, 3, DEV)
    tk = np.full(cfg.B, 30, np.int32)
    tp = np.full(cfg.B, 0.9, np.float32)
    _check(sv, x, cfg, tk, tp, "trunc32/raw drafts")


def test_trunc32_special_values(sv, route):
    """Per sequence (mod 8): 0 values that share their upper 22 key bits
    (1 + n 2^-23), 1 integer ties, 2 -inf in a third of the entries with
    +-0, 3 magnitudes near 3e6 (a bin's values span far more than the
    float64 range of the softmax), 4 one value of +40 dominating, 5 all but
    one value -inf, 6 one NaN (invalid), 7 one +inf (invalid)."""
    cfg = SMALL.scaled(B=32, V=4096)
    x = make_inputs(cfg, 4, DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(31)
    V = cfg.V
    for key in ("target", "draft"):
        t = x[key]
        for b in range(cfg.B):
            for i in range(t.shape[1]):
                kind = b % 8
                r = torch.rand(V, generator=g, device=DEV)
                if kind == 0:
                    t[b, i] = 1.0 + torch.randint(0, 50, (V,), generator=g, device=DEV) * 2.0 ** -23
                elif kind == 1:
                    t[b, i] = torch.randint(-3, 3, (V,), generator=g, device=DEV).float()
                elif kind == 2:
                    t[b, i] = torch.where(r < 0.3, float("-inf"), t[b, i])
                    t[b, i] = torch.where((r >= 0.3) & (r < 0.4), 0.0, t[b, i])
                    t[b, i] = torch.where((r >= 0.4) & (r < 0.5), -0.0, t[b, i])
                elif kind == 3:
                    t[b, i] = t[b, i] * 1e6 - 3e6
                elif kind == 4:
                    t[b, i, int(r[0] * V)] = 40.0
                elif kind == 5:
                    t[b, i] = float("-inf")
                    t[b, i, int(r[0] * V)] = -5.0
                elif kind == 6 and key == "target" and i == 0:
                    t[b, i, int(r[0] * V)] = float("nan")
                elif kind == 7 and key == "draft" and i == 0:
                    t[b, i, int(r[0] * V)] = float("inf")
    rng = np.random.default_rng(32)
    tk = rng.choice([0, 1, 5, 100, 2000, V - 1], cfg.B).astype(np.int32)
    tp = rng.choice([1.0, 0.3, 0.9, 0.99], cfg.B).astype(np.float32)
    # drafts from the truncated law where it is defined (valid rows)
    d = to_host_f64(x["draft"])
    toks = np.zeros((cfg.B, cfg.K), dtype=np.int32)
    for b in range(cfg.B):
        for i in range(cfg.K):
            row = d[b, i]
            if np.isnan(row).any() or np.isposinf(row).any():
                toks[b, i] = 0
                continue
            q, _ = O.truncated_softmax(row, cfg.T, int(tk[b]), float(tp[b]))
            toks[b, i] = rng.choice(q.size, p=q)
    x["tokens"] = torch.as_tensor(toks, device=DEV).contiguous()
    tok, alen, ref = _check(sv, x, cfg, tk, tp, f"trunc32/special values/{route}")
    a = alen.cpu().numpy()
    assert np.all(a[6::8] == -1) and np.all(a[7::8] == -1)


def test_trunc32_window_edges(sv):
    cfg = SMALL.scaled(B=32)
    x = window_edge_inputs(cfg, 5, DEV)
    tk, tp = _settings(cfg.B, cfg.V, 25)
    _resample_drafts(x, cfg.T, tk, tp, 26)
    _check(sv, x, cfg, tk, tp, "trunc32/window edges")


def test_trunc32_low_temperature_scaled_path(sv):
    cfg = SMALL.scaled(B=24)
    x = make_inputs(cfg, 6, DEV)
    T = 0.02
    tk, tp = _settings(cfg.B, cfg.V, 27)
    _resample_drafts(x, T, tk, tp, 28)
    _check(sv, x, cfg, tk, tp, "trunc32/low temperature", T=T)


def test_trunc32_with_stops(sv):
    cfg = SMALL
    x = make_inputs(cfg, 7, DEV)
    tk, tp = _settings(cfg.B, cfg.V, 29)
    _resample_drafts(x, cfg.T, tk, tp, 30)
    rng = np.random.default_rng(33)
    toks = x["tokens"].cpu().numpy()
    eos = int(np.bincount(toks.ravel()).argmax())
    kb = rng.integers(0, cfg.K + 1, cfg.B).astype(np.int32)
    mx = rng.integers(1, cfg.K + 3, cfg.B).astype(np.int32)
    _check(sv, x, cfg, tk, tp, "trunc32/stops", stops=(eos, kb, mx))


def test_trunc32_top_k_one_is_greedy(sv):
    cfg = SMALL.scaled(B=64)
    x = make_inputs(cfg, 8, DEV, "greedy")
    v = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, x["target"].dtype)
    g_tok, g_len, _ = [t.clone() for t in v.verify(x["target"], x["draft"], x["tokens"],
                                                   x["uniforms"], cfg.T, "greedy")]
    v.set_truncation(torch.ones(cfg.B, dtype=torch.int32, device=DEV), None)
    s_tok, s_len, _ = v.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], cfg.T,
                               "stochastic")
    torch.cuda.synchronize()
    t, d = x["target"], x["draft"]
    uniq = ((t == t.max(-1, keepdim=True).values).sum(-1) == 1).all(-1) & \
           ((d == d.max(-1, keepdim=True).values).sum(-1) == 1).all(-1)
    u = uniq.cpu().numpy()
    assert u.sum() > cfg.B // 2
    assert np.array_equal(s_tok.cpu().numpy()[u], g_tok.cpu().numpy()[u])
    assert np.array_equal(s_len.cpu().numpy()[u], g_len.cpu().numpy()[u])


def test_trunc32_with_residual(sv):
    """Truncation and the residual side output in one call: the residual's
    support is the untruncated draft's top m, from the own-read route."""
    cfg = SMALL.scaled(B=16)
    x = make_inputs(cfg, 9, DEV)
    tk, tp = _settings(cfg.B, cfg.V, 34)
    _resample_drafts(x, cfg.T, tk, tp, 35)
    v = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, torch.float32)
    aux = v.enable_aux()
    v.set_truncation(torch.as_tensor(tk, device=DEV), torch.as_tensor(tp, device=DEV))
    sup, res = v.set_residual(16)
    tok, alen, hist = v.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], cfg.T)
    torch.cuda.synchronize()
    rows = np.arange(cfg.B)
    ref = oracle_for(x, rows, "stochastic", trunc=(tk, tp))
    compare(rows, ref, tok, alen, "stochastic", aux, "trunc32/residual")
    T32 = float(np.float32(cfg.T))
    r_sup, r_res = O.drift_batch(to_host_f64(x["target"]), to_host_f64(x["draft"]), T32, 16,
                                 alen.cpu().numpy(), None)
    g_res = res.cpu().numpy()
    assert np.array_equal(sup.cpu().numpy(), r_sup)
    both = np.isnan(g_res) & np.isnan(r_res)
    assert np.all(both | (np.abs(g_res - r_res) <= 1e-9))


@pytest.mark.parametrize("V,K,B", [(1001, 3, 8), (3, 1, 4), (16, 2, 1), (8191, 1, 5)])
def test_trunc32_scalar_and_small_shapes(sv, V, K, B, route):
    cfg = SMALL.scaled(B=B, K=K, V=V)
    x = make_inputs(cfg, 12, DEV)
    for b in range(0, B, 2):
        x["target"][b, 0, (7 * b) % V] = 2.0 ** -30
        x["draft"][b, 0, (3 * b + 1) % V] = -200.0
    rng = np.random.default_rng(36)
    tk = rng.integers(0, V + 1, B).astype(np.int32)
    tp = rng.choice([1.0, 0.3, 0.7, 0.95], B).astype(np.float32)
    _resample_drafts(x, cfg.T, tk, tp, 37)
    _check(sv, x, cfg, tk, tp, f"trunc32/V={V} K={K} B={B}/{route}")


def test_trunc32_c5_sampled(sv, route):
    """The c5 shape (B = 1024, K = 4, V = 128256, fp32, its p = q and
    zero-mass sequences included) with top_k = 50 and top_p = 0.9 on every
    sequence; the oracle checks 24 sampled sequences."""
    cfg = CONFIGS["c5"]
    x = make_inputs(cfg, 0, DEV)
    tk = np.full(cfg.B, 50, np.int32)
    tp = np.full(cfg.B, 0.9, np.float32)
    rows = np.random.default_rng(38).choice(cfg.B, 24, replace=False)
    _check(sv, x, cfg, tk, tp, f"trunc32/c5 sampled/{route}", rows=np.sort(rows))


@pytest.mark.parametrize("route", ["list", "list-multi"], indirect=True)
def test_trunc32_top_p_alone_one_read_and_fallback(sv, route):
    """Top-p alone at the c5 vocabulary (V = 128256): the one-read route copies
    the keys above a sampled cut while the row streams; with top_p = 0.5 and
    0.9 the crossing lies in the copy, with 0.999 the kept set (tens of
    thousands of tokens) overflows it and the row falls back to the mass
    reads. Every sequence against the oracle. At top_p = 0.999 the masses of
    the value levels at the cut are about 1e-6 apart, so nearly every such
    row's cut lies within 1e-6 of moving: a third of the rows are expected in
    the excuse band (mismatches must still be none)."""
    cfg = CONFIGS["c5"].scaled(B=24, K=2)
    x = make_inputs(cfg, 9, DEV)
    tp = np.tile(np.array([0.5, 0.9, 0.999], np.float32), cfg.B // 3)
    tk = np.zeros(cfg.B, np.int32)
    _resample_drafts(x, cfg.T, tk, tp, 25)
    _check(sv, x, cfg, None, tp, f"trunc32/top-p alone/{route}", excused_fraction=0.45)


@pytest.mark.parametrize("route", ["list", "list-multi"], indirect=True)
def test_trunc32_large_top_k_one_read(sv, route):
    """Top-k beyond the list pass's lists (500, 1000, 3000 at the c5
    vocabulary), alone or with top_p = 0.95 or 0.5: the list pass hands these
    rows over, and the one-read route finds the k-th largest value and the
    level in its copy of the row's top part (or, on the other route, the
    multi-read pass does). Every sequence against the oracle."""
    cfg = CONFIGS["c5"].scaled(B=24, K=2)
    x = make_inputs(cfg, 10, DEV)
    tk = np.tile(np.array([500, 1000, 3000, 1000, 500, 3000], np.int32), cfg.B // 6)
    tp = np.tile(np.array([1.0, 0.95, 0.5, 1.0, 0.95, 0.95], np.float32), cfg.B // 6)
    _resample_drafts(x, cfg.T, tk, tp, 26)
    _check(sv, x, cfg, tk, tp, f"trunc32/large top-k/{route}")


def test_trunc32_c5_top_p_alone_sampled(sv):
    """The c5 shape with top_p = 0.9 alone on every sequence (the one-read
    route); the oracle checks 24 sampled sequences."""
    cfg = CONFIGS["c5"]
    x = make_inputs(cfg, 0, DEV)
    tp = np.full(cfg.B, 0.9, np.float32)
    rows = np.random.default_rng(39).choice(cfg.B, 24, replace=False)
    _check(sv, x, cfg, None, tp, "trunc32/c5 top-p alone sampled", rows=np.sort(rows))


def test_trunc32_candidates_beyond_buffer(sv):
    """Rows whose candidate values do not fit the LDS buffer take the digit
    reads under the default setting. Sequences b % 4 < 3 hold rows of
    1 + 0.1 u (all values in one first-digit bin, [1, 1.125)) at T = 0.05:
    top-k at half the vocabulary, top-p = 0.5 alone, and top-k 40 with
    top-p 0.9 (the cut bin holds every value of the row); sequences
    b % 4 == 3 keep their plain rows with top-k 40 and top-p 0.9, which fit."""
    cfg = SMALL.scaled(B=32, T=0.05)
    x = make_inputs(cfg, 13, DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(41)
    for key in ("target", "draft"):
        t = x[key]
        for b in range(cfg.B):
            if b % 4 < 3:
                t[b] = 1.0 + 0.1 * torch.rand(t.shape[1:], generator=g, device=DEV)
    m = np.arange(cfg.B) % 4
    tk = np.select([m == 0, m == 1], [cfg.V // 2, 0], 40).astype(np.int32)
    tp = np.select([m == 0, m == 1], [1.0, 0.5], 0.9).astype(np.float32)
    _resample_drafts(x, cfg.T, tk, tp, 39)
    _check(sv, x, cfg, tk, tp, "trunc32/beyond buffer")


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 524296), (torch.bfloat16, 65537),
                                     (torch.float32, 262148), (torch.float32, 65537)])
def test_trunc_vocabulary_limits(sv, dtype, V):
    """Past the finish's tile limit (524288 bf16 / 262144 fp32 values in
    16-byte chunks, 65536 on the scalar path) a truncated call is refused with
    SV_EUNSUPPORTED before anything is enqueued; without truncation the same
    shape verifies."""
    B, K = 1, 1
    g = torch.Generator(device=DEV)
    g.manual_seed(43)
    target = torch.randn((B, K + 1, V), generator=g, device=DEV).to(dtype)
    draft = torch.randn((B, K, V), generator=g, device=DEV).to(dtype)
    tokens = torch.zeros((B, K), dtype=torch.int32, device=DEV)
    uniforms = torch.full((B, K + 1), 0.5, dtype=torch.float32, device=DEV)
    v = sv.SpecVerifier(B, K, V, dtype)
    out = (torch.full((B, K + 1), -7, dtype=torch.int32, device=DEV),
           torch.full((B,), -7, dtype=torch.int32, device=DEV),
           torch.full((K + 1,), 7, dtype=torch.int32, device=DEV))
    v.set_truncation(torch.full((B,), 5, dtype=torch.int32, device=DEV), None)
    with pytest.raises(sv.SpecVerifyError) as e:
        v.verify(target, draft, tokens, uniforms, 1.0, out=out)
    assert e.value.code == sv.SV_EUNSUPPORTED
    torch.cuda.synchronize()
    assert int(out[0].min()) == -7 and int(out[1][0]) == -7 and int(out[2].max()) == 7
    v.clear_truncation()
    tok, alen, _ = v.verify(target, draft, tokens, uniforms, 1.0)
    torch.cuda.synchronize()
    assert int(alen[0]) in (0, 1)


def test_trunc32_list_holds_every_token(sv, route):
    """V = 256 (16-byte chunks), so top_k = V - 1 makes the list pass keep
    every token (its `complete` case, where ties at the cut are counted in
    the list itself); half the rows hold integer ties."""
    cfg = SMALL.scaled(B=8, K=2, V=256)
    x = make_inputs(cfg, 14, DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(47)
    for key in ("target", "draft"):
        for b in range(0, cfg.B, 2):
            x[key][b] = torch.randint(-2, 3, x[key][b].shape, generator=g, device=DEV).float()
    tk = np.array([255, 255, 254, 128, 5, 1, 200, 255], np.int32)
    tp = np.array([1.0, 0.9, 0.5, 0.95, 1.0, 1.0, 0.3, 0.99], np.float32)
    _resample_drafts(x, cfg.T, tk, tp, 48)
    _check(sv, x, cfg, tk, tp, f"trunc32/list holds every token/{route}")
