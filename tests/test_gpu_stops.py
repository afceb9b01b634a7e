"""GPU parity of the stopping rules (end-of-sequence token, per-sequence
draft count k_b, emission budget m_b) against the oracle, on every path:
greedy and margin scans, and the three stochastic paths (per-sequence finish
after the streaming pass, the multi-kernel scan/tile/pick path, and the one
kernel per sequence).
"""

import numpy as np
import pytest
import torch

from oracle import spec_oracle as O
from tests.parity import compare, oracle_for
from workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


@pytest.fixture(scope="module")
def sv():
    import speculative_decoding_verification_temp_amd as pkg
    pkg.load_library()
    torch.cuda.set_device(DEV)
    return pkg


def _stops(x, cfg, seed, bad=False):
    """eos = the most frequent drafted token (so that it is hit often), random
    k_b in [0, K] and m_b in [1, K + 2]; with bad=True a few invalid values."""
    rng = np.random.default_rng(seed)
    toks = x["tokens"].cpu().numpy()
    eos = int(np.bincount(toks.ravel()).argmax())
    kb = rng.integers(0, cfg.K + 1, cfg.B).astype(np.int32)
    mx = rng.integers(1, cfg.K + 3, cfg.B).astype(np.int32)
    if bad:
        kb[1], kb[2], mx[3] = -1, cfg.K + 1, 0
    return eos, kb, mx


def _run(sv, x, cfg, mode, stops, decay=0.9):
    eos, kb, mx = stops
    v = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, x["target"].dtype, ema_decay=decay)
    aux = v.enable_aux()
    kb_d = None if kb is None else torch.as_tensor(kb, device=DEV).contiguous()
    mx_d = None if mx is None else torch.as_tensor(mx, device=DEV).contiguous()
    v.set_stops(eos, kb_d, mx_d)
    tok, alen, hist = v.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"],
                               mode, tau=x.get("tau", 0.0))
    torch.cuda.synchronize()
    return v, aux, tok, alen, hist


def _check_stop_invariants(tok, alen, x, stops, K):
    eos, kb, mx = stops
    t = tok.cpu().numpy().astype(np.int64)
    a = alen.cpu().numpy().astype(np.int64)
    d = x["tokens"].cpu().numpy()
    for b in np.flatnonzero(a >= 0):
        e = [int(v) for v in t[b] if v >= 0]
        assert np.all(t[b, len(e):] == -1)
        assert 1 <= len(e) <= min(mx[b], kb[b] + 1)
        assert a[b] <= len(e) and np.array_equal(t[b, :a[b]], d[b, :a[b]])
        if eos in e:
            assert e.index(eos) == len(e) - 1


@pytest.mark.parametrize("mode", ["stochastic", "greedy", "margin"])
def test_stops_full_batch_fp32(sv, mode):
    cfg = CONFIGS["c1"].scaled(B=96)
    x = make_inputs(cfg, 2, DEV, "stochastic" if mode == "stochastic" else "greedy")
    x["tau"] = 0.3
    stops = _stops(x, cfg, 5, bad=True)
    v, aux, tok, alen, hist = _run(sv, x, cfg, mode, stops)
    rows = np.arange(cfg.B)
    ema = O.EmaState(cfg.B, 0.9)
    ref = oracle_for(x, rows, mode, tau=0.3, ema=ema, stops=stops)
    rep = compare(rows, ref, tok, alen, mode, aux, f"stops/c1/{mode}")
    assert np.array_equal(hist.cpu().numpy(), ref.hist)
    assert np.all(alen.cpu().numpy()[[1, 2, 3]] == -1)
    _check_stop_invariants(tok, alen, x, stops, cfg.K)
    e, s = v.ema()
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy(), ema.steps)
    assert np.max(np.abs(e.cpu().numpy() - ema.ema)) <= 1e-12
    print(f"stops/c1/{mode}: {rep}", flush=True)


@pytest.mark.parametrize("path", ["finish", "multikernel", "fused"])
def test_stops_bf16_stochastic_paths(sv, monkeypatch, path):
    monkeypatch.setenv("SPEC_VERIFY_FUSED_MIN_B", "1" if path == "fused" else "0")
    monkeypatch.setenv("SPEC_VERIFY_FINISH_SEQ", "0" if path == "multikernel" else "1")
    cfg = CONFIGS["c2"].scaled(B=64)
    x = make_inputs(cfg, 3, DEV)
    stops = _stops(x, cfg, 9)
    v, aux, tok, alen, hist = _run(sv, x, cfg, "stochastic", stops)
    rows = np.arange(cfg.B)
    ref = oracle_for(x, rows, "stochastic", stops=stops)
    rep = compare(rows, ref, tok, alen, "stochastic", aux, f"stops/c2/{path}")
    assert np.array_equal(hist.cpu().numpy(), ref.hist)
    _check_stop_invariants(tok, alen, x, stops, cfg.K)
    print(f"stops/c2/{path}: {rep}", flush=True)


def test_rows_past_the_draft_count_are_not_needed(sv):
    cfg = CONFIGS["c1"].scaled(B=8)
    x = make_inputs(cfg, 4, DEV)
    kb = np.full(cfg.B, 2, dtype=np.int32)
    x["target"][0, 3, 7] = float("nan")      # target row 3 > k_b
    x["draft"][1, 2, :] = float("-inf")      # draft row 2 >= k_b
    x["tokens"][2, 3] = cfg.V + 9            # drafted token at position 3 >= k_b
    stops = (-1, kb, None)
    v, aux, tok, alen, hist = _run(sv, x, cfg, "stochastic", stops)
    a = alen.cpu().numpy()
    assert np.all(a >= 0) and np.all(a <= 2)
    rows = np.arange(cfg.B)
    compare(rows, oracle_for(x, rows, "stochastic", stops=stops), tok, alen, "stochastic", aux,
            "stops/unneeded rows")


def test_set_stops_arguments_and_reset(sv):
    cfg = CONFIGS["c1"].scaled(B=16)
    x = make_inputs(cfg, 6, DEV)
    v = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, x["target"].dtype)
    assert v.lib.spec_verify_set_stops(v._h, -2, None, None) == sv.SV_EINVAL
    assert v.lib.spec_verify_set_stops(None, -1, None, None) == sv.SV_EINVAL
    plain = [t.clone() for t in v.verify(x["target"], x["draft"], x["tokens"], x["uniforms"],
                                         x["T"])]
    v.set_stops(int(x["tokens"][0, 0]), None, torch.ones(cfg.B, dtype=torch.int32, device=DEV))
    one = v.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"])
    torch.cuda.synchronize()
    assert np.all((one[0].cpu().numpy() >= 0).sum(axis=1) == 1)
    v.clear_stops()
    again = v.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"])
    torch.cuda.synchronize()
    assert torch.equal(plain[0], again[0]) and torch.equal(plain[1], again[1])
