"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Small configurations and special cases are compared on the full batch here;
the full-size configurations are compared on whole batches in
test_gpu_full_batch.py.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import spec_oracle as O
from tests.parity import check_invariants, compare, oracle_for
from workloads import (CONFIGS, const_alpha_inputs, make_inputs, mc_inputs, to_host_f64,
                       window_edge_inputs)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


@pytest.fixture(scope="module")
def sv():
    import speculative_decoding_verification_temp_amd as pkg
    pkg.load_library()          # fails loudly when the library is missing
    torch.cuda.set_device(DEV)
    return pkg


def _verify(sv, x, cfg, mode, B=None, V=None, K=None, decay=None):
    B = B or x["target"].shape[0]
    K = K or x["target"].shape[1] - 1
    V = V or x["target"].shape[2]
    v = sv.SpecVerifier(B, K, V, x["target"].dtype, ema_decay=decay or cfg.ema_decay)
    aux = v.enable_aux()
    tok, alen, hist = v.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], mode,
                               tau=x.get("tau", 0.0))
    torch.cuda.synchronize()
    return v, aux, tok, alen, hist


def _sample(B, n, seed):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(B, size=min(n, B), replace=False))


def _log(msg):
    print(msg, flush=True)


# --------------------------------------------------------------------------
# full-batch parity on small configurations
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["stochastic", "greedy", "margin"])
def test_c1_full_batch(sv, mode):
    cfg = CONFIGS["c1"]
    x = make_inputs(cfg, 0, DEV, "stochastic" if mode == "stochastic" else "greedy")
    x["tau"] = 0.3
    v, aux, tok, alen, hist = _verify(sv, x, cfg, mode)
    rows = np.arange(cfg.B)
    ref = oracle_for(x, rows, mode, tau=0.3)
    rep = compare(rows, ref, tok, alen, mode, aux, f"c1/{mode}")
    check_invariants(tok, alen, hist, x["tokens"], cfg.V, cfg.K)
    assert np.array_equal(hist.cpu().numpy(), ref.hist)
    _log(f"c1/{mode}: {rep}")


def test_c2_full_batch(sv):
    cfg = CONFIGS["c2"]
    x = make_inputs(cfg, 0, DEV)
    v, aux, tok, alen, hist = _verify(sv, x, cfg, "stochastic")
    rows = np.arange(cfg.B)
    ref = oracle_for(x, rows, "stochastic")
    rep = compare(rows, ref, tok, alen, "stochastic", aux, "c2")
    check_invariants(tok, alen, hist, x["tokens"], cfg.V, cfg.K)
    # an excused mismatch moves at most one count between two bins
    h = hist.cpu().numpy().astype(np.int64)
    assert np.abs(h - ref.hist).sum() <= 2 * rep["mismatches"]
    _log(f"c2: {rep} alpha~{np.mean(ref.accept_len) / cfg.K:.3f}")


def test_c2_forced_segments_agree(sv, monkeypatch):
    """The streaming pass split into several segments per row gives the same
    decisions (segment partials are combined by exact power-of-two rescaling)."""
    cfg = CONFIGS["c2"]
    x = make_inputs(cfg, 1, DEV)
    outs = []
    for nseg in ("1", "3"):
        monkeypatch.setenv("SPEC_VERIFY_NSEG", nseg)
        v, aux, tok, alen, hist = _verify(sv, x, cfg, "stochastic")
        outs.append((tok.clone(), alen.clone(), aux["p_d"].clone()))
        v.close()
    rows = np.arange(cfg.B)
    ref = oracle_for(x, rows, "stochastic")
    for tok, alen, _ in outs:
        compare(rows, ref, tok, alen, "stochastic", None, "c2/nseg")
    # fp32 group sums round differently per partition: ~1e-8 relative
    assert torch.allclose(outs[0][2], outs[1][2], rtol=1e-6, atol=0)


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_fused_and_pipeline_paths_agree(sv, monkeypatch, name):
    """The three stochastic paths match the oracle and each other: the
    streaming pass then one workgroup per sequence (default; its wavefronts
    claim the draw tiles from a counter, or take fixed tiles), the streaming
    pass then separate scan, tile-sum and pick kernels (the path for V >
    524288), and one workgroup per sequence for everything (forced on)."""
    cfg = CONFIGS[name]
    x = make_inputs(cfg, 5, DEV)
    outs = {}
    for path, min_b, fin, claim in (("pipeline", "0", "1", "1"), ("fixed-tiles", "0", "1", "0"),
                                    ("multikernel", "0", "0", "1"), ("fused", "1", "1", "1")):
        monkeypatch.setenv("SPEC_VERIFY_FUSED_MIN_B", min_b)
        monkeypatch.setenv("SPEC_VERIFY_FINISH_SEQ", fin)
        monkeypatch.setenv("SPEC_VERIFY_CLAIM_TILES", claim)
        v, aux, tok, alen, hist = _verify(sv, x, cfg, "stochastic")
        outs[path] = (tok.clone(), alen.clone(), hist.clone(),
                      {k: t.clone() for k, t in aux.items()})
        v.close()
    rows = np.arange(cfg.B)
    ref = oracle_for(x, rows, "stochastic")
    for path, (tok, alen, hist, aux) in outs.items():
        rep = compare(rows, ref, tok, alen, "stochastic", aux, f"{name}/{path}")
        check_invariants(tok, alen, hist, x["tokens"], cfg.V, cfg.K)
        _log(f"{name}/{path}: {rep}")
    a = outs["pipeline"]
    for other in ("fixed-tiles", "multikernel", "fused"):
        b = outs[other]
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
        assert torch.allclose(a[3]["p_d"], b[3]["p_d"], rtol=1e-6, atol=0)
        assert torch.allclose(a[3]["z"], b[3]["z"], rtol=1e-9, atol=1e-15)


# --------------------------------------------------------------------------
# statistical checks (the sampler recovers p) and tiny vocabularies
# --------------------------------------------------------------------------

def _mc_cases():
    rng = np.random.default_rng(16)
    p16 = rng.dirichlet(np.ones(16))
    q16 = rng.dirichlet(np.ones(16))
    q16[[2, 5, 11]] = 0.0
    q16 /= q16.sum()
    return [("V3", np.array([0.6, 0.3, 0.1]), np.array([0.2, 0.5, 0.3])), ("V16", p16, q16)]


@pytest.mark.parametrize("name,p,q", _mc_cases())
def test_monte_carlo_recovers_target(sv, name, p, q):
    N = 200_000
    x = mc_inputs(p, q, N, 20260923, device=DEV)
    v, aux, tok, alen, hist = _verify(sv, x, None, "stochastic", decay=0.99)
    first = tok[:, 0].cpu().numpy().astype(np.int64)
    # the law the kernels sample is softmax of the stored fp32 logits
    pf = O.softmax_t(to_host_f64(x["target"][0, 0]), 1.0)
    freq = np.bincount(first, minlength=len(p)) / N
    se = np.sqrt(pf * (1 - pf) / N)
    assert np.all(np.abs(freq - pf) <= 5 * se + 1e-12), (freq, pf)
    zq = np.flatnonzero(q == 0)
    kept = alen.cpu().numpy() == 1
    assert not np.isin(first[kept], zq).any()
    check_invariants(tok, alen, hist, x["tokens"], len(p), 1)
    rows = np.arange(3000)
    ref = oracle_for(x, rows, "stochastic")
    rep = compare(rows, ref, tok, alen, "stochastic", aux, f"mc/{name}")
    _log(f"mc/{name}: freq {np.round(freq, 4)} p {np.round(pf, 4)} {rep}")


def test_draw_precision_large_vocab(sv):
    """Many one-draft sequences at V = 128256: every sequence is compared with
    the oracle, so the rate of draws that differ (all of which must lie within
    1e-6 of a boundary) is measured, not sampled. At this vocabulary a token's
    share of [0, 1) is ~1e-5 on average, so the draw needs float64-accurate
    weights to keep that rate under 1e-4."""
    cfg = CONFIGS["c3"].scaled(B=8192, K=1)
    x = make_inputs(cfg, 7, DEV)
    v, aux, tok, alen, hist = _verify(sv, x, cfg, "stochastic")
    check_invariants(tok, alen, hist, x["tokens"], cfg.V, cfg.K)
    rows = np.arange(cfg.B)
    ref = oracle_for(x, rows, "stochastic")
    rep = compare(rows, ref, tok, alen, "stochastic", aux, "draw precision")
    _log(f"draw precision V=128256: {rep}")
    assert rep["mismatches"] <= 1e-4 * 2 * cfg.B


def test_constant_alpha_closed_form(sv):
    alpha, K, B = 0.6, 5, 100_000
    x = const_alpha_inputs(alpha, K, B, 99, device=DEV)
    v, aux, tok, alen, hist = _verify(sv, x, None, "stochastic", decay=0.99)
    a = alen.cpu().numpy()
    E = (1 - alpha ** (K + 1)) / (1 - alpha)
    em = a + 1
    assert abs(em.mean() - E) < 5 * em.std() / math.sqrt(B)
    h = hist.cpu().numpy().astype(np.float64)
    probs = np.array([alpha ** j * (1 - alpha) for j in range(K)] + [alpha ** K])
    chi2 = ((h - probs * B) ** 2 / (probs * B)).sum()
    import scipy.stats
    assert chi2 < scipy.stats.chi2.ppf(0.9999, K)


def test_scalar_path_odd_vocab_bf16(sv):
    cfg = CONFIGS["c2"].scaled(B=48, V=1001)
    for mode in ("stochastic", "greedy", "margin"):
        x = make_inputs(cfg, 0, DEV, "stochastic" if mode == "stochastic" else "greedy")
        x["tau"] = 0.3
        v, aux, tok, alen, hist = _verify(sv, x, cfg, mode)
        rows = np.arange(cfg.B)
        ref = oracle_for(x, rows, mode, tau=0.3)
        compare(rows, ref, tok, alen, mode, aux, f"V1001/{mode}")
        check_invariants(tok, alen, hist, x["tokens"], cfg.V, cfg.K)


def test_bf16_values_outside_table_window(sv):
    """bf16 rows holding +-0, magnitudes below 2^-25, magnitudes of 128 and
    more, -inf, and dominant +150 entries: the draw's table lookups flag these
    values and recompute those lanes term by term. Full batch against the
    oracle, ragged last tile (V = 32000)."""
    cfg = CONFIGS["c2"].scaled(B=64, K=4, T=1.0)
    x = window_edge_inputs(cfg, 0, DEV)
    v, aux, tok, alen, hist = _verify(sv, x, cfg, "stochastic")
    rows = np.arange(cfg.B)
    ref = oracle_for(x, rows, "stochastic")
    rep = compare(rows, ref, tok, alen, "stochastic", aux, "window edges")
    check_invariants(tok, alen, hist, x["tokens"], cfg.V, cfg.K)
    assert np.array_equal(hist.cpu().numpy(), ref.hist)
    assert np.all(alen.cpu().numpy() >= 0)
    _log(f"window edges: {rep}")


@pytest.mark.parametrize("case", ["low_temperature", "shifted_logits"])
def test_bf16_large_reference_scaled_draw(sv, case):
    """Rows whose integer reference |R| = |ceil(max(x) log2(e) / T)| exceeds 500
    (T = 0.02, or logits shifted to about -900) take the draw path that scales
    every term by 2^-R as it is formed. Full batch against the oracle."""
    if case == "low_temperature":
        cfg = CONFIGS["c2"].scaled(B=48, K=3, T=0.02)
        x = make_inputs(cfg, 1, DEV)
    else:
        cfg = CONFIGS["c2"].scaled(B=48, K=3, T=1.0)
        x = make_inputs(cfg, 2, DEV)
        for key in ("target", "draft"):
            x[key] = (x[key].to(torch.float32) - 900.0).to(torch.bfloat16).contiguous()
    v, aux, tok, alen, hist = _verify(sv, x, cfg, "stochastic")
    rows = np.arange(cfg.B)
    ref = oracle_for(x, rows, "stochastic")
    rep = compare(rows, ref, tok, alen, "stochastic", aux, case)
    check_invariants(tok, alen, hist, x["tokens"], cfg.V, cfg.K)
    assert np.array_equal(hist.cpu().numpy(), ref.hist)
    _log(f"{case}: {rep}")


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------

def test_p_equals_q_all_accepted(sv):
    cfg = CONFIGS["c1"].scaled(B=32)
    x = make_inputs(cfg, 3, DEV)
    x["draft"] = x["target"][:, : cfg.K].contiguous()
    v, aux, tok, alen, hist = _verify(sv, x, cfg, "stochastic")
    assert np.all(alen.cpu().numpy() == cfg.K)
    assert torch.equal(aux["p_d"][: cfg.B], aux["q_d"][: cfg.B])
    assert np.all(aux["z"].cpu().numpy()[: cfg.B] == -1.0)
    rows = np.arange(cfg.B)
    compare(rows, oracle_for(x, rows, "stochastic"), tok, alen, "stochastic", aux, "p=q")


def test_invalid_inputs_are_reported(sv):
    cfg = CONFIGS["c1"].scaled(B=8)
    x = make_inputs(cfg, 4, DEV)
    x["tokens"][0, 1] = cfg.V              # out of range
    x["tokens"][1, 0] = -3                 # negative
    x["target"][2, 3, 17] = float("nan")   # NaN in a target row
    x["draft"][3, 0, :] = float("-inf")    # draft row without a finite maximum
    x["target"][4, 4, 5] = float("inf")    # +inf in the bonus row
    v, aux, tok, alen, hist = _verify(sv, x, cfg, "stochastic")
    a = alen.cpu().numpy()
    assert list(a[:5]) == [-1] * 5 and np.all(a[5:] >= 0)
    assert np.all(tok.cpu().numpy()[:5] == -1)
    st = v.stats()
    assert st["invalid"] == 5 and st["sequences"] == 3
    rows = np.arange(cfg.B)
    compare(rows, oracle_for(x, rows, "stochastic"), tok, alen, "stochastic", None, "invalid")
    check_invariants(tok, alen, hist, x["tokens"], cfg.V, cfg.K)
    # greedy reads target rows only
    vg = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, x["target"].dtype)
    tg, ag, hg = vg.verify(x["target"], None, x["tokens"], None, 1.0, "greedy")
    torch.cuda.synchronize()
    compare(rows, oracle_for(x, rows, "greedy"), tg, ag, "greedy", None, "invalid/greedy")


def test_determinism_bitwise(sv):
    cfg = CONFIGS["c2"]
    x = make_inputs(cfg, 2, DEV)
    r1 = _verify(sv, x, cfg, "stochastic")
    r2 = _verify(sv, x, cfg, "stochastic")
    assert torch.equal(r1[2], r2[2]) and torch.equal(r1[3], r2[3]) and torch.equal(r1[4], r2[4])
    for k in ("p_d", "q_d", "z"):
        assert torch.equal(r1[1][k], r2[1][k])


def test_argument_errors_enqueue_nothing(sv):
    cfg = CONFIGS["c1"]
    x = make_inputs(cfg, 0, DEV)
    v = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, x["target"].dtype)
    out = (torch.full((cfg.B, cfg.K + 1), 7, dtype=torch.int32, device=DEV),
           torch.full((cfg.B,), 7, dtype=torch.int32, device=DEV),
           torch.full((cfg.K + 1,), 7, dtype=torch.int32, device=DEV))
    L = v.lib
    import ctypes
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [p(x["target"]), p(x["draft"]), p(x["tokens"]), p(x["uniforms"])]
    outs = [p(o) for o in out]
    assert L.spec_verify(v._h, 0, *args, 1.0, 0, 0.0, *outs, s) == sv.SV_EINVAL
    assert L.spec_verify(v._h, cfg.B + 1, *args, 1.0, 0, 0.0, *outs, s) == sv.SV_EINVAL
    assert L.spec_verify(v._h, cfg.B, *args, 0.0, 0, 0.0, *outs, s) == sv.SV_EINVAL
    assert L.spec_verify(v._h, cfg.B, *args, float("nan"), 0, 0.0, *outs, s) == sv.SV_EINVAL
    assert L.spec_verify(v._h, cfg.B, *args, 1.0, 5, 0.0, *outs, s) == sv.SV_EINVAL
    assert L.spec_verify(v._h, cfg.B, args[0], None, args[2], args[3], 1.0, 0, 0.0, *outs,
                         s) == sv.SV_EINVAL
    assert L.spec_verify(v._h, cfg.B, *args, 1.0, 2, float("inf"), *outs, s) == sv.SV_EINVAL
    assert b"tau" in L.spec_verify_last_error(v._h)
    torch.cuda.synchronize()
    for o in out:
        assert torch.all(o == 7)
    with pytest.raises(sv.SpecVerifyError):
        v.verify(x["target"], x["draft"], x["tokens"].long(), x["uniforms"], 1.0)


def test_ema_tracks_oracle_and_accessors(sv):
    cfg = CONFIGS["c2"].scaled(B=32, V=4096)
    v = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, cfg.torch_dtype, ema_decay=0.9)
    ema = O.EmaState(cfg.B, 0.9)
    rows = np.arange(cfg.B)
    for step in range(5):
        x = make_inputs(cfg, step, DEV)
        tok, alen, hist = v.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], cfg.T)
        torch.cuda.synchronize()
        ref = oracle_for(x, rows, "stochastic", ema=ema)
        compare(rows, ref, tok, alen, "stochastic", None, f"ema step {step}")
    e, s = v.ema()
    torch.cuda.synchronize()
    assert np.all(s.cpu().numpy() == 5)
    assert np.max(np.abs(e.cpu().numpy() - ema.ema)) <= 1e-12
    v.set_ema(torch.full((cfg.B,), 0.5, dtype=torch.float64), torch.ones(cfg.B, dtype=torch.int32))
    e, s = v.ema()
    torch.cuda.synchronize()
    assert torch.all(e == 0.5) and torch.all(s == 1)
    v.reset_ema()
    e, s = v.ema()
    torch.cuda.synchronize()
    assert torch.all(e == 0) and torch.all(s == 0)


def test_profiling_events(sv):
    """The profiling window counts the recorded calls; the streaming-pass time
    is positive and, when call ends are recorded, no longer than the call."""
    cfg = CONFIGS["c2"].scaled(B=16)
    x = make_inputs(cfg, 0, DEV)
    v = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, x["target"].dtype)
    for call_end in (False, True):
        v.profile(True, call_end=call_end)
        for _ in range(3):
            v.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"])
        pass_ms, call_ms, n = v.profile_read()
        assert n == 3 and pass_ms > 0.0
        if call_end:
            assert call_ms >= pass_ms
        else:
            assert call_ms == 0.0
        v.profile(False)



def test_read_probe_entry_point(sv):
    """The streaming-read measurement aid runs on a device buffer and rejects
    misaligned or ragged sizes before enqueueing anything."""
    L = sv.load_library()
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device=DEV)
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    sv.read_probe(buf, sink)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream(DEV).cuda_stream
    ptr = buf.data_ptr()
    assert L.spec_verify_read_probe(ptr + 4, 1024, sink.data_ptr(), s) == sv.SV_EINVAL
    assert L.spec_verify_read_probe(ptr, 1000, sink.data_ptr(), s) == sv.SV_EINVAL
    assert L.spec_verify_read_probe(None, 1024, sink.data_ptr(), s) == sv.SV_EINVAL
    assert L.spec_verify_read_probe(ptr, 1024, None, s) == sv.SV_EINVAL
