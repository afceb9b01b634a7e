"""GPU parity of the draft residual side output against the oracle.

Supports must match exactly (token ids in order); residuals within 1e-9
(both sides sum the same 32 float64 exponentials in different orders).
Cases: a full c2 batch with per-sequence draft counts and invalid sequences
(also as the second call on a verifier whose first call read every row),
rows with many ties, V below m, -inf logits inside the support, draft rows
with 70000 equal values, every route to the support (the streaming pass's
candidate lists with one and three segments per row, merged inside the
finish or by their own kernel, the kernel that reads
the rows itself after truncation, on rows not in 16-byte chunks and after the
one-kernel path, also on full-length truncated rows with a row handed to the
full-histogram pass), verification outputs unchanged by the side output, and
argument errors.
"""

import numpy as np
import pytest
import torch

from oracle import spec_oracle as O
from workloads import CONFIGS, make_inputs, to_host_f64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
TOL = 1e-9


@pytest.fixture(scope="module")
def sv():
    import speculative_decoding_verification_temp_amd as pkg
    pkg.load_library()
    torch.cuda.set_device(DEV)
    return pkg


def _run(sv, x, cfg, m, kb=None):
    v = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, x["target"].dtype)
    sup, res = v.set_residual(m)
    if kb is not None:
        v.set_stops(-1, torch.as_tensor(kb, device=DEV).contiguous(), None)
    tok, alen, hist = v.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"])
    torch.cuda.synchronize()
    return sup.cpu().numpy(), res.cpu().numpy(), alen.cpu().numpy()


def _check(x, cfg, m, sup, res, alen, kb=None, label=""):
    # the call takes the temperature as float32: the oracle uses that value
    T32 = float(np.float32(x["T"]))
    ref_sup, ref_res = O.drift_batch(to_host_f64(x["target"]), to_host_f64(x["draft"]), T32, m,
                                     alen, kb)
    assert np.array_equal(sup, ref_sup), f"{label}: support differs at " \
        f"{np.argwhere(sup != ref_sup)[:5]}"
    both_nan = np.isnan(res) & np.isnan(ref_res)
    same_inf = np.isinf(res) & (res == ref_res)
    close = np.abs(res - ref_res) <= TOL
    assert np.all(both_nan | same_inf | close), f"{label}: residual err " \
        f"{np.nanmax(np.abs(res - ref_res)[~(both_nan | same_inf)])}"
    print(f"{label}: {int((sup >= 0).sum())} support entries checked", flush=True)


@pytest.mark.parametrize("merge", ["in-finish", "own-kernel"])
def test_residual_c2_with_draft_counts(sv, monkeypatch, merge):
    """Per-sequence draft counts and each way a sequence is invalid (a token
    out of range, a draft count above K, a NaN in a target row and in a draft
    row): the merge inside the finish decides validity as the scan does, and
    its own kernel reads the scan's accept lengths."""
    monkeypatch.setenv("SPEC_VERIFY_MERGE_IN_FINISH", "1" if merge == "in-finish" else "0")
    cfg = CONFIGS["c2"].scaled(B=32)
    x = make_inputs(cfg, 3, DEV)
    kb = np.random.default_rng(4).integers(0, cfg.K + 1, cfg.B).astype(np.int32)
    x["tokens"][5, 0] = cfg.V + 3              # invalid sequences
    kb[5] = cfg.K
    kb[7] = cfg.K + 2
    x["target"][9, 0, 100] = float("nan")
    x["draft"][11, 1, 50] = float("nan")
    kb[11] = cfg.K
    sup, res, alen = _run(sv, x, cfg, 32, kb)
    assert alen[5] == -1 and alen[7] == -1 and alen[9] == -1 and alen[11] == -1
    assert (alen >= 0).sum() == cfg.B - 4
    _check(x, cfg, 32, sup, res, alen, kb, f"residual/c2 {merge}")


def test_residual_many_ties_and_small_m(sv):
    cfg = CONFIGS["c2"].scaled(B=16, V=4000)
    x = make_inputs(cfg, 6, DEV)
    for key in ("target", "draft"):
        x[key] = (torch.round(x[key].float() * 2) / 2).to(x[key].dtype).contiguous()
    for m in (1, 7, 64):
        sup, res, alen = _run(sv, x, cfg, m)
        _check(x, cfg, m, sup, res, alen, label=f"residual/ties m={m}")


def test_residual_v_below_m_and_neg_inf(sv):
    cfg = CONFIGS["c2"].scaled(B=8, V=24, K=3)
    x = make_inputs(cfg, 7, DEV)
    x["draft"][2, :, 10:] = float("-inf")      # only 10 finite draft values: -inf in the support
    x["target"][3, 0, :5] = float("-inf")
    sup, res, alen = _run(sv, x, cfg, 32)
    assert np.all(sup[:, :, 24:] == -1)
    _check(x, cfg, 32, sup, res, alen, label="residual/V<m")


def test_residual_70000_way_tie(sv):
    cfg = CONFIGS["c3"].scaled(B=2, K=2)
    x = make_inputs(cfg, 8, DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(9)
    for b in range(cfg.B):
        for i in range(cfg.K):
            perm = torch.randperm(cfg.V, generator=g, device=DEV)
            x["draft"][b, i, perm[:70000]] = 5.0 if b == 0 else -5.0   # a 70000-way tie
    sup, res, alen = _run(sv, x, cfg, 32)
    _check(x, cfg, 32, sup, res, alen, label="residual/70000-way tie")


def test_set_residual_arguments(sv):
    cfg = CONFIGS["c1"]
    v32 = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, torch.float32)
    buf = torch.zeros(cfg.B * cfg.K * 64, dtype=torch.int32, device=DEV)
    dbl = torch.zeros(cfg.B * cfg.K * 64, dtype=torch.float64, device=DEV)
    assert v32.lib.spec_verify_set_residual(v32._h, 32, sv._ptr(buf), sv._ptr(dbl)) == sv.SV_OK
    v = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, torch.bfloat16)
    for m in (0, 65, -1):
        assert v.lib.spec_verify_set_residual(v._h, m, sv._ptr(buf), sv._ptr(dbl)) == sv.SV_EINVAL
    assert v.lib.spec_verify_set_residual(v._h, 8, sv._ptr(buf), None) == sv.SV_EINVAL
    assert v.lib.spec_verify_set_residual(v._h, 8, None, None) == sv.SV_OK
    assert v.lib.spec_verify_set_residual(None, 8, None, None) == sv.SV_EINVAL


@pytest.mark.parametrize("route", ["streaming", "streaming-3seg", "streaming-merge-kernel",
                                   "own-truncated", "own-scalar", "own-one-kernel"])
def test_residual_routes(sv, monkeypatch, route):
    """Every route to the support: the streaming pass's lists (one and three
    segments per row, merged inside the finish or by their own kernel) and
    the kernel that reads the draft rows itself (with truncation, on rows not
    in 16-byte chunks, after the one-kernel path)."""
    monkeypatch.setenv("SPEC_VERIFY_NSEG", "3" if route == "streaming-3seg" else "0")
    monkeypatch.setenv("SPEC_VERIFY_MERGE_IN_FINISH",
                       "0" if route == "streaming-merge-kernel" else "1")
    monkeypatch.setenv("SPEC_VERIFY_FUSED_MIN_B", "1" if route == "own-one-kernel" else "0")
    V = {"own-scalar": 4001, "streaming-3seg": 40000}.get(route, 8000)   # 3 segments need V/8 >= 3072
    cfg = CONFIGS["c2"].scaled(B=24, V=V)
    x = make_inputs(cfg, 11, DEV)
    x["draft"][1] = torch.round(x["draft"][1].float() * 2).to(x["draft"].dtype) / 2   # ties
    x["draft"][2, 0, ::3] = float("-inf")
    v = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, x["target"].dtype)
    if route == "own-truncated":
        v.set_truncation(torch.full((cfg.B,), 50, dtype=torch.int32, device=DEV),
                         torch.full((cfg.B,), 0.9, dtype=torch.float32, device=DEV))
    sup, res = v.set_residual(16)
    tok, alen, hist = v.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"])
    torch.cuda.synchronize()
    _check(x, cfg, 16, sup.cpu().numpy(), res.cpu().numpy(), alen.cpu().numpy(),
           label=f"residual/{route}")


@pytest.mark.parametrize("merge", ["in-finish", "own-kernel"])
def test_residual_second_call_with_draft_counts(sv, monkeypatch, merge):
    """Two calls on one verifier: the first reads every row and leaves its
    candidate lists behind; the second has per-sequence draft counts (and a
    draft count above K), so its streaming pass skips rows whose lists still
    hold the first call's keys. Every output of the second call matches the
    oracle: the skipped positions get -1 and NaN, the others their own rows'
    support."""
    monkeypatch.setenv("SPEC_VERIFY_MERGE_IN_FINISH", "1" if merge == "in-finish" else "0")
    cfg = CONFIGS["c2"].scaled(B=32)
    v = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, torch.bfloat16)
    sup, res = v.set_residual(32)
    x1 = make_inputs(cfg, 21, DEV)
    v.verify(x1["target"], x1["draft"], x1["tokens"], x1["uniforms"], x1["T"])
    torch.cuda.synchronize()
    x2 = make_inputs(cfg, 22, DEV)
    kb = np.random.default_rng(23).integers(0, cfg.K + 1, cfg.B).astype(np.int32)
    kb[3] = cfg.K + 1
    v.set_stops(-1, torch.as_tensor(kb, device=DEV).contiguous(), None)
    tok, alen, hist = v.verify(x2["target"], x2["draft"], x2["tokens"], x2["uniforms"], x2["T"])
    torch.cuda.synchronize()
    a = alen.cpu().numpy()
    assert a[3] == -1 and (a >= 0).sum() == cfg.B - 1
    _check(x2, cfg, 32, sup.cpu().numpy(), res.cpu().numpy(), a, kb,
           f"residual/second call {merge}")


def test_residual_truncated_full_rows(sv):
    """Truncation and the residual side output on full-length c3 rows (the
    row-reading kernel, its wavefronts' thresholds seeded from the
    workgroup's first group): a draft row with a value outside the window
    pass's bins (its row goes on to the full-histogram pass), a draft row
    with a 70000-way tie at the top, -inf values in the support, 40 tied
    values at a row's start and per-sequence draft counts; every position
    against the oracle."""
    cfg = CONFIGS["c3"].scaled(B=6)
    x = make_inputs(cfg, 31, DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(32)
    x["draft"][0, 1, 777] = 200.0                     # outside the window (|x| >= 2^7)
    perm = torch.randperm(cfg.V, generator=g, device=DEV)
    x["draft"][1, 2, perm[:70000]] = 9.0              # a 70000-way tie above every other value
    x["draft"][2, 0, ::2] = float("-inf")
    x["draft"][3, 3, :40] = 30.0                      # the top 40 tied at the row start
    kb = np.array([7, 7, 7, 5, 7, 2], dtype=np.int32)
    v = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, x["target"].dtype)
    v.set_truncation(torch.tensor([50, 20, 0, 1000, 50, 3], dtype=torch.int32, device=DEV),
                     torch.tensor([0.9, 1.0, 0.95, 0.5, 1.0, 0.9], dtype=torch.float32,
                                  device=DEV))
    v.set_stops(-1, torch.as_tensor(kb, device=DEV).contiguous(), None)
    sup, res = v.set_residual(32)
    tok, alen, hist = v.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"])
    torch.cuda.synchronize()
    a = alen.cpu().numpy()
    assert np.all(a >= 0)
    _check(x, cfg, 32, sup.cpu().numpy(), res.cpu().numpy(), a, kb,
           "residual/truncated full rows")


def test_residual_leaves_verification_unchanged(sv):
    """The streaming pass computes its normalisers the same way with the
    top-m lists on: tokens, accept lengths and the histogram are bitwise
    those of a call without the side output."""
    cfg = CONFIGS["c3"].scaled(B=64)
    x = make_inputs(cfg, 12, DEV)
    outs = []
    for m in (0, 32):
        v = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, x["target"].dtype)
        if m:
            v.set_residual(m)
        tok, alen, hist = v.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"])
        torch.cuda.synchronize()
        outs.append((tok.cpu().numpy(), alen.cpu().numpy(), hist.cpu().numpy()))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_residual_c3_sampled(sv):
    """The full c3 batch with m = 32 as bench.py runs it (the streaming pass's
    lists): at every drafted position the support's draft logits, in order,
    are the 32 largest of the row (torch's topk as the checker) and the
    residual is finite; sampled positions match the oracle exactly."""
    cfg = CONFIGS["c3"]
    x = make_inputs(cfg, 13, DEV)
    v = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, x["target"].dtype)
    sup, res = v.set_residual(32)
    tok, alen, hist = v.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"])
    torch.cuda.synchronize()
    valid = alen >= 0
    assert bool(valid.all())
    top = torch.topk(x["draft"].float(), 32, dim=-1).values          # [B, K, 32], descending
    got = torch.gather(x["draft"].float(), 2, sup.long())
    assert torch.equal(got, top)
    assert bool(torch.isfinite(res).all())
    rng = np.random.default_rng(14)
    picks = rng.choice(cfg.B * cfg.K, 48, replace=False)
    T32 = float(np.float32(x["T"]))
    s_np, r_np = sup.cpu().numpy(), res.cpu().numpy()
    for p in picks:
        b, i = divmod(int(p), cfg.K)
        S, r = O.drift_residual(to_host_f64(x["target"][b, i]), to_host_f64(x["draft"][b, i]),
                                T32, 32)
        assert np.array_equal(s_np[b, i], S), (b, i)
        assert np.max(np.abs(r_np[b, i] - r)) <= TOL, (b, i)
    print(f"residual/c3: {cfg.B * cfg.K} positions against topk, {len(picks)} against the oracle",
          flush=True)


@pytest.mark.parametrize("route", ["streaming", "streaming-3seg", "streaming-merge-kernel",
                                   "own-scalar", "own-one-kernel"])
def test_residual_fp32_routes(sv, monkeypatch, route):
    """fp32 logits (64-bit token keys) on every route: the streaming pass's
    lists with one and three segments (merged inside the finish or by their
    own kernel), the row-reading kernel on rows not in 16-byte chunks and
    after the one-kernel path; ties and -inf included."""
    monkeypatch.setenv("SPEC_VERIFY_NSEG", "3" if route == "streaming-3seg" else "0")
    monkeypatch.setenv("SPEC_VERIFY_MERGE_IN_FINISH",
                       "0" if route == "streaming-merge-kernel" else "1")
    monkeypatch.setenv("SPEC_VERIFY_FUSED_MIN_B", "1" if route == "own-one-kernel" else "0")
    V = {"own-scalar": 4001, "streaming-3seg": 20000}.get(route, 8000)   # 3 segments: V/4 >= 3072
    cfg = CONFIGS["c1"].scaled(B=24, V=V)
    x = make_inputs(cfg, 15, DEV)
    x["draft"][1] = torch.round(x["draft"][1] * 2) / 2                  # ties
    x["draft"][2, 0, ::3] = float("-inf")
    x["draft"][3, 1, 7] = -0.0
    x["draft"][3, 1, 9] = 0.0
    v = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, x["target"].dtype)
    sup, res = v.set_residual(24)
    tok, alen, hist = v.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"])
    torch.cuda.synchronize()
    _check(x, cfg, 24, sup.cpu().numpy(), res.cpu().numpy(), alen.cpu().numpy(),
           label=f"residual/fp32 {route}")


def test_residual_c5_sampled(sv):
    """The full c5 batch (fp32, B = 1024, K = 4, its p = q and zero-mass
    sequences) with m = 32: supports against torch's topk at every drafted
    position of a valid sequence, sampled positions against the oracle."""
    cfg = CONFIGS["c5"]
    x = make_inputs(cfg, 16, DEV)
    v = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, x["target"].dtype)
    sup, res = v.set_residual(32)
    tok, alen, hist = v.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"])
    torch.cuda.synchronize()
    valid = (alen >= 0).cpu().numpy()
    top = torch.topk(x["draft"], 32, dim=-1).values
    got = torch.gather(x["draft"], 2, sup.clamp(min=0).long())
    same = (got == top).all(dim=-1).all(dim=-1).cpu().numpy()
    assert np.all(same[valid])
    assert np.all(sup.cpu().numpy()[~valid] == -1)
    rng = np.random.default_rng(17)
    T32 = float(np.float32(x["T"]))
    s_np, r_np = sup.cpu().numpy(), res.cpu().numpy()
    checked = 0
    for p in rng.choice(cfg.B * cfg.K, 40, replace=False):
        b, i = divmod(int(p), cfg.K)
        if not valid[b]:
            continue
        S, r = O.drift_residual(to_host_f64(x["target"][b, i]), to_host_f64(x["draft"][b, i]),
                                T32, 32)
        assert np.array_equal(s_np[b, i], S), (b, i)
        ok = np.isclose(r_np[b, i], r, rtol=0, atol=TOL) | (np.isinf(r) & (r_np[b, i] == r))
        assert np.all(ok), (b, i)
        checked += 1
    print(f"residual/c5: {int(valid.sum()) * cfg.K} positions against topk, {checked} against "
          f"the oracle", flush=True)
