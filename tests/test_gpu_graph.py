"""spec_verify captured into a HIP graph and replayed.

A call never allocates, synchronises or touches the default stream, and its
histogram is zeroed by its first kernel (no memset node), so it can be
captured. The test captures one stochastic call with every option on
(truncation, stopping rules, the draft residual side output, the aux side
outputs), then for several steps copies fresh inputs into the captured
buffers, replays, and compares everything the call writes with an eager
verifier set up the same way on the same inputs, and the tokens with the
oracle. Eager work and synchronisation sit between the replays. A second
case captures plain greedy and margin calls, a third a walk-order call.
"""

import numpy as np
import pytest
import torch

from oracle import spec_oracle as O
from tests.parity import compare
from workloads import CONFIGS, make_inputs, to_host_f64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


@pytest.fixture(scope="module")
def sv():
    import speculative_decoding_verification_temp_amd as pkg
    pkg.load_library()          # fails loudly when the library is missing
    torch.cuda.set_device(DEV)
    return pkg


def _setup(sv, cfg, tk, tp, kb, mx, eos):
    v = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, cfg.torch_dtype, ema_decay=0.9)
    aux = v.enable_aux()
    v.set_truncation(tk, tp)
    v.set_stops(eos, kb, mx)
    sup, res = v.set_residual(16)
    out = (torch.full((cfg.B, cfg.K + 1), -7, dtype=torch.int32, device=DEV),
           torch.full((cfg.B,), -7, dtype=torch.int32, device=DEV),
           torch.full((cfg.K + 1,), -7, dtype=torch.int32, device=DEV))
    return v, aux, sup, res, out


def _snapshot(aux, sup, res, out, v):
    e, s = v.ema()
    torch.cuda.synchronize()
    return [t.clone() for t in out] + [aux[k].clone() for k in ("p_d", "q_d", "z")] + \
        [sup.clone(), res.clone(), e, s]


def _same(a, b, label):
    names = ("tokens", "accept_len", "hist", "p_d", "q_d", "z", "support", "residual", "ema",
             "steps")
    for x, y, n in zip(a, b, names):
        if x.is_floating_point():
            assert torch.equal(torch.nan_to_num(x, nan=-123.0), torch.nan_to_num(y, nan=-123.0)), \
                f"{label}: {n} differs"
        else:
            assert torch.equal(x, y), f"{label}: {n} differs"


@pytest.mark.parametrize("cfg_name", ["c2", "c1"])
def test_graph_replay_with_every_option(sv, cfg_name):
    cfg = CONFIGS[cfg_name]
    rng = np.random.default_rng(61)
    tk = torch.as_tensor(rng.choice([0, 20, 200], cfg.B).astype(np.int32), device=DEV)
    tp = torch.as_tensor(rng.choice([1.0, 0.9, 0.6], cfg.B).astype(np.float32), device=DEV)
    kb = torch.as_tensor(rng.integers(0, cfg.K + 1, cfg.B).astype(np.int32), device=DEV)
    mx = torch.as_tensor(rng.integers(1, cfg.K + 2, cfg.B).astype(np.int32), device=DEV)
    eos = 5
    vg, aux_g, sup_g, res_g, out_g = _setup(sv, cfg, tk, tp, kb, mx, eos)
    ve, aux_e, sup_e, res_e, out_e = _setup(sv, cfg, tk, tp, kb, mx, eos)

    x0 = make_inputs(cfg, 70, DEV)
    buf = {k: x0[k].clone() for k in ("target", "draft", "tokens", "uniforms")}

    def call(v, out, inp):
        v.verify(inp["target"], inp["draft"], inp["tokens"], inp["uniforms"], cfg.T,
                 "stochastic", out=out)

    # warm-up on a side stream, then capture one call
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        call(vg, out_g, buf)
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()
    call(ve, out_e, buf)                 # the eager twin sees the same warm-up call
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(vg, out_g, buf)

    for step in range(4):
        x = make_inputs(cfg, 71 + step, DEV)
        for k in buf:
            buf[k].copy_(x[k])
        for t in out_g:
            t.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(aux_g, sup_g, res_g, out_g, vg)
        call(ve, out_e, x)               # eager work between the replays
        torch.cuda.synchronize()
        ref = _snapshot(aux_e, sup_e, res_e, out_e, ve)
        _same(got, ref, f"{cfg_name} step {step}")
        # and the oracle on the same inputs
        o = O.verify_batch(to_host_f64(x["target"]), to_host_f64(x["draft"]),
                           x["tokens"].cpu().numpy(), x["uniforms"].cpu().double().numpy(),
                           cfg.T, O.MODE_STOCHASTIC, eos=eos, draft_len=kb.cpu().numpy(),
                           max_emit=mx.cpu().numpy(), top_k=tk.cpu().numpy(),
                           top_p=tp.cpu().numpy())
        rep = compare(np.arange(cfg.B), o, out_g[0], out_g[1], "stochastic", None,
                      f"graph/{cfg_name}/step {step}")
        print(f"graph {cfg_name} step {step}: {rep}", flush=True)
    st_g, st_e = vg.stats(), ve.stats()
    assert st_g["sequences"] == st_e["sequences"] and st_g["invalid"] == st_e["invalid"]


@pytest.mark.parametrize("mode", ["greedy", "margin"])
def test_graph_replay_argmax_modes(sv, mode):
    cfg = CONFIGS["c1"].scaled(B=16)
    v = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, cfg.torch_dtype)
    x0 = make_inputs(cfg, 80, DEV, "greedy")
    buf = {k: x0[k].clone() for k in ("target", "tokens")}
    out = (torch.empty((cfg.B, cfg.K + 1), dtype=torch.int32, device=DEV),
           torch.empty((cfg.B,), dtype=torch.int32, device=DEV),
           torch.empty((cfg.K + 1,), dtype=torch.int32, device=DEV))
    v.verify(buf["target"], None, buf["tokens"], None, 1.0, mode, 0.3, out=out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        v.verify(buf["target"], None, buf["tokens"], None, 1.0, mode, 0.3, out=out)
    for step in range(3):
        x = make_inputs(cfg, 81 + step, DEV, "greedy")
        buf["target"].copy_(x["target"])
        buf["tokens"].copy_(x["tokens"])
        g.replay()
        torch.cuda.synchronize()
        ref = O.verify_batch(to_host_f64(x["target"]), None, x["tokens"].cpu().numpy(), None,
                             1.0, O.MODE_GREEDY if mode == "greedy" else O.MODE_MARGIN, 0.3)
        compare(np.arange(cfg.B), ref, out[0], out[1], mode, None, f"graph/{mode}/step {step}")
        assert np.array_equal(out[2].cpu().numpy().astype(np.int64), ref.hist)


@pytest.mark.parametrize("cfg_name,mode", [("c2", "stochastic"), ("c1", "stochastic"),
                                           ("c2", "greedy"), ("c1", "margin"),
                                           ("c2", "truncated")])
def test_graph_replay_walk_order(sv, cfg_name, mode):
    """A walk-order call (its list count is cleared by its first kernel, not
    by a memset) captured once and replayed on fresh inputs with stopping
    rules on: every output equals an eager twin's, the tokens the oracle's
    walk-order reading."""
    cfg = CONFIGS[cfg_name]
    rng = np.random.default_rng(62)
    kb = torch.as_tensor(rng.integers(0, cfg.K + 1, cfg.B).astype(np.int32), device=DEV)
    tk = torch.as_tensor(rng.choice([0, 20, 200], cfg.B).astype(np.int32), device=DEV)
    tp = torch.as_tensor(rng.choice([1.0, 0.9, 0.6], cfg.B).astype(np.float32), device=DEV)

    def setup():
        v = sv.SpecVerifier(cfg.B, cfg.K, cfg.V, cfg.torch_dtype, ema_decay=0.9)
        aux = v.enable_aux()
        v.set_stops(-1, kb, None)
        if mode == "truncated":
            v.set_truncation(tk, tp)
        v.set_walk_order(True)
        out = (torch.full((cfg.B, cfg.K + 1), -7, dtype=torch.int32, device=DEV),
               torch.full((cfg.B,), -7, dtype=torch.int32, device=DEV),
               torch.full((cfg.K + 1,), -7, dtype=torch.int32, device=DEV))
        return v, aux, out

    vg, aux_g, out_g = setup()
    ve, aux_e, out_e = setup()
    stoch = mode in ("stochastic", "truncated")
    gen_mode = "stochastic" if stoch else "greedy"
    x0 = make_inputs(cfg, 90, DEV, gen_mode)
    names = ("target", "draft", "tokens", "uniforms") if stoch else ("target", "tokens")
    buf = {k: x0[k].clone() for k in names}
    aux_keys = ("p_d", "q_d", "z") if stoch else ("p_d", "argmax")

    def call(v, out, inp):
        if stoch:
            v.verify(inp["target"], inp["draft"], inp["tokens"], inp["uniforms"], cfg.T,
                     "stochastic", out=out)
        else:
            v.verify(inp["target"], None, inp["tokens"], None, cfg.T, mode, tau=0.3, out=out)

    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        call(vg, out_g, buf)
    torch.cuda.current_stream(DEV).wait_stream(side)
    call(ve, out_e, buf)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(vg, out_g, buf)
    for step in range(4):
        x = make_inputs(cfg, 91 + step, DEV, gen_mode)
        for k in buf:
            buf[k].copy_(x[k])
        for t in out_g:
            t.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in out_g] + [aux_g[k].clone() for k in aux_keys]
        call(ve, out_e, x)
        torch.cuda.synchronize()
        ref = [t.clone() for t in out_e] + [aux_e[k].clone() for k in aux_keys]
        for a, b in zip(got, ref):
            if a.is_floating_point():
                a, b = torch.nan_to_num(a, nan=-123.0), torch.nan_to_num(b, nan=-123.0)
            assert torch.equal(a, b), f"walk graph {cfg_name} {mode} step {step}"
        m = {"stochastic": O.MODE_STOCHASTIC, "truncated": O.MODE_STOCHASTIC,
             "greedy": O.MODE_GREEDY, "margin": O.MODE_MARGIN}[mode]
        kw = dict(top_k=tk.cpu().numpy(), top_p=tp.cpu().numpy()) if mode == "truncated" else {}
        o = O.verify_batch(to_host_f64(x["target"]),
                           to_host_f64(x["draft"]) if stoch else None,
                           x["tokens"].cpu().numpy(), x["uniforms"].cpu().double().numpy(),
                           cfg.T, m, 0.3, draft_len=kb.cpu().numpy(), walk_order=True, **kw)
        compare(np.arange(cfg.B), o, out_g[0], out_g[1], "stochastic" if stoch else mode, None,
                f"graph/walk/{cfg_name}/{mode}/step {step}")
