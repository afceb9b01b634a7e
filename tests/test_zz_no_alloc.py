"""The allocation-free entry point (spec_verify_noalloc) against the handle
entry point (spec_verify) on the same inputs: two calls in a row through the
C ABI, the second with a smaller input, on every route it serves; results must
be bitwise identical (the same kernels run, with their workspace in the
library's fixed scratch array instead of the handle's). Sizes past the
array's limit are refused with nothing enqueued."""

import numpy as np
import pytest
import torch

from tests.parity import check_invariants
from workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


@pytest.fixture(scope="module")
def sv():
    import speculative_decoding_verification_temp_amd as pkg
    pkg.load_library()          # fails loudly when the library is missing
    torch.cuda.set_device(DEV)
    return pkg


def _outs(B, K, fill=-7):
    return (torch.full((B, K + 1), fill, dtype=torch.int32, device=DEV),
            torch.full((B,), fill, dtype=torch.int32, device=DEV),
            torch.full((K + 1,), -fill, dtype=torch.int32, device=DEV))


def _both(sv, x, mode, tau=0.0):
    """(handle outputs, no-alloc outputs) for one input dict."""
    B, K1, V = x["target"].shape
    K = K1 - 1
    v = sv.SpecVerifier(B, K, V, x["target"].dtype)
    ref = v.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], mode, tau)
    got = _outs(B, K)
    sv.verify_noalloc(x["target"], x["draft"], x["tokens"], x["uniforms"], x["T"], mode, tau,
                      got)
    torch.cuda.synchronize()
    v.close()
    return ref, got


def _same(ref, got, label):
    for a, b, name in zip(ref, got, ("tokens", "accept_len", "hist")):
        assert torch.equal(a, b), f"{label}: {name} differs"


@pytest.mark.parametrize("case", ["stochastic", "margin", "greedy"])
def test_noalloc_matches_handle_calls(sv, case):
    if case == "stochastic":
        # c5 at full size (fp32, B = 1024), then c2 (bf16, B = 64), then a
        # scalar-path shape (V = 1001)
        steps = [(CONFIGS["c5"], "stochastic"), (CONFIGS["c2"], "stochastic"),
                 (CONFIGS["c2"].scaled(B=16, K=3, V=1001), "stochastic")]
    else:
        # c4 at full size (B = 128, V = 151936), then a small c1 shape
        steps = [(CONFIGS["c4"], case), (CONFIGS["c1"].scaled(B=3), case)]
    for i, (cfg, mode) in enumerate(steps):
        print(f"noalloc {case} call {i}: {cfg.name} B={cfg.B} K={cfg.K} V={cfg.V}", flush=True)
        x = make_inputs(cfg, 11 + i, DEV, "stochastic" if mode == "stochastic" else "greedy")
        ref, got = _both(sv, x, mode, tau=0.3)
        _same(ref, got, f"{case} call {i}")
        check_invariants(got[0], got[1], got[2], x["tokens"], cfg.V, cfg.K)
        assert int(got[1].min()) >= 0


def test_noalloc_refuses_sizes_past_its_limits(sv):
    L = sv.load_library()
    import ctypes
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # row partials of B = 4096 sequences at K = 7 do not fit in 1 MiB
    B, K, V = 4096, 7, 64
    t = torch.zeros((B, K + 1, V), dtype=torch.bfloat16, device=DEV)
    d = torch.zeros((B, K, V), dtype=torch.bfloat16, device=DEV)
    tok = torch.zeros((B, K), dtype=torch.int32, device=DEV)
    u = torch.zeros((B, K + 1), dtype=torch.float32, device=DEV)
    out = _outs(B, K)
    rc = L.spec_verify_noalloc(B, K, V, 1, p(t), p(d), p(tok), p(u), 1.0, 0, 0.0,
                               *[p(o) for o in out], s)
    assert rc == sv.SV_EINVAL and b"scratch" in L.spec_verify_last_error(None)
    # the stochastic route's vocabulary limit (bf16 in 16-byte chunks)
    B, K, V = 1, 1, 524296
    t = torch.zeros((B, K + 1, V), dtype=torch.bfloat16, device=DEV)
    d = torch.zeros((B, K, V), dtype=torch.bfloat16, device=DEV)
    out2 = _outs(B, K)
    rc = L.spec_verify_noalloc(B, K, V, 1, p(t), p(d), p(tok), p(u), 1.0, 0, 0.0,
                               *[p(o) for o in out2], s)
    assert rc == sv.SV_EUNSUPPORTED
    torch.cuda.synchronize()
    for o in out + out2:
        assert int(o.abs().min()) == 7          # nothing was written
    # the binding checks the caller's outputs before anything is enqueued
    x = make_inputs(CONFIGS["c1"], 0, DEV)
    with pytest.raises(sv.SpecVerifyError):
        sv.verify_noalloc(x["target"], x["draft"], x["tokens"], x["uniforms"], 1.0,
                          "stochastic", 0.0, _outs(3, 4))
