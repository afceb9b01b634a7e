"""Host-side checks of the seeded input generators (no verification arithmetic)."""

import numpy as np
import torch

from workloads import CONFIGS, make_inputs, mc_inputs, const_alpha_inputs, to_host_f64


def _small(name, **kw):
    cfg = CONFIGS[name]
    return cfg.scaled(B=min(cfg.B, 40), V=min(cfg.V, 3000), **kw)


def test_shapes_dtypes_and_determinism():
    for name in CONFIGS:
        cfg = _small(name)
        for mode in cfg.modes:
            a = make_inputs(cfg, step=0, mode=mode)
            b = make_inputs(cfg, step=0, mode=mode)
            B, K, V = cfg.B, cfg.K, cfg.V
            assert a["target"].shape == (B, K + 1, V) and a["target"].dtype == cfg.torch_dtype
            assert a["draft"].shape == (B, K, V) and a["draft"].dtype == cfg.torch_dtype
            assert a["tokens"].shape == (B, K) and a["tokens"].dtype == torch.int32
            assert a["uniforms"].shape == (B, K + 1) and a["uniforms"].dtype == torch.float32
            for k in ("target", "draft", "tokens", "uniforms"):
                assert torch.equal(a[k], b[k])
            assert int(a["tokens"].min()) >= 0 and int(a["tokens"].max()) < V
            u = a["uniforms"].double()
            assert float(u.min()) >= 0.0 and float(u.max()) < 1.0
            assert torch.equal(u * 2 ** 24, torch.floor(u * 2 ** 24))
            c = make_inputs(cfg, step=1, mode=mode)
            assert not torch.equal(a["target"], c["target"])


def test_special_sequences_c5():
    cfg = CONFIGS["c5"].scaled(B=200, V=1000)
    x = make_inputs(cfg)
    pq, z = x["pq_idx"], x["z_idx"]
    assert len(pq) == 10 and len(z) == 10 and not set(pq) & set(z)
    K = cfg.K
    for b in pq:
        assert torch.equal(x["draft"][b], x["target"][b, :K])
    for b in z:
        masked = torch.isinf(x["draft"][b]).all(dim=0)
        assert int(masked.sum()) == 100
        # drafted tokens are never masked tokens (they have zero draft mass)
        assert not masked[x["tokens"][b].long()].any()


def test_peaked_target_c4():
    cfg = CONFIGS["c4"].scaled(B=8, V=5000)
    x = make_inputs(cfg, mode="margin")
    t = to_host_f64(x["target"])
    # one token per row carries the +6 peak on top of N(0, 2^2)
    assert t.max() > 10


def test_mc_and_const_alpha_inputs():
    x = mc_inputs([0.6, 0.3, 0.1], [0.2, 0.5, 0.3], 1000, 5)
    assert x["target"].shape == (1000, 2, 3) and x["draft"].shape == (1000, 1, 3)
    f = np.bincount(x["tokens"].numpy().ravel(), minlength=3) / 1000
    assert abs(f[1] - 0.5) < 0.06
    y = const_alpha_inputs(0.7, 5, 10, 3)
    assert torch.isinf(y["draft"][:, :, 1]).all()


def test_walk_rows_read_accounting():
    """bench.py's count of the logit rows a walk-order call reads: position
    0's rows of every valid sequence (target row 0, and draft row 0 when
    k_b > 0 in stochastic mode), plus the other needed rows (target rows
    1..k_b, draft rows 1..k_b-1) of the sequences whose walk keeps position
    0 (j >= 1); invalid sequences (j = -1) are not counted."""
    import bench
    j = np.array([0, 1, 7, -1, 0, 3])
    kb = np.array([7, 7, 7, 7, 0, 3])
    # stochastic: 2 + (2 + 7 + 6) + (2 + 7 + 6) + 0 + 1 + (2 + 3 + 2)
    assert bench.walk_rows_read(j, kb, "stochastic") == 2 + 15 + 15 + 0 + 1 + 7
    # greedy / margin: target rows only
    assert bench.walk_rows_read(j, kb, "greedy") == 1 + 8 + 8 + 0 + 1 + 4
    assert bench.walk_rows_read(j, kb, "margin") == bench.walk_rows_read(j, kb, "greedy")
