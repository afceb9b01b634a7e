"""Seeded synthetic workloads shaped like the pages' verification setting.

Each configuration fixes B sequences, K drafted positions, a vocabulary of V
tokens, the logit dtype, the temperature and the verification mode(s). Target
logits are Gaussian (one config adds a single peaked token per row); draft
logits are an affine function of the fp32 target plus fresh Gaussian noise,
taken before rounding to the storage dtype. Drafted tokens are drawn from the
draft's own sampling law at the call's temperature (Gumbel-max on the stored
draft logits) for stochastic runs, and are the draft argmax for greedy and
margin runs. Uniforms are fp32 multiples of 2^-24 in [0, 1).

Seeds: numpy SeedSequence([20260923, config, step, stream]) with stream
0 = logits, 1 = draft sampling, 2 = verify uniforms, 3 = special-sequence
selection. Logits are drawn with a torch generator on the requested device,
so a GPU run and its host copy see the same values.

Nothing here computes any part of the verification itself.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch

SEED_BASE = 20260923


@dataclass(frozen=True)
class Config:
    name: str
    index: int
    B: int
    K: int
    V: int
    dtype: str                   # "f32" or "bf16"
    T: float
    modes: tuple                 # subset of ("stochastic", "greedy", "margin")
    tau: float = 0.0
    target_sigma: float = 1.0
    peak: float = 0.0            # added to one uniform-random token per target row
    draft_scale: float = 1.0     # draft = draft_scale * target + N(0, draft_sigma^2)
    draft_sigma: float = 1.0
    frac_pq: float = 0.0         # sequences whose draft rows copy the target rows
    frac_zeroed: float = 0.0     # sequences with draft mass removed on part of V
    zero_frac: float = 0.0       # fraction of V removed in those sequences
    steps: int = 1               # repeated steps (fresh logits each)
    ema_decay: float = 0.99
    note: str = ""

    def scaled(self, **kw) -> "Config":
        return replace(self, **kw)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


CONFIGS = {
    "c1": Config("c1", 1, B=4, K=4, V=1024, dtype="f32", T=1.0, modes=("stochastic",),
                 target_sigma=2.0, draft_scale=1.0, draft_sigma=1.0,
                 note="small fp32 case"),
    "c2": Config("c2", 2, B=64, K=5, V=32000, dtype="bf16", T=0.8, modes=("stochastic",),
                 target_sigma=3.0, draft_scale=0.8, draft_sigma=1.5,
                 note="in-distribution draft"),
    "c3": Config("c3", 3, B=256, K=7, V=128256, dtype="bf16", T=1.0,
                 modes=("stochastic", "greedy"), target_sigma=3.0, draft_scale=0.5,
                 draft_sigma=3.0, steps=600, ema_decay=0.99,
                 note="shifted draft, 600-step EMA run; the headline shape"),
    "c4": Config("c4", 4, B=128, K=8, V=151936, dtype="bf16", T=1.0,
                 modes=("margin", "greedy"), tau=0.3, target_sigma=2.0, peak=6.0,
                 draft_scale=1.0, draft_sigma=2.0,
                 note="peaked target, margin vs greedy"),
    "c5": Config("c5", 5, B=1024, K=4, V=128256, dtype="f32", T=0.7, modes=("stochastic",),
                 target_sigma=2.5, draft_scale=0.7, draft_sigma=2.0,
                 frac_pq=0.05, frac_zeroed=0.05, zero_frac=0.1,
                 note="fp32, p = q and zero-mass special sequences"),
}


def seed_for(cfg_index: int, step: int, stream: int) -> int:
    ss = np.random.SeedSequence([SEED_BASE, int(cfg_index), int(step), int(stream)])
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def special_sequences(cfg: Config, step: int = 0):
    """Disjoint seeded index sets: (p = q sequences, zeroed-mass sequences)."""
    rng = np.random.default_rng(seed_for(cfg.index, step, 3))
    n_pq = int(round(cfg.frac_pq * cfg.B))
    n_z = int(round(cfg.frac_zeroed * cfg.B))
    perm = rng.permutation(cfg.B)
    return np.sort(perm[:n_pq]), np.sort(perm[n_pq:n_pq + n_z]), rng


def uniforms(B: int, K: int, seed: int, device) -> torch.Tensor:
    g = _gen(device, seed)
    u = torch.randint(0, 1 << 24, (B, K + 1), generator=g, device=device, dtype=torch.int64)
    return (u.to(torch.float64) / float(1 << 24)).to(torch.float32)


def _gumbel_max(logits: torch.Tensor, T: float, gen: torch.Generator) -> torch.Tensor:
    """Exact sampler for softmax(logits / T) without forming the softmax."""
    out = torch.empty(logits.shape[:-1], dtype=torch.int64, device=logits.device)
    flat = logits.reshape(-1, logits.shape[-1])
    oflat = out.reshape(-1)
    step = max(1, (1 << 26) // max(1, logits.shape[-1]))
    for r0 in range(0, flat.shape[0], step):
        x = flat[r0:r0 + step].to(torch.float32)
        u = torch.rand(x.shape, generator=gen, device=x.device, dtype=torch.float32)
        u.clamp_(min=1e-30, max=1.0 - 2.0 ** -24)
        g = -torch.log(-torch.log(u))
        oflat[r0:r0 + step] = torch.argmax(x / T + g, dim=-1)
    return out


def make_inputs(cfg: Config, step: int = 0, device="cpu", mode: str | None = None) -> dict:
    """Build one step of a configuration on `device`.

    Returns a dict with target [B, K+1, V], draft [B, K, V] (storage dtype),
    tokens [B, K] int32, uniforms [B, K+1] float32 and the scalars.
    """
    mode = mode or cfg.modes[0]
    B, K, V = cfg.B, cfg.K, cfg.V
    g = _gen(device, seed_for(cfg.index, step, 0))
    t32 = torch.randn((B, K + 1, V), generator=g, device=device, dtype=torch.float32)
    t32.mul_(cfg.target_sigma)
    if cfg.peak:
        pk = torch.randint(0, V, (B, K + 1, 1), generator=g, device=device)
        t32.scatter_add_(2, pk, torch.full((B, K + 1, 1), cfg.peak, device=device))
    d32 = torch.randn((B, K, V), generator=g, device=device, dtype=torch.float32)
    d32.mul_(cfg.draft_sigma).add_(t32[:, :K], alpha=cfg.draft_scale)
    target = t32.to(cfg.torch_dtype)
    del t32
    draft = d32.to(cfg.torch_dtype)
    del d32

    pq_idx, z_idx, rng = special_sequences(cfg, step)
    if len(pq_idx):
        sel = torch.as_tensor(pq_idx, device=device)
        draft[sel] = target[sel, :K]
    if len(z_idx):
        nz = int(math.floor(cfg.zero_frac * V))
        for b in z_idx:
            toks = torch.as_tensor(rng.choice(V, size=nz, replace=False), device=device)
            draft[int(b)][:, toks] = float("-inf")

    g1 = _gen(device, seed_for(cfg.index, step, 1))
    if mode == "stochastic":
        tokens = _gumbel_max(draft, cfg.T, g1)
    else:
        tokens = torch.argmax(draft.to(torch.float32), dim=-1)
    u = uniforms(B, K, seed_for(cfg.index, step, 2), device)
    return dict(target=target, draft=draft, tokens=tokens.to(torch.int32).contiguous(),
                uniforms=u, T=cfg.T, mode=mode, tau=cfg.tau, cfg=cfg, step=step,
                pq_idx=pq_idx, z_idx=z_idx)


def window_edge_inputs(cfg: Config, step: int = 0, device="cpu") -> dict:
    """bf16-style logits that reach every special value a float64 exponential
    table over 2^-25 <= |x| < 2^7 does not cover. In a seeded ~2.2% of the
    entries of every target and draft row: +-0.0 (1%), +-2^-30 (0.5%), -inf
    (0.5%) and values in (-228, -128] (0.2%); in the target rows of even
    sequences also +150 at ~0.02% of the entries, which then dominate p.
    Drafted tokens are sampled from the modified draft rows at T."""
    x = make_inputs(cfg, step, device, "stochastic")
    g = _gen(device, seed_for(cfg.index, step, 4))
    for key in ("target", "draft"):
        t = x[key].to(torch.float32)
        u = torch.rand(t.shape, generator=g, device=device)
        sgn = torch.where(torch.rand(t.shape, generator=g, device=device) < 0.5, -1.0, 1.0)
        big = -128.0 - 100.0 * torch.rand(t.shape, generator=g, device=device)
        t = torch.where(u < 0.010, 0.0 * sgn, t)
        t = torch.where((u >= 0.010) & (u < 0.015), sgn * 2.0 ** -30, t)
        t = torch.where((u >= 0.015) & (u < 0.020), torch.full_like(t, float("-inf")), t)
        t = torch.where((u >= 0.020) & (u < 0.022), big, t)
        if key == "target":
            even = (torch.arange(cfg.B, device=device) % 2 == 0).view(-1, 1, 1)
            t = torch.where(even & (u >= 0.9998), torch.full_like(t, 150.0), t)
        x[key] = t.to(cfg.torch_dtype).contiguous()
    g1 = _gen(device, seed_for(cfg.index, step, 5))
    x["tokens"] = _gumbel_max(x["draft"], cfg.T, g1).to(torch.int32).contiguous()
    return x


def _log(p) -> np.ndarray:
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, dtype=np.float64))


def mc_inputs(p, q, N: int, seed: int, device="cpu", K: int = 1) -> dict:
    """N independent one-draft sequences whose rows are the given laws:
    target rows = log p, draft rows = log q, drafts drawn from q."""
    rng = np.random.default_rng(seed)
    V = len(p)
    d = rng.choice(V, size=(N, K), p=np.asarray(q, dtype=np.float64))
    u = (rng.integers(0, 1 << 24, size=(N, K + 1)) / float(1 << 24)).astype(np.float32)
    lt = torch.as_tensor(_log(p), dtype=torch.float32)
    lq = torch.as_tensor(_log(q), dtype=torch.float32)
    target = lt.expand(N, K + 1, V).contiguous().to(device)
    draft = lq.expand(N, K, V).contiguous().to(device)
    return dict(target=target, draft=draft,
                tokens=torch.as_tensor(d, dtype=torch.int32).to(device),
                uniforms=torch.as_tensor(u).to(device), T=1.0, mode="stochastic", tau=0.0)


def const_alpha_inputs(alpha: float, K: int, B: int, seed: int, device="cpu") -> dict:
    """V = 2, draft law (1, 0), target law (alpha, 1 - alpha) at every position:
    the draft is always token 0 and is kept with probability alpha."""
    rng = np.random.default_rng(seed)
    u = (rng.integers(0, 1 << 24, size=(B, K + 1)) / float(1 << 24)).astype(np.float32)
    t = torch.as_tensor(_log([alpha, 1.0 - alpha]), dtype=torch.float32)
    d = torch.as_tensor(_log([1.0, 0.0]), dtype=torch.float32)
    return dict(target=t.expand(B, K + 1, 2).contiguous().to(device),
                draft=d.expand(B, K, 2).contiguous().to(device),
                tokens=torch.zeros((B, K), dtype=torch.int32, device=device),
                uniforms=torch.as_tensor(u).to(device), T=1.0, mode="stochastic", tau=0.0)


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a logit tensor (bf16 or fp32) to a float64 host array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
