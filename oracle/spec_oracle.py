"""Plain fp64 CPU oracle for batched speculative-decoding verification.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module. The product path (the HIP
library and its Python binding) never calls it and shares no code with it.

It states, slowly and literally, what one verification step computes for each
sequence: temperature softmax of every needed logit row, the ordered acceptance
walk, the residual or bonus draw, the emitted tokens, the accepted-length
histogram and a per-slot acceptance EMA. Everything is float64 numpy; nothing is
blocked, fused or reordered.

Sources (the five pages this method is described on), abbreviated below:

  [DVC]   "Speculative Decoding: Draft, Verify, and Correct"
  [SMB]   "Speculative Decoding: How a Small Model Speeds Up a Big One Without
           Changing Its Output"
  [RNR]   "Speculative decoding: why correcting a rejection is not resampling
           from the target"
  [MNW]   "Margins, Not Windows: Training-Free Per-Step Lossy Speculative
           Decoding" (AdaptiveSpec summary)

Conventions the pages leave open, and the reading taken here (each one is also
listed with its reason in the design notes):

  * Acceptance: a draft d is kept with probability min(1, p(d)/q(d)); with one
    supplied uniform u it is kept iff p(d) >= q(d) or u < p(d)/q(d) (strict).
    q(d) = 0 therefore always keeps the draft ([SMB] "Seeing It in Code",
    [RNR] s.2).
  * Uniform consumption: u[b, i] decides position i; u[b, K] drives the single
    correction or bonus draw. Greedy and margin modes use no uniforms.
  * Inverse CDF: weights in index order 0..V-1, C_v the inclusive prefix sum,
    draw = smallest v with C_v > u * C_{V-1}; if rounding leaves no such v, the
    largest v with positive weight. Zero-weight tokens are never drawn.
  * Residual normaliser Z = sum_v max(0, p_v - q_v), summed as a prefix sum in
    index order (never as 1 - sum min(p, q)). Z = 0 after a rejection can only
    come from rounding; the draw then falls back to p_j (counted).
  * Bonus token: always emitted when all K drafts are kept (stochastic: drawn
    from p_K; greedy/margin: argmax of target row K).
  * argmax: lowest index among equal maxima of the raw logits.
  * Margin rule: every position is tested in order; a draft is kept iff it is
    the target argmax or p(d)/p(argmax) > tau (strict), with p at the call's
    temperature. The first failing position is the rejection and its
    correction is the target argmax.
  * Invalid input: a sequence with a drafted token outside [0, V), or with a
    needed logit row holding NaN or +inf or no finite maximum (all -inf), is
    marked invalid: accept_len -1, tokens all -1, not counted in the histogram,
    EMA untouched. Needed rows: all K+1 target rows, plus all K draft rows in
    stochastic mode.
  * Walk-order reading (optional; stochastic mode, with or without
    truncation, and the greedy and margin modes; [DVC]
    "Verify several proposed tokens in one target pass": at the first
    rejection the correction is drawn and later proposals are discarded;
    [SMB] "Seeing It in Code": the walk over the drafts stops at the first
    disagreement). The rows of position i are read only when the walk
    reaches it, i.e. once every earlier position has been kept. The sequence
    is then invalid only when something the walk reads is unusable: the
    drafted token or the target or draft row of a position up to the first
    rejection, or target row k_b when every position is kept; rows past the
    first rejection are never looked at. End-of-sequence and budget stops
    cut the emission, not the reading. p(d) and q(d) are NaN past the first
    rejection. In the greedy and margin modes the walk reads target rows
    only, stops at the first position that fails its rule, and the argmax
    side output is -1 for the rows it does not read (the margin ratio NaN).
    With truncation every row the walk reads is truncated as in the full
    reading (top_p <= 0 or NaN still makes the sequence invalid), and only
    those rows' top-p cuts count among the decisions. With every row and
    token usable the result equals that of the full reading (the argmax side
    output aside).
  * EMA: per call and slot, x = accept_len / K; the first observation of a slot
    sets it, later ones do ema = decay * ema + (1 - decay) * x.
  * Stopping rules ([DVC] "Verify several proposed tokens in one target pass"
    and "Speculation needs cache rollback": end-of-sequence and length limits
    may end a cycle before the draft block is used up, and the returned tokens
    must agree with them). Optional per call: an end-of-sequence token id eos
    (-1 = none), and per sequence a draft count k_b in [0, K] and an emission
    budget m_b >= 1. The walk tests positions 0..k_b-1 only (j <= k_b, the
    bonus comes from target row k_b); the candidate emission d_0..d_{j-1}, c is
    cut after its first eos and to its first m_b tokens; accept_len is the
    number of drafts emitted; the correction or bonus c is drawn only when it
    is emitted (still with u[b, K]). Needed rows become target rows 0..k_b and
    draft rows 0..k_b-1; k_b outside [0, K] or m_b < 1 makes the sequence
    invalid. The EMA observes accept_len / k_b and skips sequences with
    k_b = 0. With eos = -1, k_b = K and m_b >= K + 1 every rule above reduces
    to the plain cycle.
  * Truncation ([RNR] s.1: p and q are the distributions the samplers really
    use, after temperature, masks and truncation; s.2: a mask applied only
    after the correction breaks the guarantee). Optional per sequence: top_k
    and top_p, applied in that order to every target and draft row of a
    stochastic sequence before anything else uses p or q (greedy and margin
    modes do not sample and ignore them). top-k (1 <= top_k < V) keeps the
    tokens whose logit is at least the top_k-th largest logit counted with
    multiplicity, so a tie at the cut keeps every tied token. top-p
    (top_p < 1) then keeps, on the renormalised top-k distribution, each
    token whose kept tokens with strictly larger logits hold less than top_p
    of the mass: whole value levels from the top, up to and including the
    first level at which the mass reaches top_p. The kept tokens are
    renormalised; dropped tokens get probability exactly 0 in the acceptance
    ratio, the residual and the bonus draw. top_k <= 0 or >= V and
    top_p >= 1 mean no truncation; top_p <= 0 or NaN makes the sequence
    invalid.
  * Tree-shape policy ([MNW] s.3, dynamic draft tree-shaping), optional,
    after the EMA update of each sequence: a draft confidence score
    DCS = min(1, conf * acc / d) from the draft's top-1 probability conf
    (supplied by the caller, in [0, 1]), the slot's rolling acceptance acc
    (the EMA; [MNW]'s alpha = 0.3 is decay 0.7) and a saturation divisor d > 0
    (the pages give neither the combination nor d: this product is a reading,
    and the part of the policy that is parity-unpinned). The next shape
    (nsteps, top-k, ndt) interpolates linearly from (3, 4, 4) at DCS = 0 to
    (7, 1, 8) at DCS = 1, each rounded half up. Five consecutive zero-accept
    steps (accept_len = 0 with k_b > 0) restore the starting shape (3, 4, 4)
    and restart the slot's EMA. Invalid sequences and conf outside [0, 1]
    give shape (-1, -1, -1) and leave the policy state alone.
  * Draft residual side output ([DRIFT] "The update rule and its objective":
    at every drafted position both distributions are restricted to a shared
    top-m support and the residual is the target log-probability minus the
    draft log-probability there; m = 32 in "Ablations"). Optional, stochastic
    mode: for each valid sequence and position i < k_b, the support S is the
    m tokens with the largest draft logits (ties to the lower index; all V
    tokens when V <= m), listed by descending draft logit then index; both
    temperature softmaxes are restricted to S and renormalised, and
    r(v) = log p_S(v) - log q_S(v) = (x_t(v) - x_d(v)) / T
           - log sum_S exp(x_t / T) + log sum_S exp(x_d / T).
    "Shared top m" is read as the draft's top m (the candidates the draft's
    bias adjusts). Other positions and invalid sequences: support -1,
    residual NaN.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

MODE_STOCHASTIC = 0
MODE_GREEDY = 1
MODE_MARGIN = 2


# --------------------------------------------------------------------------
# Distributions
# --------------------------------------------------------------------------

def row_is_valid(x) -> bool:
    """A logit row is usable iff it has no NaN, no +inf and a finite maximum."""
    x = np.asarray(x, dtype=np.float64)
    if x.size == 0:
        return False
    if np.isnan(x).any() or np.isposinf(x).any():
        return False
    return bool(np.isfinite(x.max()))


def softmax_t(x, T: float) -> np.ndarray:
    """Sampling distribution of one logit row at temperature T.

    p(v) = exp((x_v - M) / T) / sum_w exp((x_w - M) / T), M = max_w x_w.
    The distribution that acceptance and correction use must be the one the
    sampler really draws from, i.e. after temperature ([DVC] "Preserve the
    distribution you actually intend"; [RNR] s.1). -inf logits get exactly 0.
    """
    x = np.asarray(x, dtype=np.float64)
    M = x.max()
    e = np.exp((x - M) / float(T))
    return e / e.sum()


def truncation_keep(x, T: float, top_k: int = 0, top_p: float = 1.0):
    """Tokens kept by top-k and then top-p truncation of one logit row.

    Returns (keep mask, top-p boundary distance). The distance is the
    smallest |mass above a level - top_p| over the value levels of the top-k
    set (mass in units of the renormalised top-k distribution): how close
    the top-p cut came to moving. inf when top-p is off.
    """
    x = np.asarray(x, dtype=np.float64)
    V = x.size
    keep = np.ones(V, dtype=bool)
    if 1 <= top_k < V:
        kth = np.sort(x)[::-1][top_k - 1]      # k-th largest, with multiplicity
        keep &= x >= kth
    dist = math.inf
    if top_p < 1.0:
        p = softmax_t(x, T)
        w = np.where(keep, p, 0.0)
        w = w / w.sum()
        # the kept tokens by value, largest first, grouped into value levels
        vals, ws = x[keep], w[keep]
        order = np.argsort(-vals, kind="stable")
        vals, ws = vals[order], ws[order]
        starts = np.flatnonzero(np.concatenate([[True], vals[1:] != vals[:-1]]))
        level_mass = np.add.reduceat(ws, starts)
        above = 0.0                    # mass of the levels above the current one
        lowest_kept = vals[0]
        for s0, m in zip(starts, level_mass):
            dist = min(dist, abs(above - top_p))
            if above < top_p:
                lowest_kept = vals[s0]
            above += m
        keep &= x >= lowest_kept
    return keep, dist


def truncated_softmax(x, T: float, top_k: int = 0, top_p: float = 1.0):
    """p after temperature and truncation: softmax_t restricted to the kept
    tokens and renormalised. Returns (p, top-p boundary distance)."""
    keep, dist = truncation_keep(x, T, top_k, top_p)
    p = np.where(keep, softmax_t(x, T), 0.0)
    return p / p.sum(), dist


def argmax_lowest(x) -> int:
    """Index of the largest raw logit; the lowest index wins a tie."""
    x = np.asarray(x, dtype=np.float64)
    M = x.max()
    return int(np.flatnonzero(x == M)[0])


# --------------------------------------------------------------------------
# One-position building blocks ([DVC] "Name the two distributions at one
# prefix", "Why the correction recovers the target"; [RNR] s.2)
# --------------------------------------------------------------------------

def acceptance_probability(p, q) -> np.ndarray:
    """a(v) = min(1, p(v) / q(v)); a(v) = 1 where q(v) = 0 (p >= q there)."""
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    a = np.ones_like(p)
    lo = p < q
    a[lo] = p[lo] / q[lo]
    return a


def accepted_mass(p, q) -> np.ndarray:
    """Mass that reaches each token through an accepted proposal: q(v) a(v)."""
    q = np.asarray(q, dtype=np.float64)
    return q * acceptance_probability(p, q)


def positive_residual(p, q):
    """Unnormalised residual [p - q]_+ and its index-order total Z.

    Z is the rejection probability: it equals 1 - sum min(p, q) when both sum
    to one, but is computed from the positive parts so that p = q gives
    exactly 0 ([DVC] "Why the correction recovers the target"; [RNR] s.2).
    """
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    r = np.maximum(p - q, 0.0)
    Z = float(np.cumsum(r)[-1]) if r.size else 0.0
    return r, Z


def residual_distribution(p, q) -> np.ndarray:
    """Normalised residual r = [p - q]_+ / Z (undefined when Z = 0)."""
    r, Z = positive_residual(p, q)
    if Z <= 0.0:
        raise ZeroDivisionError("residual undefined: Z = 0 (p == q)")
    return r / Z


def inverse_cdf(w, u: float):
    """Draw from the weights w with one uniform u in [0, 1).

    Returns (token, boundary_distance). token = smallest v with C_v > u * C_end
    where C is the inclusive prefix sum in index order; when rounding leaves no
    such v, the largest v with w_v > 0. The distance is how far u lies from the
    nearest edge of the chosen token's interval, in u units.
    """
    w = np.asarray(w, dtype=np.float64)
    C = np.cumsum(w)
    total = C[-1]
    t = float(u) * total
    v = int(np.searchsorted(C, t, side="right"))
    if v >= w.size:
        v = int(np.flatnonzero(w > 0.0)[-1])
    lo = C[v - 1] / total if v > 0 else 0.0
    hi = C[v] / total
    dist = min(abs(float(u) - lo), abs(float(u) - hi))
    return v, dist


# --------------------------------------------------------------------------
# One sequence ([DVC] "Verify several proposed tokens in one target pass";
# [SMB] "The Guarantee Behind Rejection Sampling"; [RNR] s.5; [MNW] s.3)
# --------------------------------------------------------------------------

@dataclass
class SequenceResult:
    tokens: np.ndarray            # [K+1] int64, -1 after the last emitted token
    accept_len: int               # drafts emitted (plain cycle: j, emitted = j + 1); -1 if invalid
    p_d: np.ndarray               # [K] p_i(d_i) (stochastic); margin ratio (margin); NaN (greedy)
    q_d: np.ndarray               # [K] q_i(d_i) (stochastic); NaN otherwise
    z: float                      # residual Z at j (stochastic, j < k_b, correction emitted); -1 otherwise
    argmax: np.ndarray            # [K+1] lowest-index argmax of target rows 0..k_b, else -1
    min_dist: float               # smallest boundary distance among decisions taken
    zero_q_accepts: int = 0
    z0_fallback: int = 0
    valid: bool = True
    dists: list = field(default_factory=list)
    draft_len: int = -1           # k_b used by the walk


def verify_sequence(target, draft, tokens, u, T: float, mode: int,
                    tau: float = 0.0, eos: int = -1, draft_len: int | None = None,
                    max_emit: int | None = None, top_k: int = 0,
                    top_p: float = 1.0, walk_order: bool = False) -> SequenceResult:
    """Verify one sequence.

    target: [K+1, V] logits, draft: [K, V] logits (stochastic only),
    tokens: [K] drafted tokens, u: [K+1] uniforms (stochastic only).
    eos, draft_len (k_b) and max_emit (m_b) are the optional stopping rules,
    top_k and top_p the optional truncation, walk_order the optional reading
    of the rows in walk order, all as in the module docstring; the defaults
    give the plain cycle.
    """
    target = np.asarray(target, dtype=np.float64)
    K = target.shape[0] - 1
    V = target.shape[1]
    kb = K if draft_len is None else int(draft_len)
    m = K + 1 if max_emit is None else int(max_emit)
    toks = np.asarray(tokens, dtype=np.int64).reshape(K)
    nan_k = np.full(K, np.nan)
    out = np.full(K + 1, -1, dtype=np.int64)
    walk_order = bool(walk_order)

    valid = 0 <= kb <= K and m >= 1
    if mode == MODE_STOCHASTIC:
        draft = np.asarray(draft, dtype=np.float64)
    if not walk_order:       # (walk order: rows and tokens are checked as the walk reads them)
        valid = valid and bool(np.all((toks[:kb] >= 0) & (toks[:kb] < V)))
        valid = valid and all(row_is_valid(target[i]) for i in range(kb + 1))
        if mode == MODE_STOCHASTIC:
            valid = valid and all(row_is_valid(draft[i]) for i in range(kb))
            valid = valid and float(top_p) > 0.0      # NaN compares false
    elif mode == MODE_STOCHASTIC:
        valid = valid and float(top_p) > 0.0          # (a parameter, not a row)
    # per-row argmax side output: rows 0..k_b (rows past k_b are not read)
    argmax = np.array([argmax_lowest(target[i]) if i <= kb and row_is_valid(target[i]) else -1
                       for i in range(K + 1)], dtype=np.int64)
    if not valid:
        return SequenceResult(out, -1, nan_k.copy(), nan_k.copy(), -1.0, argmax,
                              math.inf, valid=False)
    if walk_order and mode != MODE_STOCHASTIC:
        # greedy and margin walks in walk order: position i's target row is
        # read once every earlier position is kept; the walk stops at the
        # first position that fails its rule or whose row or token is not
        # usable, and reads target row k_b when every position is kept
        t = kb
        for i in range(kb):
            if not (0 <= toks[i] < V and row_is_valid(target[i])):
                t = i
                break
            if toks[i] == argmax[i]:
                continue
            if mode == MODE_MARGIN:
                p = softmax_t(target[i], T)
                if p[toks[i]] / p[argmax[i]] > tau:
                    continue
            t = i
            break
        argmax[t + 1:] = -1        # rows the walk does not read
        usable = row_is_valid(target[t]) and (t == kb or 0 <= toks[t] < V)
        if not usable:
            return SequenceResult(out, -1, nan_k.copy(), nan_k.copy(), -1.0, argmax,
                                  math.inf, valid=False)

    acc_dists = []       # (position, distance of that position's decision)
    zero_q = 0
    p_d = nan_k.copy()
    q_d = nan_k.copy()

    # 1. the ordered walk over positions 0..kb-1: j = first rejection, else kb
    if mode == MODE_STOCHASTIC:
        u = np.asarray(u, dtype=np.float64).reshape(K + 1)

        def kept(i):
            """The acceptance test of position i (counts q(d) = 0 accepts and
            records the decision's distance to its boundary)."""
            nonlocal zero_q
            P, Q = p_d[i], q_d[i]
            if P >= Q:
                if Q == 0.0:
                    zero_q += 1
                if Q > 0.0:
                    acc_dists.append((i, abs(u[i] - P / Q)))
                return True
            ratio = P / Q
            acc_dists.append((i, abs(u[i] - ratio)))
            return bool(u[i] < ratio)

        j = kb
        if walk_order:
            # read position i's rows only once the walk reaches it; a row or
            # token the walk reads that is not usable makes the sequence
            # invalid, later ones are never looked at; each row read is
            # truncated, and its top-p cut is a decision too
            p_rows, q_rows = [], []
            for i in range(kb):
                if not (0 <= toks[i] < V and row_is_valid(target[i])
                        and row_is_valid(draft[i])):
                    return SequenceResult(out, -1, nan_k.copy(), nan_k.copy(), -1.0, argmax,
                                          math.inf, valid=False)
                pi, dt = truncated_softmax(target[i], T, top_k, top_p)
                qi, dq = truncated_softmax(draft[i], T, top_k, top_p)
                acc_dists += [(-1, d) for d in (dt, dq) if d < math.inf]
                p_rows.append(pi)
                q_rows.append(qi)
                p_d[i] = p_rows[i][toks[i]]
                q_d[i] = q_rows[i][toks[i]]
                if not kept(i):
                    j = i
                    break
            if j == kb:
                if not row_is_valid(target[kb]):
                    return SequenceResult(out, -1, nan_k.copy(), nan_k.copy(), -1.0, argmax,
                                          math.inf, valid=False)
                pb, db = truncated_softmax(target[kb], T, top_k, top_p)
                acc_dists += [(-1, db)] if db < math.inf else []
                p_rows.append(pb)
        else:
            tp = [truncated_softmax(target[i], T, top_k, top_p) for i in range(kb + 1)]
            tq = [truncated_softmax(draft[i], T, top_k, top_p) for i in range(kb)]
            p_rows = [p for p, _ in tp]
            q_rows = [q for q, _ in tq]
            # a top-p cut close to moving is a decision too (every needed row)
            acc_dists += [(-1, d) for _, d in tp + tq if d < math.inf]
            for i in range(kb):
                p_d[i] = p_rows[i][toks[i]]
                q_d[i] = q_rows[i][toks[i]]
            for i in range(kb):
                if not kept(i):
                    j = i
                    break
    elif mode == MODE_GREEDY:
        j = kb
        for i in range(kb):
            if toks[i] != argmax[i]:
                j = i
                break
    elif mode == MODE_MARGIN:
        for i in range(kb):
            if argmax[i] >= 0:       # (walk order: rows past the walk are not read)
                p = softmax_t(target[i], T)
                p_d[i] = p[toks[i]] / p[argmax[i]]
        j = kb
        for i in range(kb):
            if toks[i] == argmax[i]:
                continue
            acc_dists.append((i, abs(p_d[i] - tau)))
            if not (p_d[i] > tau):
                j = i
                break
    else:
        raise ValueError(f"unknown mode {mode}")

    # 2. stopping rules: emission d_0..d_{j-1}, c, cut after the first eos
    #    among the kept drafts and to m tokens
    L = j + 1
    for i in range(j):
        if toks[i] == eos:
            L = i + 1
            break
    L = min(L, m)
    n_drafts = min(j, L)
    emit_c = L > j

    # 3. the correction (j < kb) or bonus (j = kb), only when it is emitted
    z = -1.0
    z0 = 0
    c = -1
    draw_dist = None
    if emit_c:
        if mode == MODE_STOCHASTIC:
            if j < kb:
                r, Z = positive_residual(p_rows[j], q_rows[j])
                z = Z
                if Z > 0.0:
                    c, draw_dist = inverse_cdf(r, u[K])
                else:
                    z0 += 1
                    c, draw_dist = inverse_cdf(p_rows[j], u[K])
            else:
                c, draw_dist = inverse_cdf(p_rows[kb], u[K])
        else:
            c = int(argmax[j])

    # decisions at positions the emission reaches are the ones that matter
    dists = [d for (i, d) in acc_dists if i < L]
    if draw_dist is not None:
        dists.append(draw_dist)

    out[:n_drafts] = toks[:n_drafts]
    if emit_c:
        out[j] = c
    return SequenceResult(out, n_drafts, p_d, q_d, z, argmax,
                          min(dists) if dists else math.inf,
                          zero_q_accepts=zero_q, z0_fallback=z0, valid=True,
                          dists=dists, draft_len=kb)


# --------------------------------------------------------------------------
# Batch, histogram and EMA ([RNR] s.7 on recording the accepted-length
# distribution; [MNW] s.3 on a rolling acceptance history)
# --------------------------------------------------------------------------

class EmaState:
    """Per-slot acceptance EMA: float64 value and observation count."""

    def __init__(self, n_slots: int, decay: float):
        self.decay = float(decay)
        self.ema = np.zeros(n_slots, dtype=np.float64)
        self.steps = np.zeros(n_slots, dtype=np.int64)

    def observe(self, slot: int, x: float) -> None:
        if self.steps[slot] == 0:
            self.ema[slot] = x
        else:
            self.ema[slot] = self.decay * self.ema[slot] + (1.0 - self.decay) * x
        self.steps[slot] += 1


def draft_topm_support(draft_row, m: int) -> np.ndarray:
    """The m tokens with the largest draft logits, ties to the lower index,
    in that order (all tokens when V <= m)."""
    x = np.asarray(draft_row, dtype=np.float64)
    order = np.lexsort((np.arange(x.size), -x))
    return order[:min(m, x.size)]


def drift_residual(target_row, draft_row, T: float, m: int):
    """(support, residual) of one drafted position: log p_S - log q_S on the
    draft's top-m support S, both laws restricted to S and renormalised."""
    S = draft_topm_support(draft_row, m)
    xt = np.asarray(target_row, dtype=np.float64)[S] / float(T)
    xd = np.asarray(draft_row, dtype=np.float64)[S] / float(T)

    def lse(v):
        mx = v.max()
        return mx + math.log(np.exp(v - mx).sum())

    return S, (xt - lse(xt)) - (xd - lse(xd))


def drift_batch(target, draft, T: float, m: int, accept_len, draft_len=None):
    """Side output for a batch: support [B, K, m] (-1 where not defined) and
    residual [B, K, m] (NaN there), for valid sequences (accept_len >= 0)
    and positions i < k_b. Slots past V (V < m) stay -1 / NaN."""
    B, K = draft.shape[0], draft.shape[1]
    sup = np.full((B, K, m), -1, dtype=np.int64)
    res = np.full((B, K, m), np.nan)
    for b in range(B):
        if accept_len[b] < 0:
            continue
        kb = K if draft_len is None else int(draft_len[b])
        for i in range(kb):
            S, r = drift_residual(target[b, i], draft[b, i], T, m)
            sup[b, i, :S.size] = S
            res[b, i, :S.size] = r
    return sup, res


START_SHAPE = (3, 4, 4)      # (nsteps, top-k, ndt): wide and shallow
DEEP_SHAPE = (7, 1, 8)       # deep and narrow
BREAKER_STEPS = 5


def shape_for(dcs: float):
    """(nsteps, top-k, ndt) at confidence dcs in [0, 1]: each component moves
    linearly from START_SHAPE to DEEP_SHAPE, rounded half up."""
    return tuple(int(math.floor(a + (b - a) * dcs + 0.5)) for a, b in zip(START_SHAPE, DEEP_SHAPE))


class TreePolicy:
    """Per-slot tree-shape policy state (the zero-accept streak) and step."""

    def __init__(self, n_slots: int, d: float):
        self.d = float(d)
        self.streak = np.zeros(n_slots, dtype=np.int64)

    def step(self, ema: EmaState, slot: int, valid: bool, accept_len: int, draft_len: int,
             conf: float):
        """Shape for the next step of `slot`, after its EMA update; returns
        (shape, dcs)."""
        conf = float(conf)
        if not valid or not (0.0 <= conf <= 1.0):
            return (-1, -1, -1), math.nan
        if draft_len > 0:
            self.streak[slot] = self.streak[slot] + 1 if accept_len == 0 else 0
        if self.streak[slot] >= BREAKER_STEPS:
            self.streak[slot] = 0
            ema.ema[slot] = 0.0
            ema.steps[slot] = 0
            return START_SHAPE, 0.0
        acc = ema.ema[slot] if ema.steps[slot] > 0 else 0.0
        dcs = min(1.0, conf * acc / self.d)
        return shape_for(dcs), dcs


@dataclass
class BatchResult:
    tokens: np.ndarray        # [B, K+1] int64
    accept_len: np.ndarray    # [B] int64
    hist: np.ndarray          # [K+1] int64
    p_d: np.ndarray           # [B, K]
    q_d: np.ndarray           # [B, K]
    z: np.ndarray             # [B]
    argmax: np.ndarray        # [B, K+1]
    min_dist: np.ndarray      # [B]
    zero_q_accepts: int
    z0_fallbacks: int
    invalid: int
    shape: np.ndarray = None  # [B, 3] next tree shape (policy only)
    dcs: np.ndarray = None    # [B] draft confidence score (policy only)
    n_decisions: int = 0      # decisions with a boundary distance (tests, draws, cuts)


def verify_batch(target, draft, tokens, uniforms, T: float, mode: int,
                 tau: float = 0.0, ema: EmaState | None = None,
                 rows=None, eos: int = -1, draft_len=None, max_emit=None,
                 top_k=None, top_p=None, policy: TreePolicy | None = None,
                 conf=None, walk_order: bool = False) -> BatchResult:
    """Verify every sequence b (or only those listed in `rows`).

    target [B, K+1, V], draft [B, K, V] (stochastic), tokens [B, K],
    uniforms [B, K+1]. Arrays may be any float dtype; they are widened to
    float64 one sequence at a time. When `ema` is given, slot b is updated
    for every valid verified sequence b with k_b > 0. eos, draft_len [B] and
    max_emit [B] (indexed by b) are the optional stopping rules, top_k [B]
    and top_p [B] the optional truncation. With `policy` (which needs `ema`)
    and conf [B] (the draft's top-1 probabilities), each sequence's next
    tree shape is computed after its EMA update. walk_order: the rows are
    read in walk order (module docstring).
    """
    B = target.shape[0]
    K = target.shape[1] - 1
    idx = list(range(B)) if rows is None else [int(b) for b in rows]
    n = len(idx)
    out = BatchResult(
        tokens=np.full((n, K + 1), -1, dtype=np.int64),
        accept_len=np.full(n, -1, dtype=np.int64),
        hist=np.zeros(K + 1, dtype=np.int64),
        p_d=np.full((n, K), np.nan), q_d=np.full((n, K), np.nan),
        z=np.full(n, -1.0), argmax=np.full((n, K + 1), -1, dtype=np.int64),
        min_dist=np.full(n, math.inf), zero_q_accepts=0, z0_fallbacks=0,
        invalid=0)
    if policy is not None:
        out.shape = np.full((n, 3), -1, dtype=np.int64)
        out.dcs = np.full(n, math.nan)
    for k, b in enumerate(idx):
        res = verify_sequence(
            target[b],
            draft[b] if (draft is not None and mode == MODE_STOCHASTIC) else None,
            tokens[b],
            uniforms[b] if (uniforms is not None and mode == MODE_STOCHASTIC) else None,
            T, mode, tau, eos=eos,
            draft_len=None if draft_len is None else int(draft_len[b]),
            max_emit=None if max_emit is None else int(max_emit[b]),
            top_k=0 if top_k is None else int(top_k[b]),
            top_p=1.0 if top_p is None else float(top_p[b]), walk_order=walk_order)
        out.tokens[k] = res.tokens
        out.accept_len[k] = res.accept_len
        out.p_d[k] = res.p_d
        out.q_d[k] = res.q_d
        out.z[k] = res.z
        out.argmax[k] = res.argmax
        out.min_dist[k] = res.min_dist
        out.zero_q_accepts += res.zero_q_accepts
        out.z0_fallbacks += res.z0_fallback
        out.n_decisions += len(res.dists)
        if res.valid:
            out.hist[res.accept_len] += 1
            if ema is not None and res.draft_len > 0:
                ema.observe(b, res.accept_len / res.draft_len)
        else:
            out.invalid += 1
        if policy is not None:
            shape, dcs = policy.step(ema, b, res.valid, res.accept_len, res.draft_len, conf[b])
            out.shape[k] = shape
            out.dcs[k] = dcs
    return out
