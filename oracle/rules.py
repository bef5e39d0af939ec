"""Oracle: the commit rules, the schedule and the block helpers (test infrastructure).

Source: mlx-arsenal research note "dLLM block decoding" -- the function table in
"What mlx-arsenal ships" (one row per rule), the swaps listed under "Reference
loop", the LLaDA2.1 loop in "Token editing (LLaDA2.1)", the "Mask conventions"
paragraph, and "Deviations from the references" (stable ties, exactly one forced
token, no factor off-by-one, per-row quotas).  Also mojo-dllm "The loop LLaDA
uses" (even per-step quotas, top-k commit) and mlxcel "Block Diffusion"
("LLaDA-2 Block Unmasking": reveal the single highest when none qualifies;
"Samplers and Reveal Policies": at least one position accepted).

Conventions of this oracle (and of the library it checks):
  * every score is a float32 value; comparisons against tau / f / gamma
    (Python floats, i.e. float64) are exact;
  * a NaN score is the worst possible score: -inf for a confidence, +inf for an
    entropy;  -0.0 and +0.0 are equal (ties broken by position);
  * rankings are Python's stable sort on an explicit key, so equal scores keep
    the lower position first;
  * the two rules that compare an arithmetic expression -- factor and
    entropy-bound -- evaluate it exactly (fractions.Fraction), so the result is
    the mathematical one and does not depend on summation order;
  * B and L come from the arrays; outputs are numpy bool (B, L) masks.
"""
import math
from fractions import Fraction

import numpy as np


def _f32(a, name):
    a = np.asarray(a)
    if a.dtype != np.float32:
        raise TypeError(f"{name} must be float32")
    return a


def _mask(a, name):
    a = np.asarray(a)
    if a.dtype != np.bool_:
        raise TypeError(f"{name} must be bool")
    return a


def _conf(c):
    c = float(c)
    return -math.inf if math.isnan(c) else c


def _ent(h):
    h = float(h)
    return math.inf if math.isnan(h) else h


def _check_param(x, name):
    x = float(x)
    if math.isnan(x):
        raise ValueError(f"{name} must not be NaN")
    return x


def _by_confidence(conf_row, cand_row):
    """Candidate positions, most confident first; equal scores keep position order."""
    C = [l for l in range(cand_row.shape[0]) if cand_row[l]]
    return sorted(C, key=lambda l: (-_conf(conf_row[l]), l))


def threshold_transfer(conf, cand, tau, strict=False):
    """Commit every candidate with conf >= tau (> tau when strict); if none passes,
    commit exactly one: the first candidate of maximal confidence.

    Function table, threshold_transfer row; "Deviations": the forced token is the
    first maximal one and exactly one is forced.  tau is one threshold, or a
    (B,) array of thresholds, one per batch row (the per-row threshold
    schedules of mlxcel "Block Diffusion", "LLaDA-2 Block Unmasking").
    """
    conf, cand = _f32(conf, "conf"), _mask(cand, "cand")
    B, L = conf.shape
    taus = np.asarray(tau, dtype=np.float64)
    if taus.ndim == 0:
        taus = np.full(B, float(taus))
    if taus.shape != (B,):
        raise ValueError("tau must be a number or a (B,) array")
    for t in taus:
        _check_param(float(t), "tau")
    out = np.zeros((B, L), dtype=bool)
    for b in range(B):
        tau = float(taus[b])
        C = [l for l in range(L) if cand[b, l]]
        if not C:
            continue
        passed = [l for l in C
                  if (_conf(conf[b, l]) > tau if strict else _conf(conf[b, l]) >= tau)]
        if passed:
            out[b, passed] = True
        else:
            best = max(_conf(conf[b, l]) for l in C)
            first = next(l for l in C if _conf(conf[b, l]) == best)
            out[b, first] = True
    return out


def decaying_threshold(tau_initial, tau_floor, decay, step):
    """max(tau_floor, tau_initial - decay * step): a threshold that falls
    linearly with the step and stops at its floor (mlxcel "Block Diffusion",
    "LLaDA-2 Block Unmasking": an initial / floor confidence threshold, 0.95 by
    default, and a linearly decaying threshold)."""
    if step < 0:
        raise ValueError("step must be >= 0")
    return max(float(tau_floor), float(tau_initial) - float(decay) * int(step))


def topk_transfer(conf, cand, k):
    """Commit the k_b most confident candidates of batch row b (stable order);
    k_b <= 0 commits nothing, k_b >= |C| commits every candidate.

    Function table, topk_transfer row ("k per row"); "Deviations": per-row quotas.
    """
    conf, cand = _f32(conf, "conf"), _mask(cand, "cand")
    k = np.asarray(k)
    B, L = conf.shape
    out = np.zeros((B, L), dtype=bool)
    for b in range(B):
        order = _by_confidence(conf[b], cand[b])
        n = min(max(int(k[b]), 0), len(order))
        out[b, order[:n]] = True
    return out


def _factor_holds(i, c, f):
    """(i + 1) * (1 - c) <= f, exactly."""
    if math.isinf(c):
        prod = -math.inf if c > 0 else math.inf
        return prod <= f
    if math.isinf(f):
        return f > 0
    return (i + 1) * (1 - Fraction(c)) <= Fraction(f)


def factor_transfer(conf, cand, f):
    """Commit the longest prefix of the candidates sorted by decreasing
    confidence c_(0) >= c_(1) >= ... on which (i + 1) * (1 - c_(i)) <= f holds,
    and at least one candidate.

    Function table, factor_transfer row; "Deviations": the reference's off-by-one
    (everything committed when only the last sorted candidate fails) is not kept.
    """
    conf, cand = _f32(conf, "conf"), _mask(cand, "cand")
    f = _check_param(f, "f")
    B, L = conf.shape
    out = np.zeros((B, L), dtype=bool)
    for b in range(B):
        order = _by_confidence(conf[b], cand[b])
        if not order:
            continue
        n = len(order)
        for i, l in enumerate(order):
            if not _factor_holds(i, _conf(conf[b, l]), f):
                n = i
                break
        out[b, order[:max(n, 1)]] = True
    return out


class _ExactSum:
    """Sum of float values over the extended reals, kept exactly."""

    def __init__(self):
        self.finite = Fraction(0)
        self.n_neg_inf = 0
        self.n_pos_inf = 0

    def add(self, h):
        if h == math.inf:
            self.n_pos_inf += 1
        elif h == -math.inf:
            self.n_neg_inf += 1
        else:
            self.finite += Fraction(h)

    def at_most(self, gamma):
        if self.n_pos_inf and self.n_neg_inf:
            return False                      # inf - inf: undefined, the test fails
        if self.n_pos_inf:
            return gamma == math.inf
        if self.n_neg_inf:
            return True
        if math.isinf(gamma):
            return gamma > 0
        return self.finite <= Fraction(gamma)


def entropy_bound_transfer(entropy, cand, gamma):
    """Commit the longest prefix of the candidates sorted by increasing entropy
    H_(0) <= H_(1) <= ... on which the exclusive prefix sum sum_{j<i} H_(j) <= gamma
    holds, and at least one candidate.

    Function table, entropy_bound_transfer row (the sum runs over j < i);
    mlxcel "Samplers and Reveal Policies": at least one position is accepted.
    """
    ent, cand = _f32(entropy, "entropy"), _mask(cand, "cand")
    gamma = _check_param(gamma, "gamma")
    B, L = ent.shape
    out = np.zeros((B, L), dtype=bool)
    for b in range(B):
        order = sorted((l for l in range(L) if cand[b, l]),
                       key=lambda l: (_ent(ent[b, l]), l))
        if not order:
            continue
        n = len(order)
        prefix = _ExactSum()                  # S_0 = 0
        for i, l in enumerate(order):
            if not prefix.at_most(gamma):
                n = i
                break
            prefix.add(_ent(ent[b, l]))
        out[b, order[:max(n, 1)]] = True
    return out


def edit_transfer(x0, prob, tokens, editable, tau_edit):
    """edit = editable & (x0 != tokens) & (prob > tau_edit): strict, no forcing.

    Function table, edit_transfer row; "Token editing (LLaDA2.1)": a committed
    position takes the new prediction when it differs and its confidence
    exceeds the editing threshold.
    """
    prob, editable = _f32(prob, "prob"), _mask(editable, "editable")
    tau_edit = _check_param(tau_edit, "tau_edit")
    x0, tokens = np.asarray(x0), np.asarray(tokens)
    B, L = prob.shape
    out = np.zeros((B, L), dtype=bool)
    for b in range(B):
        for l in range(L):
            out[b, l] = bool(editable[b, l]) and int(x0[b, l]) != int(tokens[b, l]) \
                and _conf(prob[b, l]) > tau_edit
    return out


def transfer_schedule(n_masked, steps):
    """(B, steps) per-step quotas: q[b, s] = n_b // steps + (1 if s < n_b % steps).

    mojo-dllm "The loop LLaDA uses": masked positions are spread over the steps
    evenly (32 masks over 8 steps: 4 per step); the function table's
    transfer_schedule row: linear quotas.  The remainder goes to the earliest
    steps.  A negative count is treated as 0.
    """
    steps = int(steps)
    if steps < 1:
        raise ValueError("steps must be >= 1")
    n = np.asarray(n_masked)
    B = n.shape[0]
    out = np.zeros((B, steps), dtype=np.int32)
    for b in range(B):
        nb = max(int(n[b]), 0)
        for s in range(steps):
            out[b, s] = nb // steps + (1 if s < nb % steps else 0)
    return out


def block_ranges(prompt_len, gen_len, block_len, align=False):
    """The [start, end) blocks that cover the generation region [P, P + G).

    align=False: blocks start at P, P + bl, ...  align=True: blocks are aligned
    on absolute positions, the first one starting at floor(P / bl) * bl (so it
    may begin inside the prompt).  The last block is cut at P + G; G = 0 gives
    no block.  Function table, block_ranges row (prompt-relative or
    absolute-aligned); the aligned loop of "Token editing (LLaDA2.1)".
    """
    P, G, bl = int(prompt_len), int(gen_len), int(block_len)
    if P < 0 or G < 0 or bl < 1:
        raise ValueError("need prompt_len >= 0, gen_len >= 0, block_len >= 1")
    if G == 0:
        return []
    start = (P // bl) * bl if align else P
    end_all = P + G
    out = []
    while start < end_all:
        out.append((start, min(start + bl, end_all)))
        start += bl
    return out


def block_causal_mask(L, block_len):
    """(L, L) float32 additive mask: 0 where key block <= query block, -inf elsewhere.

    Function table paragraph on mlx_arsenal.attention.block_causal_mask
    (bidirectional inside a block, causal across blocks, aligned on absolute
    positions) and "Mask conventions" (0 attend, -inf blocked).
    """
    L, bl = int(L), int(block_len)
    if L < 0 or bl < 1:
        raise ValueError("need L >= 0 and block_len >= 1")
    out = np.empty((L, L), dtype=np.float32)
    key_block = np.arange(L) // bl
    for q in range(L):
        out[q] = np.where(key_block <= q // bl, 0.0, -np.inf)
    return out
