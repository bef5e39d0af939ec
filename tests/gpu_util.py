"""Helpers of the GPU parity tests: device transfer and oracle comparisons.

Tolerances: prob and entropy within 1e-5 relative for float32 logits and 2e-3
for bf16 logits (absolute floor 1e-30); x0, masks, schedules bit-exact, except
sampled near-ties (oracle's best and second-best score within 1e-4 * max(1,
|best|)) and near-bound positions of end-to-end rule comparisons (within 1e-6
of the decision boundary), which are counted and reported, never silently
accepted.
"""
import sys

import numpy as np
import torch

import oracle

RTOL = {"f32": 1e-5, "bf16": 2e-3}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(arr, dtype=None):
    """numpy -> cuda tensor; uint16 bf16 bit patterns become torch.bfloat16."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def stats_np(st):
    """(x0, prob, entropy) as numpy arrays, plus margin when it was computed."""
    torch.cuda.synchronize()
    out = (st.x0.cpu().numpy(), st.prob.cpu().numpy(), st.entropy.cpu().numpy())
    if getattr(st, "margin", None) is not None:
        out = out + (st.margin.cpu().numpy(),)
    return out


def max_rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), 1e-30))) if a.size else 0.0


def assert_stats(gpu, ref, dtype, label, mask=None, x0_exact=True, fields=("prob", "entropy")):
    """Compare (x0, prob, entropy) with the oracle on the positions in mask."""
    gx, gp, ge = gpu[0], gpu[1], gpu[2]
    rx, rp, re = ref.x0, ref.prob, ref.entropy
    if mask is None:
        mask = np.ones(gx.shape, dtype=bool)
    tol = RTOL[dtype]
    if x0_exact:
        bad = np.flatnonzero((gx != rx) & mask)
        assert bad.size == 0, f"{label}: x0 differs at {bad[:10]}"
    pairs = [("prob", gp, rp), ("entropy", ge, re)]
    if "margin" in fields:
        pairs.append(("margin", gpu[3], ref.margin))
    for name, g, r in pairs:
        if name not in fields:
            continue
        g, r = g[mask], r[mask]
        assert np.all(np.isfinite(g)), f"{label}: non-finite {name}"
        err = np.abs(g.astype(np.float64) - r) <= tol * np.abs(r) + 1e-30
        assert err.all(), (f"{label}: {name} off by rel {max_rel(g, r):.3e} "
                           f"(tol {tol}) at {np.flatnonzero(~err)[:10]}")
    log(f"  {label}: prob max rel {max_rel(gp[mask], rp[mask]):.2e}, "
        f"entropy max rel {max_rel(ge[mask], re[mask]):.2e} ({int(mask.sum())} positions)")


def sampled_near_ties(logits_f64_row, T, seed, step, b, l, suppress):
    """Indices whose oracle score is within the near-tie band of the best."""
    V = logits_f64_row.shape[0]
    g = oracle.gumbel_noise(seed, step, b, l, V)
    lp = np.where(np.isnan(logits_f64_row), -np.inf, logits_f64_row)
    s = lp / float(np.float32(T)) + g
    s[list(suppress)] = -np.inf
    best = s.max()
    band = 1e-4 * max(1.0, abs(best))
    return set(np.flatnonzero(s >= best - band).tolist())


def assert_sampled_x0(gx, ref_x0, logits, dtype, T, seed, step, suppress, positions, label):
    """x0 bit-exact except near-tie rows, where the GPU pick must be one of the
    near-tied indices.  Returns the number of near-tie rows."""
    near = 0
    for b, l in positions:
        if gx[b, l] == ref_x0[b, l]:
            continue
        row = oracle.widen_logits(logits[b, l], dtype)
        tied = sampled_near_ties(row, T, seed, step, b, l, suppress)
        assert len(tied) > 1 and int(gx[b, l]) in tied, \
            f"{label}: sampled x0 differs at {(b, l)} and is not a near-tie"
        near += 1
    log(f"  {label}: sampled x0 near-tie rows {near} of {len(positions)}")
    return near


def near_bound_positions(kind, score, cand, param, k=None):
    """Positions whose commit decision could flip under a 1e-6 change of the
    scores (the end-to-end carve-out).  score: oracle float64/float32 (B, L)."""
    B, L = score.shape
    near = np.zeros((B, L), dtype=bool)
    eps = 1e-6
    for b in range(B):
        C = np.flatnonzero(cand[b])
        if C.size == 0:
            continue
        s = score[b].astype(np.float64)
        if kind == "threshold":
            near[b, C] |= np.abs(s[C] - param) <= eps
            near[b, C] |= np.abs(s[C] - s[C].max()) <= eps
            continue
        asc = kind == "entropy_bound"
        order = sorted(C, key=lambda p: (s[p] if asc else -s[p], p))
        ss = np.array([s[p] for p in order])
        if kind == "topk":
            n = min(max(int(k[b]), 0), len(order))
        elif kind == "factor":
            ok = (np.arange(len(ss)) + 1) * (1 - ss) <= param
            n = int(np.argmin(ok)) if not ok.all() else len(ss)
            vals = (np.arange(len(ss)) + 1) * (1 - ss)
            if any(abs(vals[i] - param) <= eps for i in (n - 1, n) if 0 <= i < len(ss)):
                for i in (n - 1, n):
                    if 0 <= i < len(ss):
                        near[b, order[i]] = True
        else:
            pre = np.concatenate([[0.0], np.cumsum(ss)[:-1]])
            ok = pre <= param
            n = int(np.argmin(ok)) if not ok.all() else len(ss)
            if any(abs(pre[i] - param) <= eps for i in (n - 1, n) if 0 <= i < len(ss)):
                for i in (n - 1, n):
                    if 0 <= i < len(ss):
                        near[b, order[i]] = True
        for i in (n - 1, n):
            if 0 <= i < len(ss):
                near[b, C] |= np.abs(s[C] - ss[i]) <= eps
    return near


def assert_e2e(kind, gpu_out, ref_out, near, label):
    diff = gpu_out != ref_out
    unexplained = diff & ~near
    assert not unexplained.any(), \
        f"{label}: commit differs away from any bound at {np.argwhere(unexplained)[:10].tolist()}"
    log(f"  {label}: end-to-end {kind}: {int(diff.sum())} near-bound differences, "
        f"{int(near.sum())} near-bound positions")
