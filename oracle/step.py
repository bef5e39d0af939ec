"""Oracle: one step of the decoding loop on a token canvas (test infrastructure).

Source: mlx-arsenal research note "dLLM block decoding".
  * "The pattern": per step the candidates are the masked positions of the
    current block; statistics, one commit rule over the candidates, then the
    canvas takes x0 where committed; the block ends when no candidate is left.
  * "Token editing (LLaDA2.1)": after the mask commit, a committed position of
    the block that is not masked (editable) takes the new prediction when it
    differs and its confidence exceeds the editing threshold; the canvas takes
    x0 where committed or edited; the loop stops once a step starts with no mask
    and edits nothing.
mojo-dllm ("Why the runtime looks different"): only candidate rows need logits.
That saving changes which rows are read, never a result, so it has no oracle
counterpart: here every row's statistics are computed.

What a step returns, per batch row b:
  * tokens' = where(commit | edit, x0, tokens);
  * left[b]   = candidates of the ranking rule that it did not commit;
  * edited[b] = positions the edit rule edited.
"""
from collections import namedtuple

import numpy as np

from .stats import token_stats
from .rules import (threshold_transfer, topk_transfer, factor_transfer,
                    entropy_bound_transfer, edit_transfer)

StepResult = namedtuple("StepResult", ["stats", "commit", "edit", "tokens", "counts"])


def rank_rule(kind, stats_prob, stats_entropy, cand, param, strict=False):
    """The commit mask of one ranking rule on float32 statistics.  kind is
    "threshold" (param = tau), "topk" (param = k, one quota or (B,) quotas),
    "factor" (param = f) or "entropy_bound" (param = gamma)."""
    if kind == "threshold":
        return threshold_transfer(stats_prob, cand, param, strict=strict)
    if kind == "topk":
        k = np.broadcast_to(np.asarray(param, dtype=np.int64), (stats_prob.shape[0],))
        return topk_transfer(stats_prob, cand, k)
    if kind == "factor":
        return factor_transfer(stats_prob, cand, param)
    if kind == "entropy_bound":
        return entropy_bound_transfer(stats_entropy, cand, param)
    raise ValueError(f"unknown ranking rule {kind!r}")


def apply_step(tokens, x0, commit, edit):
    """Canvas update of one step from its masks ("The pattern":
    x <- where(commit, x0, x); "Token editing": where(commit | edit, ...)).
    commit and edit are (B, L) bool, either may be None."""
    tokens = np.asarray(tokens)
    if tokens.dtype != np.int32:
        raise TypeError("tokens must be int32")
    out = tokens.copy()
    B, L = tokens.shape
    for b in range(B):
        for l in range(L):
            take = (commit is not None and commit[b, l]) or (edit is not None and edit[b, l])
            if take:
                out[b, l] = x0[b, l]
    return out


def counts(cand, commit, edit, B):
    """(B, 2) int32: candidates not committed, positions edited, per batch row."""
    c = np.zeros((B, 2), dtype=np.int32)
    for b in range(B):
        if cand is not None:
            c[b, 0] = sum(1 for l in range(cand.shape[1]) if cand[b, l] and not commit[b, l])
        if edit is not None:
            c[b, 1] = sum(1 for l in range(edit.shape[1]) if edit[b, l])
    return c


def commit_step(logits, dtype, tokens, rank=None, edit=None, temperature=0.0, seed=None,
                step=0, suppress_ids=()):
    """One loop step.  rank = (kind, cand, param[, strict]) or None;
    edit = (editable, tau_edit) or None.  The rules run on the float32
    statistics, as in the loop."""
    tokens = np.asarray(tokens)
    B, L = tokens.shape
    st = token_stats(logits, dtype, temperature=temperature, seed=seed, step=step,
                     suppress_ids=suppress_ids)
    prob32 = st.prob.astype(np.float32)
    ent32 = st.entropy.astype(np.float32)
    commit = None
    cand = None
    if rank is not None:
        kind, cand, param = rank[0], rank[1], rank[2]
        strict = rank[3] if len(rank) > 3 else False
        commit = rank_rule(kind, prob32, ent32, cand, param, strict)
    em = None
    if edit is not None:
        editable, tau_edit = edit
        em = edit_transfer(st.x0, prob32, tokens, editable, tau_edit)
    new_tokens = apply_step(tokens, st.x0, commit, em)
    return StepResult(st, commit, em, new_tokens, counts(cand, commit, em, B))
