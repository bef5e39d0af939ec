"""The pages' decode loops driven by the oracle and a stub model (CPU only).

mlx-arsenal "dLLM block decoding" runs its reference loops verbatim in its test
suite ("Reference loop", "Token editing (LLaDA2.1)"); here the same loops run on
the oracle with a stub model that replays seeded logits, and their invariants
are checked: they terminate, every step makes progress, every masked position is
filled, and the LLaDA fixed-quota loop commits each position exactly once.
"""
import numpy as np

import oracle

V = 64
MASK = V - 1


class StubModel:
    """Returns seeded (B, L, V) float32 logits; a fresh draw on every call."""

    def __init__(self, seed):
        self.rng = np.random.default_rng(seed)
        self.calls = 0

    def __call__(self, x):
        self.calls += 1
        B, L = x.shape
        z = self.rng.standard_normal((B, L, V)).astype(np.float32) * 2
        hot = self.rng.integers(0, V - 1, size=(B, L))
        z[np.arange(B)[:, None], np.arange(L)[None, :], hot] += 6.0
        return z


def decode(model, prompt, gen_len, block_len, threshold=0.9):
    B, P = prompt.shape
    x = np.concatenate([prompt, np.full((B, gen_len), MASK, dtype=np.int32)], axis=1)
    pos = np.arange(P + gen_len)
    forwards = 0
    for start, end in oracle.block_ranges(P, gen_len, block_len):
        in_block = (pos >= start) & (pos < end)
        while True:
            cand = (x == MASK) & in_block[None, :]
            if not cand.any():
                break
            st = oracle.token_stats(model(x), "f32", suppress_ids=[MASK])
            forwards += 1
            commit = oracle.threshold_transfer(st.prob.astype(np.float32), cand, threshold)
            assert commit[cand.any(axis=1)].any(axis=1).all()      # progress in every row
            assert not np.any(commit & ~cand)
            x = np.where(commit, st.x0, x)
    return x, forwards


def test_threshold_block_decoder_fills_every_position():
    prompt = np.random.default_rng(0).integers(0, MASK, size=(2, 5)).astype(np.int32)
    x, forwards = decode(StubModel(1), prompt, gen_len=20, block_len=8)
    assert not np.any(x == MASK)
    assert np.array_equal(x[:, :5], prompt)
    assert 3 <= forwards <= 20


def test_llada_fixed_quota_commits_each_position_once():
    steps, L = 8, 32
    model = StubModel(2)
    x = np.full((1, L), MASK, dtype=np.int32)
    cand = x == MASK
    sched = oracle.transfer_schedule(cand.sum(axis=1), steps)
    times = np.zeros(L, dtype=int)
    for s in range(steps):
        st = oracle.token_stats(model(x), "f32", suppress_ids=[MASK])
        commit = oracle.topk_transfer(st.prob.astype(np.float32), cand, sched[:, s])
        assert commit.sum() == sched[0, s]
        times += commit[0]
        x = np.where(commit, st.x0, x)
        cand = x == MASK
    assert np.all(times == 1) and not np.any(x == MASK)


def test_editing_loop_terminates():
    B, P, gen_len, bl, max_post = 1, 3, 13, 8, 4
    model = StubModel(3)
    prompt = np.array([[5, 6, 7]], dtype=np.int32)
    total = -(-(P + gen_len) // bl) * bl
    x = np.concatenate([prompt, np.full((B, total - P), MASK, dtype=np.int32)], axis=1)
    pos = np.arange(total)
    forwards = 0
    for start, end in oracle.block_ranges(P, total - P, bl, align=True):
        in_block = ((pos >= start) & (pos < end) & (pos >= P))[:end]
        post = 0
        while True:
            window = x[:, :end]
            masked = (window == MASK) & in_block
            has_mask = masked.any()
            if not has_mask:
                post += 1
                if post > max_post:
                    break
            st = oracle.token_stats(model(window), "f32")
            forwards += 1
            commit = oracle.threshold_transfer(st.prob.astype(np.float32), masked, 0.95, strict=True)
            editable = in_block & ~masked
            edit = oracle.edit_transfer(st.x0, st.prob.astype(np.float32), window, editable, 0.9)
            assert not np.any(commit & edit)
            window = np.where(commit | edit, st.x0, window)
            x = np.concatenate([window, x[:, end:]], axis=1)
            if not has_mask and not edit.any():
                break
    assert not np.any(x[:, P:P + gen_len] == MASK)
    assert np.array_equal(x[:, :P], prompt)
    assert forwards <= 2 * (gen_len + 2 * (max_post + 1))
