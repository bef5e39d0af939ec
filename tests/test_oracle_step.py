"""Pins of the oracle's loop step (oracle/step.py) -- CPU only.

* A step worked by hand (tests/golden/commit_step_example.txt).
* The block loop of mlx-arsenal "dLLM block decoding" ("The pattern") driven by
  a seeded stand-in for the model: every step changes only committed positions,
  to x0; the "left" count equals the masks recounted from the new canvas; the
  loop ends with no mask, one forced token at least per step.
* The LLaDA2.1 editing loop ("Token editing (LLaDA2.1)"): edits land only on
  editable positions, and the loop stops on its own rule.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "commit_step_example.txt")

LOGITS = np.array([[[0, 0, 0, 0, 0], [0, 0, 5, 0, 9], [1, 0, 0, 0, 9],
                    [0, 0, 0, 6, 0], [0, 0, 4, 0, 0]]], dtype=np.float32)
TOKENS = np.array([[1, 4, 4, 1, 2]], dtype=np.int32)
CAND = np.array([[0, 1, 1, 0, 0]], dtype=bool)
EDITABLE = np.array([[0, 0, 0, 1, 1]], dtype=bool)
MASK_ID = 4


def _cases():
    rows = []
    with open(GOLDEN) as fh:
        for ln in fh:
            if ln.startswith("#") or not ln.strip():
                continue
            head, commit, edit, tokens, cnt = ln.split("|")
            rule, param, strict, tau_edit = head.split()
            rows.append((rule, float(param), bool(int(strict)), float(tau_edit),
                         [int(v) for v in commit.split()], [int(v) for v in edit.split()],
                         [int(v) for v in tokens.split()], [int(v) for v in cnt.split()]))
    return rows


@pytest.mark.parametrize("case", _cases())
def test_hand_worked_step(case):
    rule, param, strict, tau_edit, commit, edit, tokens, cnt = case
    param = int(param) if rule == "topk" else param
    r = oracle.commit_step(LOGITS, "f32", TOKENS, rank=(rule, CAND, param, strict),
                           edit=(EDITABLE, tau_edit), suppress_ids=[MASK_ID])
    assert r.commit.astype(int).tolist() == [commit]
    assert r.edit.astype(int).tolist() == [edit]
    assert r.tokens.tolist() == [tokens]
    assert r.counts.tolist() == [cnt]
    # the hand values of the statistics
    assert r.stats.prob[0, 1] == pytest.approx(0.98019, abs=1e-5)
    assert r.stats.prob[0, 2] == pytest.approx(0.47537, abs=1e-5)
    assert r.stats.prob[0, 3] == pytest.approx(0.99262, abs=1e-5)
    assert r.stats.entropy[0, 1] == pytest.approx(0.11908, abs=1e-5)
    assert r.stats.entropy[0, 2] == pytest.approx(1.26830, abs=1e-5)
    assert r.tokens.dtype == np.int32 and TOKENS.tolist() == [[1, 4, 4, 1, 2]]   # input untouched


def _stand_in_model(rng, B, L, V):
    x = rng.standard_normal((B, L, V)).astype(np.float32) * 2.0
    peak = rng.random((B, L)) < 0.4
    idx = rng.integers(0, V - 1, size=(B, L))
    for b in range(B):
        for l in range(L):
            if peak[b, l]:
                x[b, l, idx[b, l]] += 8.0
    return x


@pytest.mark.parametrize("rule,param", [("threshold", 0.9), ("entropy_bound", 0.5),
                                        ("factor", 1.0), ("topk", 2)])
def test_block_loop_counts_track_the_canvas(rule, param):
    rng = np.random.default_rng(7)
    B, P, G, bl, V = 2, 5, 19, 8, 40
    mask_id = V - 1
    L = P + G
    tokens = np.full((B, L), mask_id, dtype=np.int32)
    tokens[:, :P] = rng.integers(0, V - 1, size=(B, P))
    positions = np.arange(L)
    steps = 0
    for start, end in oracle.block_ranges(P, G, bl):
        in_block = (positions >= start) & (positions < end)
        for _ in range(bl + 1):
            cand = (tokens == mask_id) & in_block[None, :]
            if not cand.any():
                break
            r = oracle.commit_step(_stand_in_model(rng, B, L, V), "f32", tokens,
                                   rank=(rule, cand, param), suppress_ids=[mask_id])
            steps += 1
            changed = r.tokens != tokens
            assert not (changed & ~r.commit).any()
            assert np.array_equal(r.tokens[r.commit], r.stats.x0[r.commit])
            assert not (r.commit & ~cand).any()
            left = ((r.tokens == mask_id) & in_block[None, :]).sum(axis=1)
            assert np.array_equal(r.counts[:, 0], left)
            assert (r.counts[:, 1] == 0).all()
            # at least one commit per batch row that had candidates
            assert ((r.commit.sum(axis=1) >= 1) | (cand.sum(axis=1) == 0)).all()
            tokens = r.tokens
        else:
            pytest.fail("the block loop did not terminate")
    assert not (tokens == mask_id).any()
    assert steps >= 1


def test_editing_loop_edits_only_editable_and_stops():
    rng = np.random.default_rng(8)
    B, P, G, bl, V = 1, 4, 12, 8, 30
    mask_id = V - 1
    total = -(-(P + G) // bl) * bl
    tokens = np.full((B, total), mask_id, dtype=np.int32)
    tokens[:, :P] = rng.integers(0, V - 1, size=(B, P))
    positions = np.arange(total)
    for start, end in oracle.block_ranges(P, total - P, bl, align=True):
        in_block = (positions >= start) & (positions < end) & (positions >= P)
        post = 0
        for _ in range(bl + 40):
            masked = (tokens == mask_id) & in_block[None, :]
            has_mask = bool(masked.any())
            if not has_mask:
                post += 1
                if post > 16:
                    break
            editable = in_block[None, :] & ~masked
            r = oracle.commit_step(_stand_in_model(rng, B, total, V), "f32", tokens,
                                   rank=("threshold", masked, 0.95, True),
                                   edit=(editable, 0.9), suppress_ids=[mask_id])
            assert not (r.edit & ~editable).any()
            assert not (r.edit & r.commit).any()
            changed = r.tokens != tokens
            assert not (changed & ~(r.commit | r.edit)).any()
            assert r.counts[0, 1] == int(r.edit.sum())
            assert r.counts[0, 0] == int(((r.tokens == mask_id) & in_block[None, :]).sum())
            tokens = r.tokens
            if not has_mask and r.counts[0, 1] == 0:
                break
        else:
            pytest.fail("the editing loop did not stop")
    assert not (tokens == mask_id).any()
