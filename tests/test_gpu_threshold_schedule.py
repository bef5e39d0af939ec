"""Threshold schedules on the GPU (mlxcel "Block Diffusion", "LLaDA-2 Block
Unmasking": an initial and a floor confidence threshold, 0.95 by default, and
a linearly decaying threshold).

One threshold per batch row, standalone and fused into dllm_commit_step,
compared bit for bit with the oracle's threshold rule on the same float32
confidences; and a LLaDA-2 block of 32 positions decoded with a decaying
threshold, each row at its own step of the schedule.
"""
import math

import numpy as np
import pytest
import torch

import commit_step_amd as dc
import oracle
from gpu_util import assert_stats, log, stats_np, to_dev
from workloads import random_logits

pytestmark = pytest.mark.gpu

TAU_CHOICES = [0.0, 0.3, 0.5, 0.9, 0.95, 1.0, 1.5, -math.inf, math.inf]


@pytest.mark.parametrize("B,L", [(1, 1), (3, 7), (5, 64), (4, 256), (2, 513), (3, 1000),
                                 (1, 4096), (300, 32)])
def test_per_row_threshold_standalone(B, L):
    rng = np.random.default_rng(B * 7919 + L)
    for trial in range(6):
        if trial % 2:
            conf = rng.choice(np.float32([0.0, 0.1, 0.5, 0.9, 0.95, 1.0]), size=(B, L))
        else:
            conf = rng.uniform(0, 1, size=(B, L)).astype(np.float32)
        if trial == 5 and L >= 4:
            conf.reshape(-1)[:3] = [np.nan, np.inf, -np.inf]
        cand = rng.random((B, L)) < rng.uniform(0.05, 1.0)
        taus = rng.choice(TAU_CHOICES, size=B)
        strict = bool(trial % 3 == 1)
        got = dc.threshold_transfer(to_dev(conf), to_dev(cand),
                                    torch.from_numpy(taus).cuda(), strict).cpu().numpy()
        want = oracle.threshold_transfer(conf, cand, taus, strict)
        assert np.array_equal(got, want), f"B={B} L={L} trial={trial}"
        # one scalar threshold broadcast to every row is the scalar call
        same = torch.full((B,), float(taus[0]), dtype=torch.float64, device="cuda")
        a = dc.threshold_transfer(to_dev(conf), to_dev(cand), same, strict)
        b = dc.threshold_transfer(to_dev(conf), to_dev(cand), float(taus[0]), strict)
        assert torch.equal(a, b)
    log(f"per-row threshold B={B} L={L}: bit-exact")


@pytest.mark.parametrize("B,L,V,strict,score", [(4, 32, 32768, False, "prob"),
                                                (3, 600, 4096, True, "prob"),
                                                (2, 48, 16000, False, "neg_entropy")])
def test_per_row_threshold_fused(B, L, V, strict, score):
    rng = np.random.default_rng(L + V)
    bits, _ = random_logits(17 + L, B, L, V, "bf16", 2.5, 0.5, 6.0, 14.0)
    cand = rng.random((B, L)) < 0.7
    tokens = np.full((B, L), V - 1, dtype=np.int32)
    taus = np.array([0.95, 0.5, 0.2, -0.5][:B]) if score == "prob" else \
        np.array([-0.5, -2.0, -9.0][:B])
    tok = torch.from_numpy(tokens.copy()).cuda()
    rule = dc.Rule.threshold(to_dev(cand), torch.from_numpy(taus).cuda(), strict=strict,
                             score=score)
    r = dc.commit_step(to_dev(bits, "bf16"), tok, [rule])
    gx, gp, ge = stats_np(r.stats)
    conf = gp if score == "prob" else (-ge).astype(np.float32)
    want = oracle.threshold_transfer(conf, cand, taus, strict)
    assert np.array_equal(rule.out.cpu().numpy(), want)
    assert np.array_equal(tok.cpu().numpy(), oracle.apply_step(tokens, gx, want, None))
    ref = oracle.token_stats(bits, "bf16")
    assert_stats((gx, gp, ge), ref, "bf16", "fused per-row threshold", mask=cand)
    # token_stats with the same fused rule
    rule2 = dc.Rule.threshold(to_dev(cand), torch.from_numpy(taus).cuda(), strict=strict,
                              score=score)
    dc.token_stats(to_dev(bits, "bf16"), rules=[rule2])
    assert torch.equal(rule2.out, rule.out)
    log(f"fused per-row threshold B={B} L={L} V={V} score={score}")


def test_llada2_block_with_a_decaying_threshold():
    """A block of 32 masked positions per row; row b starts b steps into the
    schedule max(floor, 0.95 - decay * step), so the rows of one call use
    different thresholds.  Each step is checked against the oracle's rule on
    the GPU's statistics and the oracle's canvas update; every row ends fully
    committed within 32 steps (one candidate is forced per step)."""
    B, L, V, mask_id = 4, 32, 32768, 32767
    tau0, floor, decay = 0.95, 0.6, 0.02
    tokens = np.full((B, L), mask_id, dtype=np.int32)
    tok = torch.from_numpy(tokens.copy()).cuda()
    for s in range(32):
        cand = tokens == mask_id
        if not cand.any():
            break
        taus = np.array([oracle.decaying_threshold(tau0, floor, decay, s + b) for b in range(B)])
        lib_taus = np.array([dc.decaying_threshold(tau0, floor, decay, s + b) for b in range(B)])
        assert np.array_equal(taus, lib_taus)
        bits, _ = random_logits(1000 + s, B, L, V, "bf16", 3.0, 0.5, 6.0, 14.0, (mask_id,))
        rule = dc.Rule.threshold(to_dev(cand), torch.from_numpy(taus).cuda())
        r = dc.commit_step(to_dev(bits, "bf16"), tok, [rule], suppress_ids=(mask_id,))
        gx, gp, ge = stats_np(r.stats)
        commit = oracle.threshold_transfer(gp, cand, taus)
        assert np.array_equal(rule.out.cpu().numpy(), commit), f"step {s}: commit"
        tokens = oracle.apply_step(tokens, gx, commit, None)
        assert np.array_equal(tok.cpu().numpy(), tokens), f"step {s}: canvas"
        assert r.counts.cpu().numpy()[:, 0].tolist() == (tokens == mask_id).sum(1).tolist()
        if s in (0, 5):
            ref = oracle.token_stats(bits, "bf16", suppress_ids=(mask_id,))
            assert_stats((gx, gp, ge), ref, "bf16", f"llada2 step {s}", mask=cand)
    assert not (tokens == mask_id).any()
    log(f"llada2 decaying threshold: block committed after {s + 1} steps")
