"""The five synthetic workloads at full size, GPU against the oracle.

Each runs the same fused launch the benchmark times.  Statistics are compared
within tolerance at every position (for the Dream-like workload at its first
sampling step; its later steps at sampled positions); commit masks are
compared bit for bit against the oracle rules on the GPU's own statistics
(rule isolation) and end to end against the oracle rules on the oracle's
statistics, with near-bound positions reported.  The full-size oracle runs
in worker processes (oracle_pool).
"""
import types

import numpy as np
import pytest
import torch

import commit_step_amd as dc
import oracle
import oracle_pool
import workloads
from gpu_util import (RTOL, assert_e2e, assert_sampled_x0, assert_stats, log,
                      near_bound_positions, stats_np, to_dev)

pytestmark = pytest.mark.gpu


def test_config1_tiny_threshold():
    w = workloads.config1()
    log(f"{w.name}: {w.shape}")
    cand_t = to_dev(w.cand)
    rule = dc.Rule.threshold(cand_t, w.params["tau"], w.params["strict"])
    gpu = stats_np(dc.token_stats(to_dev(w.logits), suppress_ids=w.suppress_ids, rules=[rule]))
    ref = oracle.token_stats(w.logits, "f32", suppress_ids=w.suppress_ids)
    assert_stats(gpu, ref, "f32", w.name)
    out = rule.out.cpu().numpy()
    assert np.array_equal(out, oracle.threshold_transfer(gpu[1], w.cand, w.params["tau"]))
    ref_out = oracle.threshold_transfer(ref.prob.astype(np.float32), w.cand, w.params["tau"])
    near = near_bound_positions("threshold", ref.prob, w.cand, w.params["tau"])
    assert_e2e("threshold", out, ref_out, near, w.name)
    assert out.sum() >= 1


def test_config2_llada_block_loop():
    """32 teacher-forced steps: schedule, then fused stats + topk per step."""
    steps = workloads.CONFIG_PARAMS[2]["steps"]
    L = workloads.CONFIG_PARAMS[2]["L"]
    cand = np.ones((1, L), dtype=bool)
    sched_ref = oracle.transfer_schedule(cand.sum(axis=1), steps)
    sched = dc.transfer_schedule(to_dev(cand.sum(axis=1).astype(np.int32)), steps)
    assert np.array_equal(sched.cpu().numpy(), sched_ref)
    committed = np.zeros(L, dtype=int)
    near_total = 0
    for s in range(steps):
        w = workloads.config2_step(s)
        rule = dc.Rule.topk(to_dev(cand), sched[:, s].contiguous())
        gpu = stats_np(dc.token_stats(to_dev(w.logits, "bf16"), suppress_ids=w.suppress_ids,
                                      rules=[rule]))
        ref = oracle.token_stats(w.logits, "bf16", suppress_ids=w.suppress_ids)
        assert_stats(gpu, ref, "bf16", f"{w.name}")
        out = rule.out.cpu().numpy()
        assert np.array_equal(out, oracle.topk_transfer(gpu[1], cand, sched_ref[:, s]))
        ref_out = oracle.topk_transfer(ref.prob.astype(np.float32), cand, sched_ref[:, s])
        near = near_bound_positions("topk", ref.prob, cand, None, k=sched_ref[:, s])
        assert_e2e("topk", out, ref_out, near, w.name)
        near_total += int((out != ref_out).sum())
        committed += ref_out[0]
        cand = cand & ~ref_out                     # teacher-forced from the oracle
    assert np.all(committed == 1)
    log(f"config2: every position committed once; {near_total} near-bound differences")


def _prob_of(logits_row, dtype, x, suppress):
    """softmax(row)[x] in float64 over the unsuppressed tokens (NaN as -inf):
    the probability the statistics report for a proposal x."""
    row = oracle.widen_logits(logits_row, dtype)
    row = np.where(np.isnan(row), -np.inf, row)
    row[list(suppress)] = -np.inf
    m = row.max()
    e = np.exp(row - m)
    return float(e[x] / e.sum())


@pytest.mark.timeout(600)
def test_config3_dream_sampled_factor():
    """Step 0 at every position: x0 (near-tie rule), prob and entropy against
    the oracle, and the factor mask end to end against the oracle's rule on the
    oracle's statistics.  Steps 1-3 at sampled positions."""
    w = workloads.config3()
    T, seed, f = w.temperature, w.seed, w.params["f"]
    B, L, V = w.shape
    logits = to_dev(w.logits, "bf16")
    cand_t = to_dev(w.cand)
    rng = np.random.default_rng(33)
    prev = None
    log(f"{w.name}: oracle statistics of step 0 at all {B * L} positions "
        f"({oracle_pool.workers()} worker processes)")
    with oracle_pool.pool() as ex:
        rx, rp, re = oracle_pool.config3_stats(ex, w, 0)
    for step in range(w.params["steps"]):
        rule = dc.Rule.factor(cand_t, f)
        log(f"{w.name}: step {step}")
        gpu = stats_np(dc.token_stats(logits, temperature=T, seed=seed, step=step,
                                      suppress_ids=w.suppress_ids, rules=[rule]))
        out = rule.out.cpu().numpy()
        assert np.array_equal(out, oracle.factor_transfer(gpu[1], w.cand, f))
        assert (out & w.cand).sum(axis=1).min() >= 1
        if step == 0:
            every = [(b, l) for b in range(B) for l in range(L)]
            ties = assert_sampled_x0(gpu[0], rx, w.logits, "bf16", T, seed, 0, w.suppress_ids,
                                     every, f"{w.name} step 0")
            same = gpu[0] == rx
            ref = types.SimpleNamespace(x0=rx, prob=rp, entropy=re)
            assert_stats(gpu, ref, "bf16", f"{w.name} step 0, equal x0", mask=same)
            assert_stats(gpu, ref, "bf16", f"{w.name} step 0, entropy", x0_exact=False,
                         fields=("entropy",))
            # at a near-tie the statistics report the probability of the GPU's pick
            adj = rp.copy()
            for b, l in np.argwhere(~same):
                adj[b, l] = _prob_of(w.logits[b, l], "bf16", int(gpu[0][b, l]), w.suppress_ids)
            ok = np.abs(gpu[1].astype(np.float64) - adj) <= RTOL["bf16"] * adj
            assert ok.all(), f"prob of the near-tie picks off at {np.argwhere(~ok)[:5].tolist()}"
            ref_out = oracle.factor_transfer(adj.astype(np.float32), w.cand, f)
            near = near_bound_positions("factor", adj, w.cand, f)
            assert_e2e("factor", out, ref_out, near, f"{w.name} step 0")
            log(f"  {w.name} step 0: {ties} near-tie picks; committed {int(out.sum())} of "
                f"{int(w.cand.sum())} candidates")
        else:
            pos = [(int(b), int(l)) for b, l in zip(rng.integers(0, B, 12), rng.integers(0, L, 12))]
            ref = oracle.token_stats(w.logits, "bf16", temperature=T, seed=seed, step=step,
                                     suppress_ids=w.suppress_ids, positions=pos)
            mask = np.zeros((B, L), bool)
            for q in pos:
                mask[q] = True
            assert_sampled_x0(gpu[0], ref.x0, w.logits, "bf16", T, seed, step, w.suppress_ids,
                              pos, f"{w.name} step {step}")
            assert_stats(gpu, ref, "bf16", f"{w.name} step {step}",
                         mask=mask & (gpu[0] == ref.x0))
        if prev is not None:
            assert (gpu[0] != prev).mean() > 0.05          # a fresh key per step
        prev = gpu[0]


def test_config4_diffusiongemma_fused_entropy_bound_and_edit():
    w = workloads.config4()
    log(f"{w.name}: {w.shape}")
    eb = dc.Rule.entropy_bound(to_dev(w.cand), w.params["gamma"])
    ed = dc.Rule.edit(to_dev(w.editable), to_dev(w.tokens), w.params["tau_edit"])
    gpu = stats_np(dc.token_stats(to_dev(w.logits, "bf16"), rules=[eb, ed]))
    ref = oracle.token_stats(w.logits, "bf16")
    assert_stats(gpu, ref, "bf16", w.name)
    eb_out, ed_out = eb.out.cpu().numpy(), ed.out.cpu().numpy()
    assert np.array_equal(eb_out, oracle.entropy_bound_transfer(gpu[2], w.cand, w.params["gamma"]))
    assert np.array_equal(ed_out, oracle.edit_transfer(gpu[0], gpu[1], w.tokens, w.editable,
                                                       w.params["tau_edit"]))
    ref_eb = oracle.entropy_bound_transfer(ref.entropy.astype(np.float32), w.cand, w.params["gamma"])
    ref_ed = oracle.edit_transfer(ref.x0, ref.prob.astype(np.float32), w.tokens, w.editable,
                                  w.params["tau_edit"])
    assert_e2e("entropy_bound", eb_out, ref_eb,
               near_bound_positions("entropy_bound", ref.entropy, w.cand, w.params["gamma"]),
               w.name)
    near_ed = np.abs(ref.prob - w.params["tau_edit"]) <= 1e-6
    assert_e2e("edit", ed_out, ref_ed, near_ed, w.name)
    log(f"config4: committed {int(eb_out.sum())} of {int(w.cand.sum())} candidates, "
        f"edited {int(ed_out.sum())} of {int(w.editable.sum())}")


@pytest.mark.timeout(600)
def test_config5_batched_threshold_and_masks():
    p = workloads.CONFIG_PARAMS[5]
    B, L, V = p["B"], p["L"], p["V"]
    log(f"config5: generating {B}x{L}x{V} bf16")
    host = np.empty((B, L, V), dtype=np.uint16)
    for b in range(B):
        host[b] = workloads.config5_batch_row(b).logits[0]
    logits = to_dev(host, "bf16")
    cand = np.ones((B, L), bool)
    rule = dc.Rule.threshold(to_dev(cand), p["tau"], p["strict"])
    log("config5: fused launch")
    gpu = stats_np(dc.token_stats(logits, rules=[rule]))
    out = rule.out.cpu().numpy()
    # rule isolation over every batch row
    assert np.array_equal(out, oracle.threshold_transfer(gpu[1], cand, p["tau"], p["strict"]))
    # statistics and end-to-end commits at every position of every batch row
    # (the oracle takes one batch row per task)
    log(f"config5: oracle statistics of all {B} batch rows ({oracle_pool.workers()} worker processes)")
    with oracle_pool.pool() as ex:
        rx, rp, re = oracle_pool.config5_stats(ex)
    ref = types.SimpleNamespace(x0=rx, prob=rp, entropy=re)
    assert_stats(gpu, ref, "bf16", "config5")
    ref_out = oracle.threshold_transfer(rp.astype(np.float32), cand, p["tau"], p["strict"])
    near = near_bound_positions("threshold", rp, cand, p["tau"])
    assert_e2e("threshold", out, ref_out, near, f"config5, all {B} batch rows")
    assert np.all(out.sum(axis=1) >= 1)
    # block helpers of the workload
    assert dc.block_ranges(p["prompt_len"], p["gen_len"], p["block_len"], True) == \
        oracle.block_ranges(p["prompt_len"], p["gen_len"], p["block_len"], True)
    m = dc.block_causal_mask(p["mask_L"], p["block_len"]).cpu().numpy()
    assert np.array_equal(m.view(np.uint32),
                          oracle.block_causal_mask(p["mask_L"], p["block_len"]).view(np.uint32))
    del logits
    torch.cuda.empty_cache()
