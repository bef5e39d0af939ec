"""dllm_commit_step on the GPU against the oracle's loop step.

Statistics of the rows the rules look at are compared with the oracle's
(tolerances of gpu_util); the rows no rule looks at must be left exactly as
they were (their logits are NaN here, so a read would show).  The commit and
edit masks are compared bit-exactly with the oracle's rules run on the GPU's
own float32 statistics, and the canvas and counts with the oracle's update of
those masks.
"""
import numpy as np
import pytest
import torch

import commit_step_amd as dc
import oracle
import workloads
from gpu_util import assert_sampled_x0, assert_stats, log, stats_np, to_dev
from workloads import bf16_bits, random_logits

pytestmark = pytest.mark.gpu

SENT_X0, SENT_P, SENT_H = -7, -1.0, -2.0


def _canvas(rng, B, L, V, mask_id, P, frac_masked):
    """Prompt [0, P); after it, masked positions (a seeded fraction) and
    committed ones (editable)."""
    tokens = rng.integers(0, mask_id, size=(B, L)).astype(np.int32)
    masked = np.zeros((B, L), dtype=bool)
    masked[:, P:] = rng.random((B, L - P)) < frac_masked
    tokens[masked] = mask_id
    in_block = np.zeros((B, L), dtype=bool)
    in_block[:, P:] = True
    editable = in_block & ~masked
    return tokens, masked, editable


def _rank(kind, cand, param, strict=False):
    if kind == "threshold":
        return dc.Rule.threshold(cand, param, strict=strict)
    if kind == "topk":
        return dc.Rule.topk(cand, param)
    if kind == "factor":
        return dc.Rule.factor(cand, param)
    return dc.Rule.entropy_bound(cand, param)


def _run_and_check(arr, dtype, tokens, cand, editable, kind, param, strict=False, tau_edit=0.9,
                   T=0.0, seed=None, step=0, sup=(), skip_rows=True, pinned=False, label=""):
    B, L = tokens.shape
    dev_logits = to_dev(arr, dtype)
    tok = torch.from_numpy(tokens.copy()).cuda()
    cm = torch.from_numpy(cand).cuda()
    em = torch.from_numpy(editable).cuda() if editable is not None else None
    x0 = torch.full((B, L), SENT_X0, dtype=torch.int32, device="cuda")
    pr = torch.full((B, L), SENT_P, dtype=torch.float32, device="cuda")
    en = torch.full((B, L), SENT_H, dtype=torch.float32, device="cuda")
    rules = []
    if kind is not None:
        rules.append(_rank(kind, cm, param, strict))
    if em is not None:
        rules.append(dc.Rule.edit(em, None, tau_edit))
    counts = torch.empty((B, 2), dtype=torch.int32).pin_memory() if pinned else True
    log(f"commit_step {label}: {dtype} B={B} L={L} V={arr.shape[2]} rule={kind} T={T} "
        f"skip={skip_rows} pinned={pinned}")
    r = dc.commit_step(dev_logits, tok, rules, temperature=T, seed=seed, step=step,
                       suppress_ids=sup, skip_rows=skip_rows, counts=counts, out=(x0, pr, en))
    torch.cuda.synchronize()
    gx, gp, ge = stats_np(r.stats)
    need = np.zeros((B, L), dtype=bool)
    if kind is not None:
        need |= cand
    if editable is not None:
        need |= editable
    if skip_rows:
        assert (gx[~need] == SENT_X0).all() and (gp[~need] == SENT_P).all() \
            and (ge[~need] == SENT_H).all(), f"{label}: a row no rule looks at was written"
    ref = oracle.token_stats(arr, dtype, temperature=T, seed=seed, step=step, suppress_ids=sup)
    if T == 0.0:
        assert_stats((gx, gp, ge), ref, dtype, label, mask=need)
    else:
        assert_stats((gx, gp, ge), ref, dtype, label, mask=need & (gx == ref.x0), x0_exact=False)
        assert_stats((gx, gp, ge), ref, dtype, label + " entropy", mask=need, x0_exact=False,
                     fields=("entropy",))
        pos = [tuple(p) for p in np.argwhere(need)[:64]]
        assert_sampled_x0(gx, ref.x0, arr, dtype, T, seed, step, sup, pos, label + " sampled")
    commit = None
    if kind is not None:
        commit = oracle.rank_rule(kind, gp, ge, cand, param, strict)
        assert np.array_equal(rules[0].out.cpu().numpy(), commit), f"{label}: commit mask"
    edit = None
    if em is not None:
        edit = oracle.edit_transfer(gx, gp, tokens, editable, tau_edit)
        assert np.array_equal(rules[-1].out.cpu().numpy(), edit), f"{label}: edit mask"
    want = oracle.apply_step(tokens, gx, commit, edit)
    assert np.array_equal(tok.cpu().numpy(), want), f"{label}: canvas"
    want_counts = oracle.counts(cand if kind is not None else None,
                                commit, edit, B)
    got_counts = r.counts.numpy() if pinned else r.counts.cpu().numpy()
    assert np.array_equal(got_counts, want_counts), f"{label}: counts {got_counts} vs {want_counts}"
    return gx, gp, ge, tok.cpu().numpy()


@pytest.mark.parametrize("kind,param,strict,dtype,B,L,V,T", [
    ("threshold", 0.9, True, "bf16", 2, 64, 32768, 0.0),      # LLaDA2.1: threshold + edit
    ("entropy_bound", 0.5, False, "bf16", 1, 256, 20000, 0.0),
    ("factor", 1.0, False, "f32", 3, 40, 9000, 0.0),
    ("topk", 5, False, "bf16", 2, 100, 12000, 0.7),            # sampled x0
    ("threshold", 0.5, False, "bf16", 1, 600, 4096, 0.0),      # L > 512: sorted rule path
    ("topk", 37, False, "bf16", 1, 700, 5000, 0.0),            # long rows: sorted commits + canvas
    ("factor", 2.0, False, "f32", 2, 300, 3000, 0.0),
    ("entropy_bound", 1.5, False, "bf16", 1, 700, 5000, 0.0),
])
def test_commit_step_matches_oracle(kind, param, strict, dtype, B, L, V, T):
    rng = np.random.default_rng(31 + L)
    mask_id = V - 1
    tokens, masked, editable = _canvas(rng, B, L, V, mask_id, P=L // 8, frac_masked=0.6)
    bits, _ = random_logits(41 + L, B, L, V, dtype, 2.5, 0.5, 6.0, 14.0, (mask_id,))
    arr = bits.copy()
    nan = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
    arr[~(masked | editable)] = nan                       # rows no rule looks at
    _run_and_check(arr, dtype, tokens, masked, editable, kind, param, strict,
                   T=T, seed=99 if T > 0 else None, step=3, sup=(mask_id,),
                   label=f"{kind}")


def test_commit_step_without_skipping_and_pinned_counts():
    rng = np.random.default_rng(5)
    B, L, V = 2, 48, 16000
    mask_id = V - 1
    tokens, masked, editable = _canvas(rng, B, L, V, mask_id, P=6, frac_masked=0.5)
    bits, _ = random_logits(6, B, L, V, "bf16", 2.5, 0.5, 6.0, 14.0, (mask_id,))
    a = _run_and_check(bits, "bf16", tokens, masked, editable, "threshold", 0.8,
                       sup=(mask_id,), skip_rows=False, label="no skipping")
    b = _run_and_check(bits, "bf16", tokens, masked, editable, "threshold", 0.8,
                       sup=(mask_id,), skip_rows=True, pinned=True, label="skip, pinned counts")
    need = masked | editable
    assert np.array_equal(a[0][need], b[0][need]) and np.array_equal(a[1][need], b[1][need])
    assert np.array_equal(a[3], b[3])


def test_commit_step_edit_only_and_rank_only():
    rng = np.random.default_rng(9)
    B, L, V = 1, 80, 8192
    mask_id = V - 1
    tokens, masked, editable = _canvas(rng, B, L, V, mask_id, P=8, frac_masked=0.4)
    bits, _ = random_logits(10, B, L, V, "f32", 2.0, 0.6, 8.0, 14.0, (mask_id,))
    _run_and_check(bits, "f32", tokens, masked, editable, None, None, sup=(mask_id,),
                   tau_edit=0.5, label="edit only")
    _run_and_check(bits, "f32", tokens, masked, None, "topk", 3, sup=(mask_id,),
                   label="rank only")


def test_commit_step_diffusiongemma_canvas():
    """The 256 x 262144 bf16 canvas: entropy_bound + edit on its own
    candidates and committed positions."""
    w = workloads.config4()
    p = w.params
    _run_and_check(w.logits, "bf16", w.tokens, w.cand, w.editable, "entropy_bound",
                   p["gamma"], tau_edit=p["tau_edit"], label="diffusiongemma canvas")


def test_llada_block_loop_runs_on_the_device():
    """The LLaDA block of 32 masked positions decoded over 32 steps with the
    even quotas of transfer_schedule and topk, the canvas and the counts kept
    on the device; each step checked against the oracle's update of the
    GPU's own masks; the block ends fully committed."""
    p = workloads.CONFIG_PARAMS[2]
    B, L, V, steps, mask_id = p["B"], p["L"], p["V"], p["steps"], p["mask_id"]
    tokens = np.full((B, L), mask_id, dtype=np.int32)
    tok = torch.from_numpy(tokens.copy()).cuda()
    quotas = oracle.transfer_schedule(np.array([L], dtype=np.int32), steps)
    x0 = torch.empty((B, L), dtype=torch.int32, device="cuda")
    pr = torch.empty((B, L), dtype=torch.float32, device="cuda")
    en = torch.empty((B, L), dtype=torch.float32, device="cuda")
    for s in range(steps):
        w = workloads.config2_step(s)
        cand = tokens == mask_id
        cm = torch.from_numpy(cand).cuda()
        k = torch.from_numpy(np.ascontiguousarray(quotas[:, s]).astype(np.int32)).cuda()
        rule = dc.Rule.topk(cm, k)
        r = dc.commit_step(to_dev(w.logits, "bf16"), tok, [rule], suppress_ids=w.suppress_ids,
                           out=(x0, pr, en))
        gx, gp, ge = stats_np(r.stats)
        commit = oracle.rank_rule("topk", gp, ge, cand, quotas[:, s])
        assert np.array_equal(rule.out.cpu().numpy(), commit), f"step {s}: commit"
        tokens = oracle.apply_step(tokens, gx, commit, None)
        assert np.array_equal(tok.cpu().numpy(), tokens), f"step {s}: canvas"
        assert r.counts.cpu().numpy().tolist() == [[int((tokens == mask_id).sum()), 0]]
        if s in (0, steps // 2, steps - 1):
            ref = oracle.token_stats(w.logits, "bf16", suppress_ids=w.suppress_ids)
            assert_stats((gx, gp, ge), ref, "bf16", f"llada step {s}", mask=cand)
    assert not (tokens == mask_id).any()
    log("llada block loop: 32 steps, all committed")


@pytest.mark.parametrize("i", range(128))
def test_random_commit_steps(i):
    """Seeded random commit steps: dtype, shape (odd and split vocabularies,
    short and long batch rows), rank rule and its parameter, edit rule or none,
    row skipping or not, greedy or sampled; rows no rule looks at hold NaN when
    they are skipped."""
    rng = np.random.default_rng(7000 + i)
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    V = int(rng.choice([64, 1001, 4096, 5003, 9000, 20000, 40000]))
    B = int(rng.integers(1, 4))
    L = int(rng.choice([8, 32, 64, 100, 256, 300]))
    kind = str(rng.choice(["threshold", "topk", "factor", "entropy_bound", "none"]))
    with_edit = bool(rng.random() < 0.5) or kind == "none"
    skip_rows = bool(rng.random() < 0.6)
    T = 0.0 if rng.random() < 0.6 else float(np.float32(rng.uniform(0.5, 1.2)))
    mask_id = V - 1
    tokens, masked, editable = _canvas(rng, B, L, V, mask_id, P=L // 8,
                                       frac_masked=float(rng.uniform(0.2, 0.9)))
    bits, _ = random_logits(8000 + i, B, L, V, dtype, float(rng.uniform(1.0, 3.5)), 0.5, 4.0,
                            14.0, (mask_id,))
    arr = bits.copy()
    if skip_rows:
        nan = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
        arr[~(masked | (editable if with_edit else False))] = nan
    param = {"threshold": float(rng.choice([0.5, 0.9])), "topk": int(rng.integers(0, 9)),
             "factor": float(rng.choice([0.5, 1.0, 2.0])),
             "entropy_bound": float(rng.choice([0.2, 0.5, 1.5])), "none": None}[kind]
    strict = bool(rng.integers(2))
    _run_and_check(arr, dtype, tokens, masked, editable if with_edit else None,
                   None if kind == "none" else kind, param, strict if kind == "threshold" else False,
                   T=T, seed=int(rng.integers(0, 2 ** 40)) if T > 0 else None,
                   step=int(rng.integers(0, 50)), sup=(mask_id,), skip_rows=skip_rows,
                   label=f"random {i}")
