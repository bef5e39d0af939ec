"""GPU parity of dllm_token_stats against the oracle (through the C-ABI binding).

Shapes span several workgroup iterations, ragged tails, the scalar-load path
(V not a multiple of 8), split rows (few rows, large V) and the largest
vocabulary of the workloads.
"""
import numpy as np
import pytest
import torch

import commit_step_amd as dc
import oracle
from gpu_util import (assert_sampled_x0, assert_stats, log, stats_np, to_dev)
from workloads import bf16_bits, random_logits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,B,L,V,sup", [
    ("f32", 2, 3, 1, ()),
    ("f32", 1, 5, 7, (3,)),
    ("bf16", 2, 4, 100, (99,)),
    ("f32", 1, 64, 4096, (4095,)),
    ("bf16", 3, 5, 5003, (0, 5002)),              # V % 8 != 0: scalar loads
    ("bf16", 1, 3, 65536 + 24, (65559,)),          # ragged last iteration
    ("f32", 2, 2, 131072 + 4, ()),                 # split rows, fp32
    ("bf16", 1, 2, 262144, ()),                    # split rows, largest V
    ("bf16", 4, 70, 32768, (7, 32767)),            # many rows, 256-thread groups
    ("f32", 1, 300, 20000, ()),                    # 512-thread groups, one row each
])
def test_greedy_parity(dtype, B, L, V, sup):
    bits, _ = random_logits(100 + V % 97, B, L, V, dtype, 2.5, 0.4, 4.0, 16.0, sup)
    logits = to_dev(bits, dtype)
    log(f"greedy {dtype} B={B} L={L} V={V} suppress={sup}")
    gpu = stats_np(dc.token_stats(logits, suppress_ids=sup))
    ref = oracle.token_stats(bits, dtype, suppress_ids=sup)
    assert_stats(gpu, ref, dtype, f"{dtype} {B}x{L}x{V}")


def test_row_stride_larger_than_v():
    B, L, V, pad = 2, 6, 3000, 24
    bits, _ = random_logits(5, B, L, V + pad, "bf16", 2.0, 0.5, 5.0, 10.0)
    full = to_dev(bits, "bf16")
    view = full[:, :, :V]
    log("row_stride > V")
    gpu = stats_np(dc.token_stats(view))
    ref = oracle.token_stats(np.ascontiguousarray(bits[:, :, :V]), "bf16")
    assert_stats(gpu, ref, "bf16", "strided")


def test_peaked_rows_keep_relative_entropy_precision():
    """Rows whose top logit stands 20..90 nats above the rest: z- is tiny and the
    entropy must still be accurate relative to its own size."""
    rng = np.random.default_rng(1)
    B, L, V = 1, 24, 50000
    x = rng.standard_normal((B, L, V)).astype(np.float32)
    for l in range(L):
        x[0, l, rng.integers(V)] += 20.0 + 3.0 * l
    log("peaked rows f32")
    gpu = stats_np(dc.token_stats(to_dev(x)))
    ref = oracle.token_stats(x, "f32")
    assert_stats(gpu, ref, "f32", "peaked f32")
    assert np.all(ref.entropy > 0)


def test_exact_ties_at_the_maximum():
    """Several copies of the row maximum: x0 is the first, prob counts all."""
    rng = np.random.default_rng(2)
    B, L, V = 2, 8, 40000
    x = np.round(rng.standard_normal((B, L, V)) * 2).astype(np.float32)   # many ties
    for l in range(L):
        pos = rng.choice(V, size=1 + l, replace=False)
        x[0, l, pos] = 9.0
        x[1, l, pos] = 60.0                         # peaked ties
    bits = bf16_bits(x)
    for dtype, arr in (("f32", x), ("bf16", bits)):
        log(f"ties {dtype}")
        gpu = stats_np(dc.token_stats(to_dev(arr, dtype)))
        ref = oracle.token_stats(arr, dtype)
        assert_stats(gpu, ref, dtype, f"ties {dtype}")


def test_rotated_sweeps_keep_first_maximum_and_suppression():
    """Greedy rows are swept starting at a row-dependent iteration: the first
    occurrence of a tied maximum must still win wherever the sweep starts, and
    suppressed ids must be honoured in iterations visited after the wrap."""
    rng = np.random.default_rng(23)
    B, L, V = 1, 300, 65536
    x = np.round(rng.standard_normal((B, L, V)) * 2).astype(np.float32)
    sup = tuple(sorted({5, 100, 16390, 33000, 49200, 65535}))
    for l in range(L):
        pos = rng.choice(V, size=2 + l % 3, replace=False)   # tied maxima across iterations
        x[0, l, pos] = 20.0
        x[0, l, sup[l % len(sup)]] = 40.0                     # suppressed raw argmax
    bits = bf16_bits(x)
    log("rotated sweeps: ties and suppression")
    gpu = stats_np(dc.token_stats(to_dev(bits, "bf16"), suppress_ids=sup))
    ref = oracle.token_stats(bits, "bf16", suppress_ids=sup)
    assert_stats(gpu, ref, "bf16", "rotated sweeps")
    f32 = stats_np(dc.token_stats(to_dev(x), suppress_ids=sup))
    assert_stats(f32, oracle.token_stats(x, "f32", suppress_ids=sup), "f32", "rotated sweeps f32")


def _special_rows(V):
    rows = []
    r = np.random.default_rng(3).standard_normal(V).astype(np.float32)
    a = r.copy(); a[[5, 77, V - 1]] = np.nan; rows.append(a)                  # NaN entries
    rows.append(np.full(V, -np.inf, np.float32))                             # all -inf
    a = np.full(V, -np.inf, np.float32); a[V // 2] = np.nan; rows.append(a)  # -inf and NaN
    a = r.copy(); a[[3, 900]] = np.inf; rows.append(a)                       # +inf entries
    a = r.copy(); a[[3]] = np.inf; a[4] = np.nan; rows.append(a)
    a = np.full(V, np.nan, np.float32); rows.append(a)                        # all NaN
    a = r.copy(); a[: V // 2] = -np.inf; rows.append(a)                       # -inf prefix
    a = r.copy(); a[0] = 1e30; rows.append(a)                                 # huge finite
    a = np.full(V, -1e30, np.float32); a[V - 1] = -1e30 + 1e24; rows.append(a)
    return np.stack(rows)[None]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [0.0, 0.8])
def test_nan_and_inf_rows(dtype, T):
    V = 3000
    x = _special_rows(V)
    arr = bf16_bits(x) if dtype == "bf16" else x
    for sup in ((), (1, 3, 2999)):
        log(f"special rows {dtype} T={T} suppress={sup}")
        gpu = stats_np(dc.token_stats(to_dev(arr, dtype), temperature=T, seed=7, step=1,
                                      suppress_ids=sup))
        ref = oracle.token_stats(arr, dtype, temperature=T, seed=7, step=1, suppress_ids=sup)
        assert_stats(gpu, ref, dtype, f"special {dtype} T={T}", x0_exact=(T == 0.0),
                     mask=(gpu[0] == ref.x0))
        assert_stats(gpu, ref, dtype, "special entropy", x0_exact=False, fields=("entropy",))
        if T > 0:
            pos = [(0, l) for l in range(x.shape[1])]
            assert_sampled_x0(gpu[0], ref.x0, arr, dtype, T, 7, 1, sup, pos, "special sampled")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [0.0, 0.8])
def test_special_rows_in_split_rows_with_a_rule(dtype, T):
    """Degenerate rows (NaN, +-inf, all -inf) split across workgroups and
    finished by the workgroup that completes their batch row, with a fused
    rule on the same statistics."""
    V = 20000
    x = _special_rows(V)
    arr = bf16_bits(x) if dtype == "bf16" else x
    B, L = x.shape[0], x.shape[1]
    cand = np.ones((B, L), dtype=bool)
    cand[0, ::3] = False
    for sup in ((), (1, 3, V - 1)):
        log(f"split special rows {dtype} T={T} suppress={sup}")
        r = dc.Rule.threshold(to_dev(cand), 0.5)
        st = dc.token_stats(to_dev(arr, dtype), temperature=T, seed=7, step=1, suppress_ids=sup,
                            rules=[r])
        gpu = stats_np(st)
        ref = oracle.token_stats(arr, dtype, temperature=T, seed=7, step=1, suppress_ids=sup)
        assert_stats(gpu, ref, dtype, f"split special {dtype} T={T}", x0_exact=(T == 0.0),
                     mask=(gpu[0] == ref.x0))
        assert_stats(gpu, ref, dtype, "split special entropy", x0_exact=False,
                     fields=("entropy",))
        want = oracle.threshold_transfer(gpu[1], cand, 0.5)
        assert np.array_equal(r.out.cpu().numpy(), want)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sparse_minus_inf_logits(dtype):
    """Masked vocabulary entries (-inf) scattered through otherwise finite rows,
    also next to a rising maximum: the fast path must keep every row finite."""
    rng = np.random.default_rng(21)
    B, L, V = 2, 12, 40000
    x = (rng.standard_normal((B, L, V)) * 3).astype(np.float32)
    x[rng.random((B, L, V)) < 0.01] = -np.inf
    for l in range(L):                     # -inf right beside rising maxima
        for k in range(1, 6):
            p = (k * 7001 + 13 * l) % (V - 1)
            x[0, l, p] = 8.0 + k + l
            x[0, l, p + 1] = -np.inf
    x[1, :, : V // 3] = -np.inf            # long masked prefix, then finite
    arr = bf16_bits(x) if dtype == "bf16" else x
    log(f"sparse -inf {dtype}")
    gpu = stats_np(dc.token_stats(to_dev(arr, dtype)))
    ref = oracle.token_stats(arr, dtype)
    assert_stats(gpu, ref, dtype, f"sparse -inf {dtype}")
    assert np.all(np.isfinite(gpu[1])) and np.all(np.isfinite(gpu[2]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_large_magnitude_logits(dtype):
    """Offsets and scales far from unit logits: weights are taken against
    RN(M log2 e) and converted back exactly; beyond |M| log2 e > FLT_MAX the
    row takes the two-pass path."""
    rng = np.random.default_rng(22)
    V = 20000
    base = rng.standard_normal(V).astype(np.float32)
    rows = [base * 2 + 3.0e4, base * 2 - 3.0e4, base * 3 + 1.0e6, base * 0.5 - 7.7e5,
            base * 1e35 + 1e37, np.float32(2.9e38) + base * 1e36,
            np.full(V, 3.0e38, np.float32) - np.abs(base) * 1e37, base * 1e36 - 3.0e38]
    x = np.stack([np.clip(r, -3.3e38, 3.3e38) for r in rows]).astype(np.float32)[None]
    arr = bf16_bits(x) if dtype == "bf16" else x
    log(f"large magnitudes {dtype}")
    gpu = stats_np(dc.token_stats(to_dev(arr, dtype)))
    ref = oracle.token_stats(arr, dtype)
    assert_stats(gpu, ref, dtype, f"large {dtype}")


def test_workspace_left_zero_filled_across_shapes():
    """The header's workspace contract: every call leaves the workspace
    zero-filled, so a later call of another shape (whose counters may lie where
    the first call's split-row partials were) starts clean."""
    shapes = [(1, 3, 262144), (2, 40, 30000), (1, 70, 65536), (3, 5, 9000)]
    need = 0
    for (B, L, V) in shapes:
        need = max(need, int(dc.load_library().dllm_token_stats_workspace_size(dc.DLLM_BF16, B, L, V)))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for i, (B, L, V) in enumerate(shapes):
            bits, rng = random_logits(300 + i, B, L, V, "bf16", 2.0, 0.5, 5.0, 12.0)
            cand = torch.from_numpy(rng.random((B, L)) < 0.5).cuda()
            r = dc.Rule.entropy_bound(cand, 0.5)
            log(f"workspace reuse {B}x{L}x{V} pass {rep}")
            st = dc.token_stats(to_dev(bits, "bf16"), temperature=0.7 if rep else 0.0, seed=5,
                                rules=[r], workspace=ws)
            torch.cuda.synchronize()
            assert int(torch.count_nonzero(ws)) == 0, f"workspace dirty after {B}x{L}x{V}"
            ref = oracle.token_stats(bits, "bf16", temperature=0.7 if rep else 0.0, seed=5)
            gpu = stats_np(st)
            if rep == 0:
                assert_stats(gpu, ref, "bf16", f"reuse {B}x{L}x{V}")
            eb = oracle.entropy_bound_transfer(gpu[2], cand.cpu().numpy(), 0.5)
            assert np.array_equal(r.out.cpu().numpy(), eb)


def test_suppressed_argmax_and_many_ids():
    rng = np.random.default_rng(4)
    B, L, V = 2, 6, 70000
    x = (rng.standard_normal((B, L, V)) * 2).astype(np.float32)
    sup = tuple(sorted(set(int(v) for v in rng.choice(V, size=62, replace=False)) | {0, V - 1}))
    for b in range(B):
        for l in range(L):
            x[b, l, sup[(b * L + l) % len(sup)]] += 30.0          # suppressed raw argmax
    bits = bf16_bits(x)
    log(f"suppress {len(sup)} ids")
    gpu = stats_np(dc.token_stats(to_dev(bits, "bf16"), suppress_ids=sup))
    ref = oracle.token_stats(bits, "bf16", suppress_ids=sup)
    assert_stats(gpu, ref, "bf16", "suppress")
    assert not np.isin(gpu[0], sup).any()


def test_sampled_suppressed_id_in_the_winning_group():
    """Gumbel-max with a suppressed id of huge raw logit next to the token that
    should win: the sampled pick shares its group of four generator words with
    the suppressed id, and must still skip it."""
    rng = np.random.default_rng(6)
    B, L, V = 1, 12, 40000
    x = (rng.standard_normal((B, L, V)) * 2).astype(np.float32)
    sup = tuple(1000 + 5 * l for l in range(L))              # every slot of a group of four
    for l in range(L):
        s0 = sup[l]
        x[0, l, s0] += 40.0                                   # suppressed raw argmax
        x[0, l, (s0 & ~3) + ((s0 + 1) & 3)] += 25.0           # the winner, same group
    bits = bf16_bits(x)
    for T in (0.7, 1.0):
        gpu = stats_np(dc.token_stats(to_dev(bits, "bf16"), temperature=T, seed=11, step=2,
                                      suppress_ids=sup))
        ref = oracle.token_stats(bits, "bf16", temperature=T, seed=11, step=2, suppress_ids=sup)
        pos = [(0, l) for l in range(L)]
        assert_sampled_x0(gpu[0], ref.x0, bits, "bf16", T, 11, 2, sup, pos, "sampled suppress")
        assert not np.isin(gpu[0], sup).any()
        assert_stats(gpu, ref, "bf16", "sampled suppress stats", mask=(gpu[0] == ref.x0))


@pytest.mark.parametrize("dtype,B,L,V,T,seed,step", [
    ("bf16", 2, 16, 8192, 0.7, 1003, 0),
    ("bf16", 1, 8, 151936, 0.7, 1003, 3),
    ("f32", 3, 10, 5000, 1.0, 2 ** 40 + 5, 17),
    ("f32", 1, 4, 40000, 0.9, 77, 5),              # split rows, 16-byte fp32 loads
    ("bf16", 1, 4, 1001, 2.5, 9, 2),               # odd V: unaligned rows, split path
])
def test_sampling_parity(dtype, B, L, V, T, seed, step):
    bits, _ = random_logits(V % 1000 + 1, B, L, V, dtype, 2.5, 0.35, 6.0, 14.0, (V - 1,))
    logits = to_dev(bits, dtype)
    log(f"sampling {dtype} B={B} L={L} V={V} T={T} seed={seed} step={step}")
    gpu = stats_np(dc.token_stats(logits, temperature=T, seed=seed, step=step,
                                  suppress_ids=(V - 1,)))
    ref = oracle.token_stats(bits, dtype, temperature=T, seed=seed, step=step,
                             suppress_ids=(V - 1,))
    pos = [(b, l) for b in range(B) for l in range(L)]
    assert_sampled_x0(gpu[0], ref.x0, bits, dtype, T, seed, step, (V - 1,), pos, "sampled")
    same = gpu[0] == ref.x0
    assert_stats(gpu, ref, dtype, "sampled stats", mask=same)
    assert_stats(gpu, ref, dtype, "sampled entropy", x0_exact=False, fields=("entropy",))


def test_sampling_is_fresh_per_step_and_zero_temperature_is_greedy():
    bits, _ = random_logits(8, 1, 64, 4096, "bf16", 1.0)
    logits = to_dev(bits, "bf16")
    greedy = stats_np(dc.token_stats(logits))[0]
    assert np.array_equal(stats_np(dc.token_stats(logits, temperature=0.0, seed=5))[0], greedy)
    a = stats_np(dc.token_stats(logits, temperature=1.0, seed=5, step=0))[0]
    b = stats_np(dc.token_stats(logits, temperature=1.0, seed=5, step=1))[0]
    assert (a != b).mean() > 0.5 and (a != greedy).mean() > 0.5


def test_repeated_launches_are_bit_identical():
    """Race check: fixed reduction orders make every launch identical."""
    for (B, L, V) in [(1, 3, 262144), (2, 40, 30000)]:
        bits, rng = random_logits(11, B, L, V, "bf16", 2.0, 0.5, 5.0, 12.0)
        logits = to_dev(bits, "bf16")
        cand = torch.from_numpy(rng.random((B, L)) < 0.5).cuda()
        first = None
        for i in range(30):
            r = dc.Rule.entropy_bound(cand, 0.5)
            st = dc.token_stats(logits, temperature=0.9 if i % 2 else 0.0, seed=3, rules=[r])
            out = [t.cpu().numpy().copy() for t in (st.x0, st.prob, st.entropy, r.out)]
            key = i % 2
            if first is None:
                first = {}
            if key not in first:
                first[key] = out
            else:
                for u, v in zip(out, first[key]):
                    assert np.array_equal(u.view(np.uint8), v.view(np.uint8))
    log("determinism ok")
