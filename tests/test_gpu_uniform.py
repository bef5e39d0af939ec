"""Uniform-noise decoding on the GPU against the oracle: the statistics
temperature and argmax output of token_stats, the canvas draws, renoise, the
stop rule, and the DiffusionGemma loop run on the device with a stand-in
model."""
import numpy as np
import pytest
import torch

import commit_step_amd as dc
import oracle
from gpu_util import assert_sampled_x0, assert_stats, log, stats_np, to_dev
from workloads import random_logits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,B,L,V,Ts,T", [
    ("f32", 2, 8, 5000, 0.55, 0.0),
    ("bf16", 1, 64, 40000, 0.4, 0.4),              # categorical sample of softmax(z)
    ("bf16", 2, 3, 262144, 2.5, 0.0),              # split rows
    ("f32", 1, 300, 9000, 0.8, 0.8),
])
def test_statistics_temperature_and_argmax(dtype, B, L, V, Ts, T):
    bits, _ = random_logits(60 + L, B, L, V, dtype, 2.5, 0.5, 4.0, 12.0)
    Ts32 = float(np.float32(Ts))
    log(f"stats temperature {dtype} B={B} L={L} V={V} Ts={Ts} T={T}")
    st = dc.token_stats(to_dev(bits, dtype), temperature=T, seed=7 if T else None, step=3,
                        stats_temperature=Ts32, argmax=True, margin=True)
    gx, gp, ge, gm = stats_np(st)
    ga = st.argmax.cpu().numpy()
    ref = oracle.token_stats(bits, dtype, temperature=T, seed=7 if T else None, step=3,
                             stats_temperature=Ts32)
    greedy = oracle.token_stats(bits, dtype)
    assert np.array_equal(ga, greedy.x0)
    if T == 0.0:
        assert_stats((gx, gp, ge, gm), ref, dtype, "scaled", fields=("prob", "entropy", "margin"))
    else:
        assert_stats((gx, gp, ge, gm), ref, dtype, "scaled sampled", x0_exact=False,
                     mask=gx == ref.x0)
        assert_stats((gx, gp, ge, gm), ref, dtype, "scaled sampled", x0_exact=False,
                     fields=("entropy", "margin"))
        pos = [(b, l) for b in range(B) for l in range(min(L, 64))]
        assert_sampled_x0(gx, ref.x0, bits, dtype, T, 7, 3, (), pos, "categorical")


@pytest.mark.parametrize("B,L,V,seed,draw", [(3, 17, 97, 5, 0), (2, 300, 262144, 2**40 + 3, 9),
                                             (1, 5, 1, 1, 1), (4, 64, 2**31 - 1, 77, 2**32 - 1)])
def test_uniform_canvas_bit_exact(B, L, V, seed, draw):
    got = dc.uniform_canvas((B, L), V, seed, draw).cpu().numpy()
    assert np.array_equal(got, oracle.uniform_canvas(B, L, V, seed, draw))


def test_renoise_bit_exact():
    rng = np.random.default_rng(2)
    s = rng.integers(0, 1000, size=(3, 70)).astype(np.int32)
    n = rng.integers(0, 1000, size=(3, 70)).astype(np.int32)
    acc = rng.random((3, 70)) < 0.4
    got = dc.renoise(torch.from_numpy(s).cuda(), torch.from_numpy(acc).cuda(),
                     torch.from_numpy(n).cuda()).cpu().numpy()
    assert np.array_equal(got, oracle.renoise(s, acc, n))


def test_stop_rule_matches_the_oracle_call_by_call():
    rng = np.random.default_rng(3)
    B, L = 5, 300
    for k, c in ((1, 0.25), (0, 0.1), (2, 0.005), (1, -0.5)):
        g = dc.StableConfidentStopping(k, c)
        o = oracle.StableConfidentStopping(k, c)
        done_o = np.zeros(B, dtype=bool)
        am = rng.integers(0, 9, size=(B, L)).astype(np.int32)
        for call in range(6):
            if call % 3 == 2:
                am[rng.integers(B), rng.integers(L)] += 1       # a change restarts the count
            h = (rng.random((B, L)) * 0.5 * c if c > 0 else rng.random((B, L))).astype(np.float32)
            h[0] = np.float32(c) if c > 0 else 0.0              # the mean exactly at the bound
            h[1, :2] = [np.inf, 0.0]                              # +inf: above a finite bound
            h[3, :2] = [-np.inf, 1.0] if call % 2 else [-np.inf, np.inf]   # -inf / undefined
            h[4, 0] = np.nan if call == 3 else h[4, 0]
            if L > 2 and c > 0:
                h[2] = np.float32(c)
                h[2, 0] = np.nextafter(np.float32(c), np.float32(10))   # a hair above
            d = g(torch.from_numpy(am).cuda(), torch.from_numpy(h).cuda()).cpu().numpy()
            done_o |= o(am, h)
            assert np.array_equal(d, done_o), (k, c, call)
    log("stop rule: call-by-call parity")


def test_stop_rule_infinite_and_large_bounds():
    """c = +-inf and a bound c L between 2^141 and 2^160, against the oracle."""
    L = 16384
    rows = np.zeros((6, L), dtype=np.float32)
    rows[0] = 3.4e38                                    # sum ~2^142
    rows[1] = 1.0
    rows[2, 0] = np.inf
    rows[3, 0] = -np.inf
    rows[4, :2] = [np.inf, -np.inf]
    rows[5] = -2.0
    am = np.zeros((6, L), dtype=np.int32)
    for c in (1.5e38, 4e38, np.inf, -np.inf, 0.5, -1.0):
        g = dc.StableConfidentStopping(0, c)
        o = oracle.StableConfidentStopping(0, c)
        d = g(torch.from_numpy(am).cuda(), torch.from_numpy(rows).cuda()).cpu().numpy()
        assert np.array_equal(d, o(am, rows)), (c, d)
    log("stop rule: infinite and large bounds")


def _stand_in_model(B, L, V, target):
    def model(canvas, step):
        # depends on the canvas: a position whose token already is the target
        # gets a sharper peak; row 1 stays unsure
        x = np.zeros((B, L, V), dtype=np.float32)
        x += np.random.default_rng(1000 + step).standard_normal((B, L, V)).astype(np.float32)
        for b in range(B):
            for l in range(L):
                if b != 1:
                    x[b, l, target[b, l]] += 6.0 + 3.0 * (canvas[b, l] == target[b, l]) + step
        return x
    return model


def test_diffusiongemma_loop_on_the_device():
    B, L, V, N, seed = 3, 40, 3000, 12, 1234
    target = np.random.default_rng(9).integers(0, V, size=(B, L))
    model = _stand_in_model(B, L, V, target)
    gamma, t_min, t_max = 0.1, 0.4, 0.8
    canvas = dc.uniform_canvas((B, L), V, seed, 0)
    stop = dc.StableConfidentStopping(1, 0.005)
    done = torch.zeros(B, dtype=torch.bool, device="cuda")
    argmax = canvas.clone()
    every = torch.ones((B, L), dtype=torch.uint8, device="cuda")
    record, steps = [], 0
    for remaining in range(N, 0, -1):
        steps += 1
        T = float(np.float32(dc.linear_temperature(remaining, N, t_min, t_max)))
        logits_np = model(canvas.cpu().numpy(), steps)
        rule = dc.Rule.entropy_bound(every, gamma)
        st = dc.token_stats(torch.from_numpy(logits_np).cuda(), temperature=T, seed=seed,
                            step=steps, stats_temperature=T, argmax=True, rules=[rule])
        gx, gp, ge = stats_np(st)[:3]
        record.append((logits_np, T, st.argmax.cpu().numpy(), gx, ge))
        # this step's statistics against the oracle
        ref = oracle.token_stats(logits_np, "f32", stats_temperature=T)
        assert np.array_equal(record[-1][2], ref.x0)
        assert_stats((ref.x0, gp, ge), ref, "f32", f"loop step {steps}", x0_exact=False,
                     fields=("entropy",))
        assert np.array_equal(rule.out.cpu().numpy(),
                              oracle.entropy_bound_transfer(ge, np.ones((B, L), bool), gamma))
        noise = dc.uniform_canvas((B, L), V, seed, steps)
        new_canvas = dc.renoise(st.x0, rule.out, noise)
        argmax = torch.where(done[:, None], argmax, st.argmax)
        canvas = torch.where(done[:, None], canvas, new_canvas)
        done = done | stop(argmax, st.entropy)
        if bool(done.all()):
            break

    def stats_fn(logits, T, step):
        lg, Tg, am, x0, ent = record[step - 1]
        assert np.array_equal(lg, logits) and Tg == T, "the two loops diverged"
        return am, x0, ent

    want, want_steps = oracle.decode_uniform(model, B, L, V, seed, num_steps=N,
                                             entropy_bound=gamma, t_min=t_min, t_max=t_max,
                                             stability_threshold=1, confidence_threshold=0.005,
                                             stats_fn=stats_fn)
    assert steps == want_steps
    assert np.array_equal(argmax.cpu().numpy(), want)
    assert np.array_equal(want[0], target[0]) and np.array_equal(want[2], target[2])
    log(f"diffusiongemma loop: {steps} steps, rows done {done.cpu().numpy().tolist()}")
