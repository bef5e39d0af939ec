#!/usr/bin/env python3
"""Throughput of the fused commit step on one MI355X.

Workload (the configuration the target is quoted on): a DiffusionGemma-like
canvas, B=1, L=256, V=262144 bf16 logits (workloads.config4), one fused launch
of dllm_token_stats (greedy) + entropy_bound (gamma 0.5, 154 candidates) +
edit (tau 0.9, 102 committed positions).  A step is that launch.

Inputs are resident in HBM before the timed region; the launch rotates over
--rotate copies of the logits (default 8 x 128 MiB = 1 GiB) so the 256 MB
Infinity Cache cannot serve repeated reads.  Before the step, a plain read of
the same copies (the read ceiling, 2 x 2000 launches) is timed; then --warmup
untimed launches, then exactly --steps launches timed with one pair of HIP
events on the stream they are enqueued on (value, ms_per_step), then the same
number of launches again (at least 20 groups of 25) in groups of 25
back-to-back launches, each group between its own pair of events
(per_launch: the median of the group means, the roofline's time per launch).

Prints one JSON line: logit GB/s (value), positions/s, steps/s, the roofline
of the kernel against the 8 TB/s HBM peak, and the oracle's throughput on
the host cores (cpu_baseline: a fork pool over this process's cores, taken
before the GPU is touched, with the one-worker figure beside it).
"""
import argparse
import ctypes
import hashlib
import glob
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "token_stats_diffusiongemma_canvas_counters.txt")


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--rotate", type=int, default=8, help="distinct copies of the logits")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum host time spent timing the oracle")
    p.add_argument("--copy-probe", action="store_true",
                   help="only run a plain 1 GiB device copy (counter calibration)")
    p.add_argument("--ceiling-launches", type=int, default=2000,
                   help="launches of each plain-read ceiling measurement")
    p.add_argument("--workload", default="diffusiongemma_canvas",
                   choices=["diffusiongemma_canvas", "diffusiongemma_stats", "llada_block_loop",
                            "tiny", "dream_canvas", "dream_unaligned", "batched"],
                   help="diffusiongemma_canvas (default, the headline step); diffusiongemma_stats "
                        "(the same canvas, dllm_token_stats with no rule fused); llada_block_loop "
                        "(the 32-step LLaDA block with dllm_commit_step); tiny (1 x 64 x 4096 "
                        "fp32, threshold); dream_canvas (4 x 256 x 151936 bf16, Gumbel-max "
                        "T = 0.7, factor); dream_unaligned (the same, rows V + 1 elements apart, "
                        "so not 16-byte aligned); batched (32 x 512 x 126464 bf16, strict "
                        "threshold)")
    return p.parse_args()


def kernel_source_hash():
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "commit_step_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "dllm_commit.h"))
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()


def read_traffic(src_hash):
    """HBM bytes per launch measured by rocprofv3 counters, if they were taken on
    the current kernel sources; else None."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as fh:
            for ln in fh:
                if "=" in ln and not ln.startswith("#"):
                    k, v = ln.strip().split("=", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256") != src_hash:
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def copy_probe():
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)


_CPU_W = None                     # the workload, inherited by the forked workers


def _oracle_positions(chunk):
    """The oracle's statistics at a list of (b, l) positions (a pool task)."""
    import oracle
    st = oracle.token_stats(_CPU_W.logits, "bf16", positions=chunk)
    return [(b, l, int(st.x0[b, l]), float(st.prob[b, l]), float(st.entropy[b, l]))
            for b, l in chunk]


def _oracle_step(pool, chunks):
    """One commit step of the oracle as it stands: statistics of every position
    (spread over the pool's workers, or in this process), then entropy_bound
    and edit on the whole canvas."""
    import numpy as np
    import oracle
    w = _CPU_W
    B, L, _ = w.shape
    x0 = np.zeros((B, L), dtype=np.int32)
    prob = np.zeros((B, L))
    ent = np.zeros((B, L))
    parts = pool.map(_oracle_positions, chunks) if pool is not None else \
        [_oracle_positions(c) for c in chunks]
    for part in parts:
        for b, l, x, pr, en in part:
            x0[b, l], prob[b, l], ent[b, l] = x, pr, en
    p = w.params
    oracle.entropy_bound_transfer(ent.astype(np.float32), w.cand, p["gamma"])
    oracle.edit_transfer(x0, prob.astype(np.float32), w.tokens, w.editable, p["tau_edit"])


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, logit_bytes, min_seconds, max_workers=16):
    """The oracle as it stands on the same canvas: a fork pool of one worker
    per core this process may run on (at most max_workers, the host share of
    one GPU), each computing the statistics of a share of the positions; the
    rules run in the parent.  Timed again with one worker for comparison.
    Must run before this process touches the GPU (the workers are forked)."""
    import multiprocessing as mp
    global _CPU_W
    _CPU_W = w
    B, L, V = w.shape
    affinity = len(os.sched_getaffinity(0))
    workers = max(1, min(affinity, max_workers))
    positions = [(b, l) for b in range(B) for l in range(L)]

    def run(pool, n_chunks, seconds):
        chunks = [positions[i::n_chunks] for i in range(n_chunks)]
        reps, t0 = 0, time.perf_counter()
        while True:
            _oracle_step(pool, chunks)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return reps, el

    reps1, el1 = run(None, 1, min_seconds / 2)
    with mp.get_context("fork").Pool(workers) as pool:
        _oracle_step(pool, [positions[i::workers] for i in range(workers)])     # start the workers
        reps, el = run(pool, workers, min_seconds)
    return {"value": round(logit_bytes * reps / el / 1e9, 4), "unit": "GB/s",
            "positions_per_s": round(B * L * reps / el, 2), "cores": workers, "kind": "oracle",
            "seconds": round(el, 2), "cpu_model": _cpu_model(), "affinity_cpus": affinity,
            "one_worker": {"value": round(logit_bytes * reps1 / el1 / 1e9, 4), "unit": "GB/s",
                           "seconds": round(el1, 2), "repetitions": reps1},
            "sample": f"the full canvas ({B}x{L}x{V} bf16) with entropy_bound and edit, "
                      f"{reps} repetition(s); numpy float64 oracle, statistics spread over "
                      f"{workers} forked worker process(es), rules in the parent"}


GROUP = 25         # back-to-back launches per pair of events in per_launch_us


def per_launch_us(launch, groups):
    """Device time per launch, as the mean over each of `groups` groups of
    GROUP back-to-back launches, each group between its own pair of HIP
    events on the launch stream (the current stream); returns the sorted
    group means in microseconds.  (A pair of events around every single
    launch adds the event packets' own time, a few microseconds, to each
    launch; over a group it adds a fraction of one.)"""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(groups)]
    for g in range(groups):
        ev[g][0].record()
        for i in range(GROUP):
            launch(g * GROUP + i)
        ev[g][1].record()
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) * 1e3 / GROUP for a, b in ev)


def launch_stats(us):
    n = len(us)
    med = us[n // 2] if n % 2 else 0.5 * (us[n // 2 - 1] + us[n // 2])
    return {"median_us": round(med, 3), "mean_us": round(sum(us) / n, 3),
            "p10_us": round(us[n // 10], 3), "p90_us": round(us[(9 * n) // 10], 3),
            "groups": n, "group_size": GROUP,
            "method": "median over the groups of each group's mean launch time; a group is "
                      f"{GROUP} back-to-back launches between one pair of HIP events"}


def llada_block_loop(args):
    """The LLaDA block (B=1, L=32, V=126464 bf16, 32 steps, top-k with the even
    quotas of transfer_schedule) as a loop of dllm_commit_step launches on the
    device canvas, timed with HIP events; the candidate masks and quotas of
    each step are recorded by one untimed pass first.  Run once reading only
    the candidate rows and once reading every row; each is timed as eager
    launches and as replays of the loop captured in a HIP graph."""
    import numpy as np
    import torch

    import commit_step_amd as dc
    import workloads

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    p = workloads.CONFIG_PARAMS[2]
    B, L, V, steps, mask_id = p["B"], p["L"], p["V"], p["steps"], p["mask_id"]
    logits = torch.empty((steps, B, L, V), dtype=torch.bfloat16, device=dev)
    for s in range(steps):
        w = workloads.config2_step(s)
        logits[s].copy_(torch.from_numpy(w.logits.view(np.int16)).view(torch.bfloat16))
    sup = w.suppress_ids
    init = torch.full((B, L), mask_id, dtype=torch.int32, device=dev)
    tok = init.clone()
    counts_n = torch.full((B,), L, dtype=torch.int32, device=dev)
    sched = dc.transfer_schedule(counts_n, steps)
    x0 = torch.empty((B, L), dtype=torch.int32, device=dev)
    pr = torch.empty((B, L), dtype=torch.float32, device=dev)
    en = torch.empty((B, L), dtype=torch.float32, device=dev)
    cands, ks, outs = [], [], []
    for s in range(steps):                               # record the trajectory
        cm = (tok == mask_id).to(torch.uint8)
        k = sched[:, s].contiguous()
        rule = dc.Rule.topk(cm, k)
        dc.commit_step(logits[s], tok, [rule], suppress_ids=sup, out=(x0, pr, en))
        cands.append(cm)
        ks.append(k)
        outs.append(rule.out)
    torch.cuda.synchronize()
    assert int((tok == mask_id).sum()) == 0, "the block did not finish"
    read_rows = sum(int(c.sum()) for c in cands)
    result = {}
    lib = dc.load_library()
    ws_bytes = int(lib.dllm_token_stats_workspace_size(dc.DLLM_BF16, B, L, V))
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    supa = (ctypes.c_int32 * len(sup))(*sup)
    fn = lib.dllm_commit_step
    for skip in (True, False):
        crules, canv, calls = [], [], []
        for s in range(steps):                          # prebuilt C arguments
            cr = (dc._CRule * 1)()
            cr[0].kind, cr[0].mask, cr[0].out = dc.RULE_TOPK, cands[s].data_ptr(), outs[s].data_ptr()
            cr[0].k = ks[s].data_ptr()
            cv = dc._CCanvas()
            cv.tokens, cv.counts, cv.skip_rows = tok.data_ptr(), None, int(skip)
            crules.append(cr)
            canv.append(cv)
            calls.append((logits[s].data_ptr(), dc.DLLM_BF16, B, L, V, V, 0.0, 0, 0, supa, len(sup),
                          x0.data_ptr(), pr.data_ptr(), en.data_ptr(), None, cr, 1, ctypes.byref(cv),
                          ws.data_ptr(), ws.numel(), stream))

        def loop():
            tok.copy_(init)
            rc = 0
            for c in calls:
                rc |= fn(*c)
            if rc:
                raise RuntimeError(lib.dllm_last_error().decode())
        for _ in range(max(1, args.warmup // 10)):
            loop()
        torch.cuda.synchronize()
        t0 = time.perf_counter()                         # >= 0.1 s: steady clocks
        while time.perf_counter() - t0 < 0.1:
            loop()
            torch.cuda.synchronize()
        reps = max(1, args.steps // 10)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            loop()
        b.record()
        torch.cuda.synchronize()
        ms_eager = a.elapsed_time(b) / reps
        assert int((tok == mask_id).sum()) == 0
        # the same loop captured once as a HIP graph (launch arguments are fixed
        # at capture; no memset nodes) and replayed: device time without host gaps
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            cs = torch.cuda.current_stream(dev).cuda_stream
            calls = [c[:-1] + (cs,) for c in calls]
            loop()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream(dev).cuda_stream
            calls = [c[:-1] + (cs,) for c in calls]
            loop()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int((tok == mask_id).sum()) == 0
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        ms_loop = a.elapsed_time(b) / reps
        assert int((tok == mask_id).sum()) == 0
        rows = read_rows if skip else steps * B * L
        result[skip] = {"ms_per_loop": round(ms_loop, 4), "us_per_step": round(ms_loop * 1e3 / steps, 3),
                        "us_per_step_eager": round(ms_eager * 1e3 / steps, 3),
                        "logit_bytes_read": rows * V * 2,
                        "logit_gb_s": round(rows * V * 2 / (ms_loop * 1e-3) / 1e9, 1)}
    line = {"metric": "LLaDA block loop: commit steps/s (dllm_commit_step on the device canvas)",
            "value": round(steps / (result[True]["ms_per_loop"] * 1e-3), 1), "unit": "steps/s",
            "n_gpus": 1, "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "llada_block_loop: B=1, L=32, V=126464 bf16, 32 steps, "
                                   "topk with transfer_schedule quotas", "steps": steps},
            "candidate_rows_only": result[True], "every_row": result[False],
            "bytes_saved_frac": round(1 - read_rows / (steps * B * L), 4)}
    print(json.dumps(line), flush=True)


def fused_workload(args):
    """One fused launch of dllm_token_stats with the configuration's rule,
    timed like the headline step; logit GB/s against the 8 TB/s peak."""
    import numpy as np
    import torch

    import commit_step_amd as dc
    import workloads

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.workload == "batched":
        p = workloads.CONFIG_PARAMS[5]
        B, L, V = p["B"], p["L"], p["V"]
        copies = [torch.empty((B, L, V), dtype=torch.bfloat16, device=dev)]
        for b in range(B):                      # 4 GiB: one batch row at a time
            w = workloads.config5_batch_row(b)
            copies[0][b].copy_(torch.from_numpy(w.logits[0].view(np.int16)).view(torch.bfloat16))
        cand = torch.ones((B, L), dtype=torch.uint8, device=dev)
        kind, param, strict, T, seed, sup = dc.RULE_THRESHOLD, p["tau"], int(p["strict"]), 0.0, 0, ()
        dtype, esz, label = dc.DLLM_BF16, 2, "batched: fused token_stats (greedy) + threshold(0.95, strict)"
    else:
        w = workloads.config1() if args.workload == "tiny" else workloads.config3()
        B, L, V = w.shape
        f32 = w.dtype == "f32"
        host = torch.from_numpy(w.logits) if f32 else \
            torch.from_numpy(w.logits.view(np.int16)).view(torch.bfloat16)
        R = max(1, args.rotate) if args.workload == "tiny" else 2
        if args.workload == "dream_unaligned":
            # rows V + 1 elements apart: every row starts at another offset
            # within 16 bytes (the split path)
            copies = []
            for _ in range(R):
                c = torch.empty((B, L, V + 1), dtype=host.dtype, device=dev)
                c[..., :V].copy_(host)
                copies.append(c)
        else:
            copies = [host.to(dev) for _ in range(R)]
        cand = torch.from_numpy(w.cand).to(dev)
        sup = tuple(w.suppress_ids)
        if args.workload == "tiny":
            kind, param, strict, T, seed = dc.RULE_THRESHOLD, w.params["tau"], int(w.params["strict"]), 0.0, 0
            label = "tiny: fused token_stats (greedy, fp32) + threshold(0.9)"
        else:
            kind, param, strict, T, seed = dc.RULE_FACTOR, w.params["f"], 0, w.temperature, w.seed
            label = "dream_canvas: fused token_stats (Gumbel-max T=0.7) + factor(1.0)"
            if args.workload == "dream_unaligned":
                label = ("dream_unaligned: the dream_canvas launch on rows V + 1 elements apart "
                         "(not 16-byte aligned)")
        dtype, esz = (dc.DLLM_F32, 4) if f32 else (dc.DLLM_BF16, 2)
    x0 = torch.empty((B, L), dtype=torch.int32, device=dev)
    prob = torch.empty((B, L), dtype=torch.float32, device=dev)
    ent = torch.empty((B, L), dtype=torch.float32, device=dev)
    out = torch.empty((B, L), dtype=torch.uint8, device=dev)
    lib = dc.load_library()
    ws = torch.zeros(max(int(lib.dllm_token_stats_workspace_size(dtype, B, L, V)), 256),
                     dtype=torch.uint8, device=dev)
    rules = (dc._CRule * 1)()
    rules[0].kind, rules[0].mask, rules[0].out = kind, cand.data_ptr(), out.data_ptr()
    rules[0].param, rules[0].strict = param, strict
    supa = (ctypes.c_int32 * max(1, len(sup)))(*sup)
    stream = torch.cuda.current_stream(dev).cuda_stream
    stride = V + 1 if args.workload == "dream_unaligned" else V
    calls = [(c.data_ptr(), dtype, B, L, V, stride, float(T), seed, 0, supa, len(sup), x0.data_ptr(),
              prob.data_ptr(), ent.data_ptr(), None, rules, 1, ws.data_ptr(), ws.numel(), stream)
             for c in copies]
    fn = lib.dllm_token_stats
    steps = args.steps if args.workload == "tiny" else max(1, args.steps // 5)
    rc = 0
    for i in range(max(1, args.warmup // 5)):
        rc |= fn(*calls[i % len(calls)])
    torch.cuda.synchronize()
    # at least 0.1 s of back-to-back launches before the timed region: the
    # GPU's clocks settle over that time (the sampled Dream-like launch ran
    # ~10% slower in its first hundred launches)
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < 0.1:
        for _ in range(20):
            rc |= fn(*calls[i % len(calls)])
            i += 1
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        rc |= fn(*calls[i % len(calls)])
    end.record()
    torch.cuda.synchronize()
    if rc:
        raise RuntimeError(lib.dllm_last_error().decode())
    ms = start.elapsed_time(end) / steps

    def one(i):
        nonlocal rc
        rc |= fn(*calls[i % len(calls)])
    per = launch_stats(per_launch_us(one, max(20, steps // GROUP)))
    if rc:
        raise RuntimeError(lib.dllm_last_error().decode())
    logit_bytes = B * L * V * esz
    gbs = logit_bytes / (ms * 1e-3) / 1e9
    line = {
        "metric": "logit GB/s of the fused token_stats + rule launch", "value": round(gbs, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": steps, "us_per_launch": round(ms * 1e3, 3),
        "per_launch": per,
        "higher_is_better": True, "dtype": "bf16" if esz == 2 else "f32", "data": "synthetic",
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "positions_per_s": round(B * L / (ms * 1e-3), 1),
        "config": {"workload": label, "B": B, "L": L, "V": V, "copies": len(copies)}}
    if args.workload == "batched":
        line["separate_calls"] = batched_separate_calls(dc, p, prob, cand, out, B, L)
    print(json.dumps(line), flush=True)


def batched_separate_calls(dc, p, prob, cand, out, B, L):
    """The batched workload's separate calls, each timed alone (device calls as
    graph replays): the standalone threshold over the fused launch's
    probabilities, transfer_schedule, block_ranges (host) and the (2048, 2048)
    additive block-causal mask."""
    import torch

    def timed(fn, n=50, reps=10):
        # n launches captured in one HIP graph, so that the binding's host cost
        # (several microseconds a call) is not what is timed
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        g.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (n * reps) * 1e3

    res = {}
    us = timed(lambda: dc.threshold_transfer(prob, cand, p["tau"], strict=p["strict"], out=out))
    moved = B * L * (4 + 1 + 1)                  # conf read, candidates read, commit written
    res["threshold_transfer"] = {"B": B, "L": L, "us": round(us, 3),
                                 "gb_s": round(moved / (us * 1e-6) / 1e9, 1)}
    n_masked = torch.full((B,), L, dtype=torch.int32, device=prob.device)
    sched = torch.empty((B, L), dtype=torch.int32, device=prob.device)
    us = timed(lambda: dc.transfer_schedule(n_masked, L, out=sched))
    res["transfer_schedule"] = {"B": B, "steps": L, "us": round(us, 3)}
    t0 = time.perf_counter()
    for _ in range(1000):
        ranges = dc.block_ranges(p["prompt_len"], p["gen_len"], p["block_len"], align=True)
    res["block_ranges"] = {"prompt_len": p["prompt_len"], "gen_len": p["gen_len"],
                           "block_len": p["block_len"], "n_ranges": len(ranges),
                           "host_us": round((time.perf_counter() - t0) * 1e3, 3)}
    ML = p["mask_L"]
    mask = torch.empty((ML, ML), dtype=torch.float32, device=prob.device)
    us = timed(lambda: dc.block_causal_mask(ML, p["block_len"], out=mask))
    gbs = ML * ML * 4 / (us * 1e-6) / 1e9
    res["block_causal_mask"] = {"L": ML, "block_len": p["block_len"], "us": round(us, 3),
                                "write_gb_s": round(gbs, 1),
                                "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2)}
    return res


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus}: this benchmark runs on exactly one GPU; the commit "
              "step shards batch rows across GPUs with no communication, so a multi-GPU figure "
              "is the one-GPU figure times N and is not measured here.", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    if args.workload == "llada_block_loop":
        llada_block_loop(args)
        return
    if args.workload in ("tiny", "dream_canvas", "dream_unaligned", "batched"):
        fused_workload(args)
        return
    fused = args.workload == "diffusiongemma_canvas"

    import numpy as np
    import torch

    import commit_step_amd as dc
    import workloads

    w = workloads.config4()
    B, L, V = w.shape
    p = w.params
    logit_bytes = B * L * V * 2
    # the oracle's baseline first: its workers are forked before this process
    # touches the GPU
    cpu = None if args.no_cpu_baseline or not fused else \
        cpu_baseline(w, logit_bytes, args.cpu_seconds)

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    R = max(1, args.rotate)
    base = torch.from_numpy(w.logits.view(np.int16)).view(torch.bfloat16).to(dev)
    rot = torch.empty((R, B, L, V), dtype=torch.bfloat16, device=dev)
    for i in range(R):
        rot[i].copy_(base)
    del base
    cand = torch.from_numpy(w.cand).to(dev)
    editable = torch.from_numpy(w.editable).to(dev)
    tokens = torch.from_numpy(w.tokens).to(dev)
    x0 = torch.empty((B, L), dtype=torch.int32, device=dev)
    prob = torch.empty((B, L), dtype=torch.float32, device=dev)
    ent = torch.empty((B, L), dtype=torch.float32, device=dev)
    eb_out = torch.empty((B, L), dtype=torch.bool, device=dev)
    ed_out = torch.empty((B, L), dtype=torch.bool, device=dev)

    lib = dc.load_library()
    ws_bytes = int(lib.dllm_token_stats_workspace_size(dc.DLLM_BF16, B, L, V))
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    rules = (dc._CRule * 2)()
    rules[0].kind, rules[0].mask, rules[0].out = dc.RULE_ENTROPY_BOUND, cand.data_ptr(), eb_out.data_ptr()
    rules[0].param = p["gamma"]
    rules[1].kind, rules[1].mask, rules[1].out = dc.RULE_EDIT, editable.data_ptr(), ed_out.data_ptr()
    rules[1].param, rules[1].tokens = p["tau_edit"], tokens.data_ptr()
    stream = torch.cuda.current_stream(dev).cuda_stream
    call_args = [(rot[i].data_ptr(), dc.DLLM_BF16, B, L, V, V, 0.0, 0, 0, None, 0,
                  x0.data_ptr(), prob.data_ptr(), ent.data_ptr(), None, rules if fused else None,
                  2 if fused else 0, ws.data_ptr(), ws.numel(), stream) for i in range(R)]
    fn = lib.dllm_token_stats

    # the plain-read ceiling first: it also brings the GPU to its steady
    # clocks, as a decode loop that runs one step after another keeps it
    ceiling = read_ceiling(lib, rot, logit_bytes, B * L, stream, args.ceiling_launches)
    rc = 0
    for i in range(args.warmup):
        rc |= fn(*call_args[i % R])
    torch.cuda.synchronize()
    if rc:
        raise RuntimeError(lib.dllm_last_error().decode())

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        rc |= fn(*call_args[i % R])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if rc:
        raise RuntimeError(lib.dllm_last_error().decode())
    ms = start.elapsed_time(end) / args.steps
    # the launches again in groups between their own events: the median of
    # the group means is the kernel's device time per launch, the roofline's
    # denominator
    rc = 0

    def one(i):
        nonlocal rc
        rc |= fn(*call_args[i % R])
    per = launch_stats(per_launch_us(one, max(20, args.steps // GROUP)))
    if rc:
        raise RuntimeError(lib.dllm_last_error().decode())
    med_ms = per["median_us"] * 1e-3

    # cand, editable, tokens in; stats, masks out (the statistics alone: stats out)
    per_position = 1 + 1 + 4 + 12 + 1 + 1 if fused else 12
    alg_bytes = logit_bytes + B * L * per_position
    achieved = alg_bytes / (med_ms * 1e-3) / 1e9
    src_hash = kernel_source_hash()
    line = {
        "metric": "logit GB/s and positions/sec for token_stats+transfer; % of HBM peak",
        "value": round(logit_bytes / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "diffusiongemma_canvas: fused token_stats (greedy) + "
                               "entropy_bound(gamma=0.5) + edit(tau=0.9)" if fused else
                               "diffusiongemma_stats: token_stats (greedy), no rule",
                   "B": B, "L": L, "V": V, "logits": "bf16", "rotated_copies": R},
        "positions_per_s": round(B * L / (ms * 1e-3), 1),
        "steps_per_s": round(1e3 / ms, 1),
        "pct_hbm_peak": round(100.0 * achieved / HBM_PEAK_GBS, 2),
        "host_wall_ms_per_step": round(wall * 1e3 / args.steps, 5),
        "per_launch": per,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic(src_hash),
                     "time": "per_launch.median_us",
                     "frac_event_mean": round(alg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "kernel": "dllm::token_stats_kernel (bf16, greedy, 16-byte loads)" +
                               (" with entropy_bound and edit fused" if fused else ""),
                     "algorithmic_bytes_per_launch": alg_bytes},
        "kernel_source_sha256": src_hash,
    }
    ceiling["step_median_over_best_read"] = round(per["median_us"] / ceiling["best_us"], 3)
    line["read_ceiling"] = ceiling
    line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


def read_ceiling(lib, rot, logit_bytes, rows, stream, launches=2000):
    """A plain read of the same rotated logit copies (dllm_read_probe, the same
    16-byte loads, no arithmetic), timed with HIP events over `launches`
    launches: once with the step's decomposition (one row per 512-thread
    workgroup) and once over 8 x 256 workgroups of 256 threads."""
    import torch

    sink = torch.zeros(1, dtype=torch.int32, device=rot.device)
    res = {}
    for name, wgs, nt in (("row_per_workgroup", rows, 512), ("grid_2048x256", 2048, 256)):
        args_i = [(rot[i].data_ptr(), logit_bytes, wgs, nt, sink.data_ptr(), stream)
                  for i in range(rot.shape[0])]
        rc = 0
        for i in range(20):
            rc |= lib.dllm_read_probe(*args_i[i % len(args_i)])
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(launches):
            rc |= lib.dllm_read_probe(*args_i[i % len(args_i)])
        b.record()
        torch.cuda.synchronize()
        if rc:
            raise RuntimeError(lib.dllm_last_error().decode())
        us = a.elapsed_time(b) / launches * 1e3
        res[name] = {"workgroups": wgs, "threads": nt, "us": round(us, 3),
                     "gb_s": round(logit_bytes / (us * 1e-6) / 1e9, 1)}
    res["launches"] = launches
    res["best_us"] = min(v["us"] for v in res.values() if isinstance(v, dict))
    return res


if __name__ == "__main__":
    main()
