"""Where the time of one statistics launch goes: a per-stage timeline from the
stage-timestamp build of the library (libdllm_commit_stages.so).

Usage:
    python -m commit_step_amd.build --stages
    python -m commit_step_amd.stage_timing --workload canvas|canvas_stats|llada_step|tiny \\
        [--launches N] [--step S]

Thread 0 of every workgroup records the device's 100 MHz real-time counter
at each stage it reaches (start, stream end, slice counted, row merged,
finalized, published, stores drained, batch row counted, rule inputs loaded,
candidates ranked, batch row done); see dllm_stage_timestamps in
include/dllm_commit.h.  After a warm-up of back-to-back launches, each
measured launch runs alone (--burst 1: records cleared before it, read after
it) or as the last of --burst back-to-back launches, as in a decode loop; the
table gives, per stage, the median over launches of the time from the first
workgroup's start, plus the chain of the workgroup that completes the batch
row.  Inputs are the seeded synthetic workloads of ``workloads``:

  canvas        1 x 256 x 262144 bf16, fused entropy_bound + edit (8 rotated copies)
  canvas_stats  the same canvas, the statistics alone
  llada_step    1 x 32 x 126464 bf16, one commit step (top-k, canvas, row skipping)
  tiny          1 x 64 x 4096 fp32, fused threshold
"""
import argparse
import ctypes
import json
import statistics
import sys
import time

import numpy as np
import torch

import commit_step_amd as dc

STAGES = ["start", "stream_end", "slice_counted", "row_merged", "published", "batch_counted",
          "batch_done", "skipped", "finalized", "stores_drained", "rule_loaded", "rule_ranked",
          "spare12", "spare13", "spare14", "spare15"]
# the completing workgroup's stages in the order it passes them
CHAIN = ["start", "stream_end", "slice_counted", "row_merged", "finalized", "published",
         "stores_drained", "batch_counted", "rule_loaded", "rule_ranked", "batch_done"]
WORKGROUPS = 4096
TICK_NS = 10.0          # s_memrealtime: 100 MHz


def _canvas(rules_on, R=8):
    import workloads
    w = workloads.config4()
    B, L, V = w.shape
    dev = torch.device("cuda:0")
    base = torch.from_numpy(w.logits.view(np.int16)).view(torch.bfloat16).to(dev)
    rot = torch.empty((R, B, L, V), dtype=torch.bfloat16, device=dev)
    for i in range(R):
        rot[i].copy_(base)
    keep = {"rot": rot}
    for name, arr in (("cand", w.cand), ("editable", w.editable), ("tokens", w.tokens)):
        keep[name] = torch.from_numpy(arr).to(dev)
    for name, dt in (("x0", torch.int32), ("prob", torch.float32), ("ent", torch.float32),
                     ("eb", torch.bool), ("ed", torch.bool)):
        keep[name] = torch.empty((B, L), dtype=dt, device=dev)
    rules = (dc._CRule * 2)()
    rules[0].kind, rules[0].mask, rules[0].out = (dc.RULE_ENTROPY_BOUND, keep["cand"].data_ptr(),
                                                  keep["eb"].data_ptr())
    rules[0].param = w.params["gamma"]
    rules[1].kind, rules[1].mask, rules[1].out = (dc.RULE_EDIT, keep["editable"].data_ptr(),
                                                  keep["ed"].data_ptr())
    rules[1].param, rules[1].tokens = w.params["tau_edit"], keep["tokens"].data_ptr()
    keep["rules"] = rules
    return keep, (B, L, V), (rules if rules_on else None), (2 if rules_on else 0)


def setup(workload, lib, step):
    """(launch(i), description, keep-alive dict) for the workload."""
    import workloads
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    if workload in ("canvas", "canvas_stats"):
        keep, (B, L, V), rules, nr = _canvas(workload == "canvas")
        ws = torch.zeros(max(256, int(lib.dllm_token_stats_workspace_size(dc.DLLM_BF16, B, L, V))),
                         dtype=torch.uint8, device=dev)
        keep["ws"] = ws
        rot = keep["rot"]
        calls = [(rot[i].data_ptr(), dc.DLLM_BF16, B, L, V, V, 0.0, 0, 0, None, 0,
                  keep["x0"].data_ptr(), keep["prob"].data_ptr(), keep["ent"].data_ptr(), None,
                  rules, nr, ws.data_ptr(), ws.numel(), stream) for i in range(rot.shape[0])]

        def launch(i):
            return lib.dllm_token_stats(*calls[i % len(calls)])
        what = (f"{B}x{L}x{V} bf16, " + ("entropy_bound + edit fused" if nr else "no rule") +
                f", {rot.shape[0]} rotated copies")
        return launch, what, keep
    if workload == "llada_step":
        p = workloads.CONFIG_PARAMS[2]
        B, L, V, mask_id = p["B"], p["L"], p["V"], p["mask_id"]
        w = workloads.config2_step(step)
        logits = torch.from_numpy(w.logits.view(np.int16)).view(torch.bfloat16).to(dev)
        init = torch.full((B, L), mask_id, dtype=torch.int32, device=dev)
        tok = init.clone()
        cand = torch.ones((B, L), dtype=torch.uint8, device=dev)
        k = torch.ones((B,), dtype=torch.int32, device=dev)
        outs = {n: torch.empty((B, L), dtype=dt, device=dev)
                for n, dt in (("x0", torch.int32), ("prob", torch.float32),
                              ("ent", torch.float32), ("out", torch.bool))}
        counts = torch.empty((B, 2), dtype=torch.int32, device=dev)
        ws = torch.zeros(max(256, int(lib.dllm_token_stats_workspace_size(dc.DLLM_BF16, B, L, V))),
                         dtype=torch.uint8, device=dev)
        rules = (dc._CRule * 1)()
        rules[0].kind, rules[0].mask, rules[0].out, rules[0].k = (
            dc.RULE_TOPK, cand.data_ptr(), outs["out"].data_ptr(), k.data_ptr())
        cv = dc._CCanvas()
        cv.tokens, cv.counts, cv.skip_rows = tok.data_ptr(), counts.data_ptr(), 1
        sup = (ctypes.c_int32 * len(w.suppress_ids))(*w.suppress_ids)
        args = (logits.data_ptr(), dc.DLLM_BF16, B, L, V, V, 0.0, 0, 0, sup, len(w.suppress_ids),
                outs["x0"].data_ptr(), outs["prob"].data_ptr(), outs["ent"].data_ptr(), None,
                rules, 1, ctypes.byref(cv), ws.data_ptr(), ws.numel(), stream)
        keep = dict(logits=logits, init=init, tok=tok, cand=cand, k=k, outs=outs, counts=counts,
                    ws=ws, rules=rules, cv=cv, sup=sup)

        def launch(i):
            tok.copy_(init)
            return lib.dllm_commit_step(*args)
        return launch, f"{B}x{L}x{V} bf16, step {step}: top-k 1 over {L} candidates, canvas", keep
    if workload == "tiny":
        w = workloads.config1()
        B, L, V = w.shape
        logits = torch.from_numpy(w.logits).to(dev)
        cand = torch.from_numpy(w.cand).to(dev)
        outs = {n: torch.empty((B, L), dtype=dt, device=dev)
                for n, dt in (("x0", torch.int32), ("prob", torch.float32),
                              ("ent", torch.float32), ("out", torch.uint8))}
        ws = torch.zeros(max(256, int(lib.dllm_token_stats_workspace_size(dc.DLLM_F32, B, L, V))),
                         dtype=torch.uint8, device=dev)
        rules = (dc._CRule * 1)()
        rules[0].kind, rules[0].mask, rules[0].out = (dc.RULE_THRESHOLD, cand.data_ptr(),
                                                      outs["out"].data_ptr())
        rules[0].param, rules[0].strict = w.params["tau"], int(w.params["strict"])
        sup = (ctypes.c_int32 * max(1, len(w.suppress_ids)))(*w.suppress_ids)
        args = (logits.data_ptr(), dc.DLLM_F32, B, L, V, V, 0.0, 0, 0, sup, len(w.suppress_ids),
                outs["x0"].data_ptr(), outs["prob"].data_ptr(), outs["ent"].data_ptr(), None,
                rules, 1, ws.data_ptr(), ws.numel(), stream)
        keep = dict(logits=logits, cand=cand, outs=outs, ws=ws, rules=rules, sup=sup)

        def launch(i):
            return lib.dllm_token_stats(*args)
        return launch, f"{B}x{L}x{V} f32, threshold fused", keep
    raise ValueError(workload)


def read_stamps(lib):
    buf = (ctypes.c_uint64 * (WORKGROUPS * len(STAGES)))()
    if lib.dllm_stage_timestamps(buf, len(buf), 0) != 0:
        raise RuntimeError(lib.dllm_last_error().decode())
    a = np.frombuffer(buf, dtype=np.uint64).reshape(WORKGROUPS, len(STAGES)).astype(np.int64)
    return a[a[:, 0] != 0]                     # the workgroups that ran


def one_launch(lib, launch, i, burst=1):
    """The records of the last of `burst` back-to-back launches (cleared
    before the first; the earlier launches' records that the last one did not
    overwrite are older than its first start, and metrics() drops them)."""
    if lib.dllm_stage_timestamps(None, 0, 1) != 0:
        raise RuntimeError(lib.dllm_last_error().decode())
    torch.cuda.synchronize()
    for j in range(burst):
        if launch(i * burst + j) != 0:
            raise RuntimeError(lib.dllm_last_error().decode())
    torch.cuda.synchronize()
    return read_stamps(lib)


def metrics(ts):
    """Per-launch times in microseconds from the first workgroup's start.
    Records older than that start belong to an earlier launch: the newest of
    them gives the gap from the earlier launch's last recorded stage."""
    t0 = ts[:, 0].min()
    older = ts[(ts > 0) & (ts < t0)]
    ts = np.where(ts >= t0, ts, 0)
    us = lambda v: float(v - t0) * TICK_NS * 1e-3    # noqa: E731
    m = {"workgroups": int(ts.shape[0]), "last_start": us(ts[:, 0].max())}
    if older.size:
        m["gap_from_previous_launch"] = float(t0 - older.max()) * TICK_NS * 1e-3
    dur = (ts[:, 1] - ts[:, 0])[ts[:, 1] > 0] * TICK_NS * 1e-3
    if dur.size:
        m["stream_median_wg"] = float(np.median(dur))
        m["stream_max_wg"] = float(dur.max())
        ends = np.sort(ts[ts[:, 1] > 0, 1])
        m["stream_end_median"] = us(ends[len(ends) // 2])
        m["stream_end_last"] = us(ends[-1])
    for k, name in enumerate(STAGES[2:], start=2):
        col = ts[:, k][ts[:, k] > 0]
        if col.size:
            m[name + "_last"] = us(col.max())
    done = ts[:, 6] > 0
    if done.any():
        c = ts[np.argmax(ts[:, 6])]                  # the workgroup completing a batch row
        for name in CHAIN:
            k = STAGES.index(name)
            if c[k] > 0:
                m["completer_" + name] = us(c[k])
    return m


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--workload", default="canvas",
                    choices=["canvas", "canvas_stats", "llada_step", "tiny"])
    ap.add_argument("--launches", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=3000)
    ap.add_argument("--step", type=int, default=0, help="llada_step: the step's logits")
    ap.add_argument("--dump", default=None,
                    help="also write every launch's per-workgroup records (ticks from the first "
                         "start, -1: stage not passed) to this JSON file")
    ap.add_argument("--lib", default=None,
                    help="another stage-timestamp build of the library to load instead")
    ap.add_argument("--burst", type=int, default=1,
                    help="back-to-back launches per measured launch (the last is recorded)")
    args = ap.parse_args()
    torch.cuda.set_device(0)
    lib = dc.load_library(stages=True) if args.lib is None else dc._open(args.lib)
    launch, what, keep = setup(args.workload, lib, args.step)
    # counter rate: two launches 0.2 s apart on the host clock
    h0 = time.perf_counter()
    a = one_launch(lib, launch, 0)[:, 0].min()
    time.sleep(0.2)
    h1 = time.perf_counter()
    b = one_launch(lib, launch, 1)[:, 0].min()
    rate_mhz = float(b - a) / (h1 - h0) / 1e6
    for i in range(args.warmup):                     # steady clocks
        launch(i)
    torch.cuda.synchronize()
    rows, raw = [], []
    for i in range(args.launches):
        ts = one_launch(lib, launch, i, args.burst)
        rows.append(metrics(ts))
        if args.dump:
            t0 = ts[:, 0].min()
            raw.append(np.where(ts >= t0, ts - t0, -1).tolist())
    if args.dump:
        with open(args.dump, "w") as fh:
            json.dump({"workload": args.workload, "tick_ns": TICK_NS, "stages": STAGES,
                       "launches": raw}, fh)
    keys = [k for k in rows[0] if all(k in r for r in rows)]
    med = {k: statistics.median(r[k] for r in rows) for k in keys}
    how = "each alone" if args.burst == 1 else f"each the last of {args.burst} back-to-back"
    print(f"# stage timeline: {args.workload} ({what}); {args.launches} launches, {how}, "
          f"after {args.warmup} back-to-back; counter rate {rate_mhz:.1f} MHz (nominal 100)")
    print("| quantity | median over launches (us) |")
    print("|---|---|")
    for k in keys:
        print(f"| {k} | {med[k]:.3f} |" if k != "workgroups" else f"| workgroups | {int(med[k])} |")
    print(json.dumps({"workload": args.workload, "launches": args.launches, "burst": args.burst,
                      "counter_rate_mhz": round(rate_mhz, 2),
                      "median_us": {k: round(v, 3) for k, v in med.items()}}), flush=True)


if __name__ == "__main__":
    sys.exit(main())
