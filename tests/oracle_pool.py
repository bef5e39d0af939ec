"""The oracle's statistics over whole full-size workloads, in worker
processes (test infrastructure).

The oracle is a plain loop over positions, one row at a time; a full-size
workload takes minutes of it in one process.  The positions are spread over
fresh worker processes (the "spawn" start method: a new interpreter that
never touches the GPU).  Each worker regenerates the seeded workload itself
instead of receiving hundreds of megabytes of logits, and keeps the last one
it built."""
import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

_cache = {}


def _workload(key):
    if key not in _cache:
        import workloads
        _cache.clear()
        name, arg = key
        if name == "config3":
            _cache[key] = workloads.config3()
        elif name == "config5_batch_row":
            _cache[key] = workloads.config5_batch_row(arg)
        else:
            raise ValueError(name)
    return _cache[key]


def _task(key, positions, kwargs):
    import oracle
    w = _workload(key)
    st = oracle.token_stats(w.logits, w.dtype, positions=positions, **kwargs)
    return [(b, l, int(st.x0[b, l]), float(st.prob[b, l]), float(st.entropy[b, l]))
            for b, l in positions]


def workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def pool():
    return ProcessPoolExecutor(workers(), mp_context=mp.get_context("spawn"))


def gather(results, shape):
    """(x0, prob, entropy) arrays from the tasks' (b, l, x0, prob, entropy)."""
    x0 = np.full(shape, -1, dtype=np.int32)
    prob = np.full(shape, np.nan)
    ent = np.full(shape, np.nan)
    for part in results:
        for b, l, x, p, h in part:
            x0[b, l], prob[b, l], ent[b, l] = x, p, h
    return x0, prob, ent


def config3_stats(ex, w, step, chunks_per_worker=4):
    """Every position of the Dream-like canvas `w` (workloads.config3()) at
    one sampling step."""
    B, L, _ = w.shape
    pos = [(b, l) for b in range(B) for l in range(L)]
    n = workers() * chunks_per_worker
    kw = dict(temperature=w.temperature, seed=w.seed, step=step,
              suppress_ids=tuple(int(i) for i in w.suppress_ids))
    futs = [ex.submit(_task, ("config3", None), pos[i::n], kw) for i in range(n)]
    return gather([f.result() for f in futs], (B, L))


def config5_stats(ex):
    """Every position of the batched workload, one task per batch row; the
    task's row is batch row 0 of its own one-row workload."""
    import workloads
    p = workloads.CONFIG_PARAMS[5]
    B, L = p["B"], p["L"]
    futs = [ex.submit(_task, ("config5_batch_row", b), [(0, l) for l in range(L)], {})
            for b in range(B)]
    parts = [[(b, l, x, pr, h) for (_, l, x, pr, h) in f.result()] for b, f in enumerate(futs)]
    return gather(parts, (B, L))
