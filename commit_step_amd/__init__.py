"""Python binding of libdllm_commit (the dLLM commit step on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
library ``libdllm_commit.so`` next to this file.  PyTorch provides device
memory and the current stream.  There is no CPU fallback: if the library is
not built, every call raises.

Names and keyword arguments follow mlx-arsenal's ``mlx_arsenal.diffusion``
functions ("dLLM block decoding", "What mlx-arsenal ships"): token_stats,
threshold_transfer, topk_transfer, factor_transfer, entropy_bound_transfer,
edit_transfer, transfer_schedule, block_ranges, block_causal_mask.
"""
import contextlib
import ctypes
import os
from collections import namedtuple

import torch

__all__ = ["Stats", "Rule", "token_stats", "threshold_transfer", "topk_transfer",
           "factor_transfer", "entropy_bound_transfer", "edit_transfer",
           "transfer_schedule", "block_ranges", "block_causal_mask",
           "workspace_size", "library_path", "load_library", "commit_step", "CommitStep",
           "linear_temperature", "uniform_canvas", "renoise", "StableConfidentStopping",
           "decaying_threshold"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdllm_commit.so")

DLLM_F32, DLLM_BF16 = 0, 1
RULE_THRESHOLD, RULE_TOPK, RULE_FACTOR, RULE_ENTROPY_BOUND, RULE_EDIT = 1, 2, 3, 4, 5
SCORE_PROB, SCORE_MARGIN, SCORE_NEG_ENTROPY = 0, 1, 2
_SCORES = {"prob": SCORE_PROB, "margin": SCORE_MARGIN, "neg_entropy": SCORE_NEG_ENTROPY}
MAX_L = 4096
MAX_SUPPRESS = 64

Stats = namedtuple("Stats", ["x0", "prob", "entropy", "margin", "argmax"])
CommitStep = namedtuple("CommitStep", ["stats", "counts"])


class _CRule(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("mask", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("param", ctypes.c_double), ("strict", ctypes.c_int),
                ("k", ctypes.c_void_p), ("tokens", ctypes.c_void_p), ("score", ctypes.c_int),
                ("taus", ctypes.c_void_p)]


class _CStatsExtra(ctypes.Structure):
    _fields_ = [("margin", ctypes.c_void_p), ("argmax", ctypes.c_void_p),
                ("stats_temperature", ctypes.c_float)]


class _CCanvas(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_void_p), ("counts", ctypes.c_void_p),
                ("skip_rows", ctypes.c_int)]


_lib = None

# The exported C entry points and their signatures (include/dllm_commit.h).
_I64, _I32, _P = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
_SIGNATURES = {
    "dllm_token_stats": (_I32, [_P, _I32, _I64, _I64, _I64, _I64, ctypes.c_float, ctypes.c_uint64,
                                ctypes.c_uint64, _P, _I32, _P, _P, _P, _P, _P, _I32, _P,
                                ctypes.c_size_t, _P]),
    "dllm_token_stats_workspace_size": (ctypes.c_size_t, [_I32, _I64, _I64, _I64]),
    "dllm_commit_step": (_I32, [_P, _I32, _I64, _I64, _I64, _I64, ctypes.c_float, ctypes.c_uint64,
                                ctypes.c_uint64, _P, _I32, _P, _P, _P, _P, _P, _I32, _P, _P,
                                ctypes.c_size_t, _P]),
    "dllm_commit_step_static": (_I32, [_P, _I32, _I64, _I64, _I64, _I64, ctypes.c_float,
                                       ctypes.c_uint64, ctypes.c_uint64, _P, _I32, _P, _P, _P, _P,
                                       _P, _I32, _P, _P]),
    "dllm_transfer_threshold": (_I32, [_P, _P, _I64, _I64, ctypes.c_double, _I32, _P, _P]),
    "dllm_transfer_threshold_rows": (_I32, [_P, _P, _P, _I64, _I64, _I32, _P, _P]),
    "dllm_decaying_threshold": (_I32, [ctypes.c_double, ctypes.c_double, ctypes.c_double, _I64,
                                       ctypes.POINTER(ctypes.c_double)]),
    "dllm_transfer_topk": (_I32, [_P, _P, _P, _I64, _I64, _P, _P]),
    "dllm_transfer_factor": (_I32, [_P, _P, _I64, _I64, ctypes.c_double, _P, _P]),
    "dllm_transfer_entropy_bound": (_I32, [_P, _P, _I64, _I64, ctypes.c_double, _P, _P]),
    "dllm_transfer_edit": (_I32, [_P, _P, _P, _P, _I64, _I64, ctypes.c_double, _P, _P]),
    "dllm_transfer_schedule": (_I32, [_P, _I64, ctypes.c_int32, _P, _P]),
    "dllm_block_ranges": (_I64, [_I64, _I64, _I64, _I32, _P, _I64]),
    "dllm_block_causal_mask": (_I32, [_I64, _I64, _P, _P]),
    "dllm_linear_temperature": (_I32, [_I32, _I32, ctypes.c_double, ctypes.c_double,
                                       ctypes.POINTER(ctypes.c_double)]),
    "dllm_uniform_canvas": (_I32, [_P, _I64, _I64, _I64, ctypes.c_uint64, ctypes.c_uint64, _P]),
    "dllm_renoise": (_I32, [_P, _P, _P, _I64, _I64, _P, _P]),
    "dllm_stable_confident_stop": (_I32, [_P, _P, _I64, _I64, _I32, ctypes.c_double, _I32, _P, _P,
                                          _P, _P]),
    "dllm_read_probe": (_I32, [_P, _I64, _I64, _I32, _P, _P]),
    "dllm_stage_timestamps": (_I32, [_P, ctypes.c_size_t, _I32]),
    "dllm_last_error": (ctypes.c_char_p, []),
}


def library_path():
    return _LIB_PATH


_STAGES_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdllm_commit_stages.so")
_lib_stages = None


def _open(path):
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def load_library(stages=False):
    """Load libdllm_commit.so (raises if it has not been built).  stages=True
    loads libdllm_commit_stages.so instead, the same library with stage
    timestamps on (for commit_step_amd.stage_timing only)."""
    global _lib, _lib_stages
    if stages:
        if _lib_stages is None:
            if not os.path.exists(_STAGES_PATH):
                raise RuntimeError(f"{_STAGES_PATH} is not built; run "
                                   "`python -m commit_step_amd.build --stages`")
            _lib_stages = _open(_STAGES_PATH)
        return _lib_stages
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m commit_step_amd.build`")
        _lib = _open(_LIB_PATH)
    return _lib


def _check(status, what):
    if status < 0:
        msg = load_library().dllm_last_error().decode(errors="replace")
        raise ValueError(f"{what} failed with status {status}: {msg}")
    return status


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    return t


def _bl(t, name, dtypes, shape=None):
    _dev(t, name)
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype in {dtypes}, not {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and t.shape != shape:
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    return t


def _on(device):
    """The device's context, skipped when it is already the current device
    (entering it costs more host time than the launch itself)."""
    if device.index is None or device.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(device)


_ws_sizes = {}


def _ws_size(dt, B, L, V, device):
    key = (dt, B, L, V, device.index)
    n = _ws_sizes.get(key)
    if n is None:
        n = int(load_library().dllm_token_stats_workspace_size(dt, B, L, V))
        _ws_sizes[key] = n
    return n


# commit_step(..., workspace=STATIC_WORKSPACE) runs dllm_commit_step_static: no
# workspace tensor, no allocation (the library's own per-GPU array; calls that
# overlap on one GPU race).
STATIC_WORKSPACE = "static"
_MASK_DTYPES = (torch.bool, torch.uint8)
_workspaces = {}


def workspace_size(logits):
    B, L, V = logits.shape
    dt = DLLM_BF16 if logits.dtype == torch.bfloat16 else DLLM_F32
    with _on(logits.device):
        return int(load_library().dllm_token_stats_workspace_size(dt, B, L, V))


def _capturing(device):
    return device.type == "cuda" and torch.cuda.is_current_stream_capturing()


def _workspace(device, stream, nbytes):
    """The default workspace: a zero-filled byte buffer per (device, stream),
    grown on demand.  The library leaves it zero-filled after every
    successful call.  Calls in flight at the same time must not share a
    workspace (their row and batch-row counters would mix), and calls on one
    stream never overlap, so one buffer per stream is safe.  A buffer cannot
    be created or grown while the stream is being captured into a graph (the
    zero fill would become a node of the graph): make one eager call of the
    same or a larger shape first, or pass ``workspace=``."""
    key = (device.type, device.index, stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        if _capturing(device):
            raise RuntimeError(
                "the default workspace of this stream has to be created or grown during graph "
                "capture; make one eager call of this shape on the stream first, or pass "
                "workspace= (zero-filled, workspace_size() bytes)")
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


class Rule:
    """A commit rule fused into token_stats (same launch).

    Build with Rule.threshold / topk / factor / entropy_bound / edit; the
    result lands in ``rule.out`` (a bool (B, L) tensor).
    """

    def __init__(self, kind, mask, param=0.0, strict=False, k=None, tokens=None, out=None,
                 score="prob"):
        if score not in _SCORES:
            raise ValueError(f"score must be one of {sorted(_SCORES)}")
        self.taus = param if isinstance(param, torch.Tensor) else None
        if self.taus is not None and kind != RULE_THRESHOLD:
            raise ValueError("only the threshold rule takes one threshold per row")
        self.param = 0.0 if self.taus is not None else float(param)
        self.kind, self.mask, self.strict = kind, mask, bool(strict)
        self.k, self.tokens, self.out, self.score = k, tokens, out, _SCORES[score]

    @classmethod
    def threshold(cls, candidates, tau, strict=False, score="prob"):
        """score: "prob" (LLaDA, maskgit_plus), "margin" (topk_margin) or
        "neg_entropy" (Dream's entropy confidence).  tau: a number, or a (B,)
        float64 device tensor with one threshold per batch row."""
        return cls(RULE_THRESHOLD, candidates, tau, strict=strict, score=score)

    @classmethod
    def topk(cls, candidates, k, score="prob"):
        return cls(RULE_TOPK, candidates, k=k, score=score)

    @classmethod
    def factor(cls, candidates, f, score="prob"):
        return cls(RULE_FACTOR, candidates, f, score=score)

    @classmethod
    def entropy_bound(cls, candidates, gamma):
        return cls(RULE_ENTROPY_BOUND, candidates, gamma)

    @classmethod
    def edit(cls, editable, tokens, tau_edit):
        """tokens: the current canvas (may be None inside commit_step, which
        passes its own canvas)."""
        return cls(RULE_EDIT, editable, tau_edit, tokens=tokens)


def _k_tensor(k, B, device):
    if isinstance(k, torch.Tensor):
        return _bl(k, "k", (torch.int32,), (B,))
    return torch.full((B,), int(k), dtype=torch.int32, device=device)


def _row_stride(logits):
    """Elements between consecutive positions of (B, L, V) logits.  Sizes 0 and
    1 carry no stride information; otherwise the rows must be unit-stride and
    evenly spaced (position (b, l) at (b * L + l) * row_stride)."""
    B, L, V = logits.shape
    if B * L * V == 0:
        return max(V, 1)
    if V > 1 and logits.stride(2) != 1:
        raise ValueError("logits rows must be contiguous (unit stride along V)")
    if L > 1:
        rs = logits.stride(1)
    elif B > 1:
        rs = logits.stride(0)
    else:
        rs = V
    if B > 1 and logits.stride(0) != L * rs:
        raise ValueError("logits positions must be evenly strided: stride(0) == L * stride(1)")
    if rs < V:
        raise ValueError("logits rows overlap (row stride < V)")
    return rs


def token_stats(logits, temperature=0.0, seed=None, step=0, suppress_ids=(), rules=(),
                out=None, workspace=None, margin=False, argmax=False, stats_temperature=None):
    """Per-position (x0, prob, entropy, margin) of (B, L, V) float32 / bfloat16 logits.

    temperature > 0 draws x0 by Gumbel-max and then needs an explicit ``seed``
    (an integer key; ``step`` selects the per-step noise).  ``rules`` is a list
    of up to two Rule objects run in the same launch; their ``out`` tensors
    are filled.  ``margin`` (or a rule ranking by margin) adds the topk_margin
    confidence p1 - p2; otherwise Stats.margin is None.  ``argmax`` adds the
    greedy argmax (useful when x0 is sampled).  ``stats_temperature`` Ts makes
    prob / entropy / margin those of softmax(logits / Ts).  ``out`` may give
    preallocated (x0, prob, entropy[, margin]) tensors.
    """
    return _stats_call(logits, temperature, seed, step, suppress_ids, rules, out, workspace,
                       None, margin, argmax, stats_temperature)


def commit_step(logits, tokens, rules, temperature=0.0, seed=None, step=0, suppress_ids=(),
                skip_rows=True, counts=True, out=None, workspace=None, margin=False, argmax=False,
                stats_temperature=None):
    """One step of the decoding loop in one launch: token_stats with up to one
    ranking rule and one edit rule, then ``tokens`` (B, L) int32 is updated in
    place to x0 wherever a position was committed or edited.

    With ``skip_rows`` the logits of positions that no rule looks at are not
    read (their x0 / prob / entropy are left as they were).  ``counts`` (True,
    or a preallocated (B, 2) int32 tensor, device or pinned host) receives per
    batch row the candidates left uncommitted and the positions edited.
    ``workspace``: None (the stream's default buffer), a zero-filled uint8
    tensor of workspace_size() bytes, or STATIC_WORKSPACE (the library's own
    per-GPU array, no allocation; shapes up to DLLM_STATIC_SCRATCH_BYTES of
    workspace; calls that overlap on one GPU race).
    Returns CommitStep(stats, counts).
    """
    B, L = logits.shape[0], logits.shape[1]
    if tokens is not None:
        _bl(tokens, "tokens", (torch.int32,), (B, L))
    if counts is True:
        counts = torch.empty((B, 2), dtype=torch.int32, device=logits.device)
    elif counts is False:
        counts = None
    if counts is not None:
        if counts.dtype != torch.int32 or tuple(counts.shape) != (B, 2) or not counts.is_contiguous():
            raise ValueError("counts must be a contiguous (B, 2) int32 tensor")
        if not (counts.is_cuda or counts.is_pinned()):
            raise ValueError("counts must be device memory or pinned host memory")
    canvas = _CCanvas()
    canvas.tokens = tokens.data_ptr() if tokens is not None else None
    canvas.counts = counts.data_ptr() if counts is not None else None
    canvas.skip_rows = int(bool(skip_rows))
    stats = _stats_call(logits, temperature, seed, step, suppress_ids, rules, out, workspace,
                        (canvas, tokens, counts), margin, argmax, stats_temperature)
    return CommitStep(stats, counts)


def _stats_call(logits, temperature, seed, step, suppress_ids, rules, out, workspace, canvas,
                margin, argmax=False, stats_temperature=None):
    _dev(logits, "logits")
    if logits.dim() != 3:
        raise ValueError("logits must be (B, L, V)")
    if logits.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("logits must be float32 or bfloat16")
    B, L, V = logits.shape
    row_stride = _row_stride(logits)
    if temperature > 0 and seed is None:
        raise ValueError("sampling (temperature > 0) needs an explicit seed")
    dev = logits.device
    want_margin = bool(margin) or any(getattr(r, "score", 0) == SCORE_MARGIN for r in rules)
    mar = None
    if out is None:
        x0 = torch.empty((B, L), dtype=torch.int32, device=dev)
        prob = torch.empty((B, L), dtype=torch.float32, device=dev)
        ent = torch.empty((B, L), dtype=torch.float32, device=dev)
    else:
        x0, prob, ent = out[0], out[1], out[2]
        mar = out[3] if len(out) > 3 else None
        _bl(x0, "x0", (torch.int32,), (B, L))
        _bl(prob, "prob", (torch.float32,), (B, L))
        _bl(ent, "entropy", (torch.float32,), (B, L))
    if want_margin and mar is None:
        mar = torch.empty((B, L), dtype=torch.float32, device=dev)
    if mar is not None:
        _bl(mar, "margin", (torch.float32,), (B, L))
    am = torch.empty((B, L), dtype=torch.int32, device=dev) if argmax else None
    extra = _CStatsExtra()
    extra.margin = mar.data_ptr() if mar is not None else None
    extra.argmax = am.data_ptr() if am is not None else None
    extra.stats_temperature = float(stats_temperature) if stats_temperature else 0.0
    sup = (ctypes.c_int32 * max(len(suppress_ids), 1))(*[int(s) for s in suppress_ids])
    crules = (_CRule * 2)()
    keep = []
    for i, r in enumerate(rules):
        _bl(r.mask, "rule mask", _MASK_DTYPES, (B, L))
        if r.out is None:
            r.out = torch.empty((B, L), dtype=torch.bool, device=dev)
        _bl(r.out, "rule out", _MASK_DTYPES, (B, L))
        c = crules[i]
        c.kind, c.mask, c.out = r.kind, r.mask.data_ptr(), r.out.data_ptr()
        c.param, c.strict, c.score = r.param, int(r.strict), r.score
        if r.taus is not None:
            c.taus = _bl(r.taus, "taus", (torch.float64,), (B,)).data_ptr()
        if r.kind == RULE_TOPK:
            kt = _k_tensor(r.k, B, dev)
            keep.append(kt)
            c.k = kt.data_ptr()
        if r.kind == RULE_EDIT:
            if r.tokens is None and canvas is None:
                raise ValueError("the edit rule needs the current tokens")
            if r.tokens is not None:
                _bl(r.tokens, "tokens", (torch.int32,), (B, L))
                c.tokens = r.tokens.data_ptr()
    dt = DLLM_BF16 if logits.dtype == torch.bfloat16 else DLLM_F32
    lib = load_library()
    with _on(dev):
        stream = _stream(logits)
        args = [logits.data_ptr(), dt, B, L, V, row_stride, float(temperature),
                int(seed or 0) & 0xFFFFFFFFFFFFFFFF, int(step), sup, len(suppress_ids),
                x0.data_ptr(), prob.data_ptr(), ent.data_ptr(), ctypes.byref(extra),
                crules if len(rules) else None, len(rules)]
        if isinstance(workspace, str):
            if workspace != STATIC_WORKSPACE or canvas is None:
                raise ValueError("workspace='static' is taken by commit_step only")
            _check(lib.dllm_commit_step_static(*args, ctypes.byref(canvas[0]), stream),
                   "dllm_commit_step_static")
            return Stats(x0, prob, ent, mar, am)
        need = _ws_size(dt, B, L, V, dev)
        ws = workspace if workspace is not None else _workspace(dev, stream, need)
        if canvas is None:
            _check(lib.dllm_token_stats(*args, ws.data_ptr(), ws.numel(), stream),
                   "dllm_token_stats")
        else:
            _check(lib.dllm_commit_step(*args, ctypes.byref(canvas[0]), ws.data_ptr(),
                                        ws.numel(), stream), "dllm_commit_step")
    return Stats(x0, prob, ent, mar, am)


def _rule_out(conf, candidates, out):
    B, L = conf.shape
    _bl(candidates, "candidates", _MASK_DTYPES, (B, L))
    if out is None:
        out = torch.empty((B, L), dtype=torch.bool, device=conf.device)
    return _bl(out, "out", _MASK_DTYPES, (B, L))


def threshold_transfer(prob, candidates, threshold, strict=False, out=None):
    """Commit candidates with prob >= threshold (> when strict); force one if none pass.
    threshold: a number, or a (B,) float64 device tensor, one per batch row."""
    _bl(prob, "prob", (torch.float32,))
    out = _rule_out(prob, candidates, out)
    B, L = prob.shape
    if isinstance(threshold, torch.Tensor):
        taus = _bl(threshold, "threshold", (torch.float64,), (B,))
        with _on(prob.device):
            _check(load_library().dllm_transfer_threshold_rows(
                prob.data_ptr(), candidates.data_ptr(), taus.data_ptr(), B, L,
                int(bool(strict)), out.data_ptr(), _stream(prob)), "dllm_transfer_threshold_rows")
        return out
    with _on(prob.device):
        _check(load_library().dllm_transfer_threshold(
            prob.data_ptr(), candidates.data_ptr(), B, L, float(threshold), int(bool(strict)),
            out.data_ptr(), _stream(prob)), "dllm_transfer_threshold")
    return out


def decaying_threshold(tau_initial, tau_floor, decay, step):
    """max(tau_floor, tau_initial - decay * step): the linearly decaying
    confidence threshold with a floor."""
    out = ctypes.c_double()
    _check(load_library().dllm_decaying_threshold(float(tau_initial), float(tau_floor),
                                                   float(decay), int(step), ctypes.byref(out)),
           "dllm_decaying_threshold")
    return out.value


def topk_transfer(prob, candidates, k, out=None):
    """Commit the k[b] most confident candidates of every batch row."""
    _bl(prob, "prob", (torch.float32,))
    out = _rule_out(prob, candidates, out)
    B, L = prob.shape
    kt = _k_tensor(k, B, prob.device)
    with _on(prob.device):
        _check(load_library().dllm_transfer_topk(
            prob.data_ptr(), candidates.data_ptr(), kt.data_ptr(), B, L, out.data_ptr(),
            _stream(prob)), "dllm_transfer_topk")
    return out


def factor_transfer(prob, candidates, factor, out=None):
    """Commit the longest confidence-sorted prefix with (i+1)(1 - c_(i)) <= factor."""
    _bl(prob, "prob", (torch.float32,))
    out = _rule_out(prob, candidates, out)
    B, L = prob.shape
    with _on(prob.device):
        _check(load_library().dllm_transfer_factor(
            prob.data_ptr(), candidates.data_ptr(), B, L, float(factor), out.data_ptr(),
            _stream(prob)), "dllm_transfer_factor")
    return out


def entropy_bound_transfer(entropy, candidates, gamma, out=None):
    """Commit the longest entropy-sorted prefix with sum_{j<i} H_(j) <= gamma."""
    _bl(entropy, "entropy", (torch.float32,))
    out = _rule_out(entropy, candidates, out)
    B, L = entropy.shape
    with _on(entropy.device):
        _check(load_library().dllm_transfer_entropy_bound(
            entropy.data_ptr(), candidates.data_ptr(), B, L, float(gamma), out.data_ptr(),
            _stream(entropy)), "dllm_transfer_entropy_bound")
    return out


def edit_transfer(x0, prob, tokens, editable, editing_threshold, out=None):
    """edit = editable & (x0 != tokens) & (prob > editing_threshold)."""
    _bl(prob, "prob", (torch.float32,))
    B, L = prob.shape
    _bl(x0, "x0", (torch.int32,), (B, L))
    _bl(tokens, "tokens", (torch.int32,), (B, L))
    out = _rule_out(prob, editable, out)
    with _on(prob.device):
        _check(load_library().dllm_transfer_edit(
            x0.data_ptr(), prob.data_ptr(), tokens.data_ptr(), editable.data_ptr(), B, L,
            float(editing_threshold), out.data_ptr(), _stream(prob)), "dllm_transfer_edit")
    return out


def transfer_schedule(n_masked, steps, out=None):
    """(B, steps) int32 quotas spreading n_masked[b] evenly, extras first."""
    _bl(n_masked, "n_masked", (torch.int32,))
    B = n_masked.shape[0]
    if out is None:
        out = torch.empty((B, int(steps)), dtype=torch.int32, device=n_masked.device)
    _bl(out, "out", (torch.int32,), (B, int(steps)))
    with _on(n_masked.device):
        _check(load_library().dllm_transfer_schedule(
            n_masked.data_ptr(), B, int(steps), out.data_ptr(), _stream(n_masked)),
            "dllm_transfer_schedule")
    return out


def block_ranges(prompt_len, gen_len, block_len, align=False):
    """List of (start, end) blocks covering [prompt_len, prompt_len + gen_len)."""
    lib = load_library()
    n = _check(lib.dllm_block_ranges(int(prompt_len), int(gen_len), int(block_len),
                                     int(bool(align)), None, 0), "dllm_block_ranges")
    buf = (ctypes.c_int64 * max(2 * n, 2))()
    _check(lib.dllm_block_ranges(int(prompt_len), int(gen_len), int(block_len),
                                 int(bool(align)), buf, n), "dllm_block_ranges")
    return [(buf[2 * i], buf[2 * i + 1]) for i in range(n)]


def block_causal_mask(L, block_len, device="cuda", out=None):
    """(L, L) float32 additive mask: 0 within and below the query's block, -inf above."""
    if out is None:
        out = torch.empty((int(L), int(L)), dtype=torch.float32, device=device)
    _bl(out, "out", (torch.float32,), (int(L), int(L)))
    with _on(out.device):
        _check(load_library().dllm_block_causal_mask(int(L), int(block_len), out.data_ptr(),
                                                     _stream(out)), "dllm_block_causal_mask")
    return out


# ---------------------------------------------------------------- uniform-noise decoding

def linear_temperature(remaining, num_steps, t_min=0.4, t_max=0.8):
    """t_min + (t_max - t_min) * remaining / num_steps."""
    out = ctypes.c_double()
    _check(load_library().dllm_linear_temperature(int(remaining), int(num_steps), float(t_min),
                                                   float(t_max), ctypes.byref(out)),
           "dllm_linear_temperature")
    return out.value


def uniform_canvas(shape, vocab_size, seed, draw, device=None, out=None):
    """(B, L) int32 tokens uniform on [0, vocab_size) (Philox, counter-based)."""
    B, L = shape
    dev = torch.device(device) if device is not None else (out.device if out is not None
                                                           else torch.device("cuda"))
    if out is None:
        out = torch.empty((B, L), dtype=torch.int32, device=dev)
    _bl(out, "out", (torch.int32,), (B, L))
    with _on(out.device):
        _check(load_library().dllm_uniform_canvas(out.data_ptr(), B, L, int(vocab_size),
                                                  int(seed) & 0xFFFFFFFFFFFFFFFF, int(draw),
                                                  _stream(out)), "dllm_uniform_canvas")
    return out


def renoise(sample, accepted, noise, out=None):
    """where(accepted, sample, noise)."""
    _bl(sample, "sample", (torch.int32,))
    B, L = sample.shape
    _bl(accepted, "accepted", _MASK_DTYPES, (B, L))
    _bl(noise, "noise", (torch.int32,), (B, L))
    if out is None:
        out = torch.empty_like(sample)
    _bl(out, "out", (torch.int32,), (B, L))
    with _on(sample.device):
        _check(load_library().dllm_renoise(sample.data_ptr(), accepted.data_ptr(),
                                           noise.data_ptr(), B, L, out.data_ptr(),
                                           _stream(sample)), "dllm_renoise")
    return out


class StableConfidentStopping:
    """Per-row stop of the uniform-noise loop: stability_threshold consecutive
    unchanged argmax canvases and mean entropy <= confidence_threshold.  Call
    with (argmax, entropy); returns the (B,) bool done tensor, which only
    grows."""

    def __init__(self, stability_threshold=1, confidence_threshold=0.005):
        self.k, self.c = int(stability_threshold), float(confidence_threshold)
        self.prev = self.count = self.done = None

    def __call__(self, argmax, entropy):
        _bl(argmax, "argmax", (torch.int32,))
        B, L = argmax.shape
        _bl(entropy, "entropy", (torch.float32,), (B, L))
        first = self.prev is None
        if first:
            dev = argmax.device
            self.prev = torch.empty((B, L), dtype=torch.int32, device=dev)
            self.count = torch.zeros((B,), dtype=torch.int32, device=dev)
            self.done = torch.zeros((B,), dtype=torch.uint8, device=dev)
        with _on(argmax.device):
            _check(load_library().dllm_stable_confident_stop(
                argmax.data_ptr(), entropy.data_ptr(), B, L, self.k, self.c, int(first),
                self.prev.data_ptr(), self.count.data_ptr(), self.done.data_ptr(),
                _stream(argmax)), "dllm_stable_confident_stop")
        return self.done.bool()
