#!/usr/bin/env python3
"""Achieved HBM GB/s of the depthwise causal conv1d (fwd, bwd, update) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole hot path over one batch of seeded synthetic
input already resident in HBM:

  large_decode (default)
                    the largest one-GPU workload and the decode workload:
                    B=8 D=8192 T=8192, [B,T,D] storage behind a transpose
                    view, BF16 weight, no bias, SiLU: forward + backward with
                    the deterministic (fixed-order) dweight; then the decode
                    update B=256 D=8192, 64 single-token steps, BF16 weight +
                    bias, SiLU, state mutated in place.  The dense and packed
                    workloads' ops are timed after it and reported beside it.
  dense             B=4 D=4096 T=2048, channel-last, BF16 weight + bias,
                    initial states, SiLU: forward (returns final states) +
                    backward (FP32 atomics, dinit).
  packed            16 sequences, T=33,280, D=5120, FP32 weight, no bias,
                    initial states: forward + backward.
  decode            B=256 D=8192 update; a step is the 64 seeded tokens.
  large             B=8 D=8192 T=8192, no bias: forward + deterministic backward.
  tiny              B=1 D=64 T=128 [B,D,T]: forward (launch-bound).
  seqidx            the dense shape with sequences of U[64,1024] tokens per row
                    marked by seq_idx (no states): forward + backward.
  dense_tc, large_tc, packed_tc, seqidx_tc
                    the same data in [B,D,T] time-contiguous storage.
  dense_w2, dense_w3, dense_noact, dense_f32bias
                    the dense workload with filter width 2 or 3, without the
                    activation, or with an FP32 weight and FP32 bias (opt-in)
                    and the deterministic dweight and dbias (opt-in).
  decode_tokens     the decode shape, 64 tokens as 8 multi-token updates of
                    8 tokens each.
  dense_odd_tc      the dense workload at T=2047 in [B,D,T] storage: rows that
                    start on 2-byte boundaries only.

The value is algorithmic bytes (every compulsory input read once, every output
written once) per step divided by the wall time per step.  Per-op times come
from HIP events recorded on the stream the kernels run on.  Rank 0 prints one
JSON line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
MALL_BYTES = 256 << 20      # MI355X memory-side (Infinity) cache
DECODE_STATES = 16          # decode: states rotated over, so each launch finds its state in HBM
SPACER_CYCLES = 200000      # GPU spin before each timed op in the per-op pass
METRIC = "achieved HBM GB/s (% of MI355X peak) for fwd, bwd and update at 1 GPU"


WORKLOADS = ["large_decode", "dense", "packed", "decode", "large", "tiny", "seqidx",
             "dense_tc", "large_tc", "packed_tc", "seqidx_tc",
             "dense_w2", "dense_w3", "dense_noact", "dense_f32bias", "decode_tokens",
             "dense_odd_tc"]
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "depthwise_causal_conv1d_02_amd", "csrc")
OP_KERNEL = {"fwd": "k_fwd_chan", "bwd": "k_bwd_chan", "update": "k_update"}
OP_KERNEL_TIME = {"fwd": "k_fwd_tc", "bwd": "k_bwd_tc", "update": "k_update"}
OP_KERNEL_TIME_PACKED = {"fwd": "k_fwd_tcp", "bwd": "k_bwd_tcp", "update": "k_update"}
OP_KERNEL_TIME_SEQ = {"fwd": "k_fwd_tcs", "bwd": "k_bwd_tcs", "update": "k_update"}
UPDATE_KERNELS = ("k_update_staged", "k_update_vec", "k_update_tokens", "k_update_any")


def op_kernels(workload):
    """op -> kernel name prefix of a workload (time-lane kernels for *_tc;
    the packed and seq_idx rows' own time-lane kernels for those rows)."""
    if not workload.endswith("_tc"):
        return OP_KERNEL
    return {"packed_tc": OP_KERNEL_TIME_PACKED,
            "seqidx_tc": OP_KERNEL_TIME_SEQ}.get(workload, OP_KERNEL_TIME)


def profile_workload(workload, op):
    """The workload name a committed profile of `op` is filed under (the
    combined default workload runs the large workload's forward and backward
    and the decode workload's update)."""
    if workload == "large_decode":
        return "decode" if op == "update" else "large"
    return workload


def source_hash():
    """Hash of the kernel sources: counter figures taken from another version
    of the kernels are not reported."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(name.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def profile_path(kernel, workload):
    return os.path.join(PROFILES, "%s_%s.md" % (kernel, workload))


def recorded_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernels changed since it was taken."""
    path = profile_path(kernel, workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if line.startswith("<!-- traffic "):
                rec = json.loads(line[len("<!-- traffic "):].rsplit("-->", 1)[0])
                if rec.get("source_hash") == source_hash():
                    return rec
    return None


def act_bytes(B, D, T):
    return B * D * T * 2


def fwd_bytes(B, D, T, R, init, final, w_bytes, bias, W=4, b_bytes=2):
    st = R * D * (W - 1) * 2  # one BF16 state tensor
    return (2 * act_bytes(B, D, T) + (st if init else 0) + (st if final else 0)
            + D * W * w_bytes + (D * b_bytes if bias else 0))


def bwd_bytes(B, D, T, R, init, dfinal, w_bytes, bias, W=4, b_bytes=2):
    st = R * D * (W - 1) * 2
    return (3 * act_bytes(B, D, T) + (2 * st if init else 0) + (st if dfinal else 0)
            + D * W * w_bytes + D * W * 4 + ((D * b_bytes + D * 4) if bias else 0))


def update_bytes(B, D, w_bytes, bias):
    return B * D * 16 + D * 4 * w_bytes + (D * 2 if bias else 0)


def update_tokens_bytes(B, D, L, w_bytes, bias):
    """L tokens per call: the state read and written once, each token read
    and its output written."""
    return B * D * (12 + 4 * L) + D * 4 * w_bytes + (D * 2 if bias else 0)


# Algorithmic bytes per launch of each op of every workload, from the shapes
# alone (the summaries of rocprofv3 runs need them without a GPU).
WORKLOAD_BYTES = {
    "dense": {"fwd": fwd_bytes(4, 4096, 2048, 4, True, True, 2, True),
              "bwd": bwd_bytes(4, 4096, 2048, 4, True, False, 2, True)},
    "seqidx": {"fwd": fwd_bytes(4, 4096, 2048, 4, False, False, 2, True) + 4 * 2048 * 4,
               "bwd": bwd_bytes(4, 4096, 2048, 4, False, False, 2, True) + 4 * 2048 * 4},
    "packed": {"fwd": fwd_bytes(1, 5120, 33280, 16, True, True, 4, False),
               "bwd": bwd_bytes(1, 5120, 33280, 16, True, False, 4, False)},
    "large": {"fwd": fwd_bytes(8, 8192, 8192, 8, False, False, 2, False),
              "bwd": bwd_bytes(8, 8192, 8192, 8, False, False, 2, False)},
    "decode": {"update": update_bytes(256, 8192, 2, True)},
    "dense_w2": {"fwd": fwd_bytes(4, 4096, 2048, 4, True, True, 2, True, W=2),
                 "bwd": bwd_bytes(4, 4096, 2048, 4, True, False, 2, True, W=2)},
    "dense_w3": {"fwd": fwd_bytes(4, 4096, 2048, 4, True, True, 2, True, W=3),
                 "bwd": bwd_bytes(4, 4096, 2048, 4, True, False, 2, True, W=3)},
    "dense_noact": {"fwd": fwd_bytes(4, 4096, 2048, 4, True, True, 2, True),
                    "bwd": bwd_bytes(4, 4096, 2048, 4, True, False, 2, True)},
    "dense_f32bias": {"fwd": fwd_bytes(4, 4096, 2048, 4, True, True, 4, True, b_bytes=4),
                      "bwd": bwd_bytes(4, 4096, 2048, 4, True, False, 4, True, b_bytes=4)},
    "dense_odd": {"fwd": fwd_bytes(4, 4096, 2047, 4, True, True, 2, True),
                  "bwd": bwd_bytes(4, 4096, 2047, 4, True, False, 2, True)},
    "decode_tokens": {"update": update_tokens_bytes(256, 8192, 8, 2, True)},
}


class Workload:
    """Device tensors of one named workload and its per-op byte counts."""

    def __init__(self, name, dev):
        import torch
        from depthwise_causal_conv1d_02_amd import synth

        self.name, self.dev = name, dev
        # "<workload>_tc": the same data in [B,D,T] storage (unit time stride)
        self.kind = name[:-3] if name.endswith("_tc") else name
        to = lambda t: None if t is None else t.to(dev)
        if self.kind == "large_decode":
            # the large workload's forward and backward, then the decode
            # workload's 64 tokens, as one step
            self.large = Workload("large", dev)
            self.decode = Workload("decode", dev)
            self.cpu, self.g = self.large.cpu, self.large.g
            self.shape = dict(self.large.shape, decode_B=self.decode.shape["B"],
                              decode_tokens=self.decode.shape["tokens"])
            self.bytes = dict(self.large.bytes, update=self.decode.bytes["update"])
            self.counts = dict(self.large.counts, update=self.decode.counts["update"])
            self.desc = ("%s; then %s" % (self.large.desc, self.decode.desc))
            return
        variant = self.kind in synth.VARIANTS
        if variant:
            self.cpu = synth.variant(self.kind)
        else:
            idx = {"tiny": 1, "dense": 2, "packed": 3, "decode": 4, "large": 5,
                   "seqidx": 6}[self.kind]
            self.cpu = synth.workload(idx)
        if name.endswith("_tc"):
            self.cpu = dict(self.cpu, x=self.cpu["x"].contiguous(),
                            dy=None if self.cpu["dy"] is None else self.cpu["dy"].contiguous())
        w = self.cpu
        self.g = {k: to(v) if isinstance(v, torch.Tensor) else v for k, v in w.items()}
        self.ops = []
        if self.kind == "decode":
            B, D = w["conv_state"].shape[:2]
            n_tok = w["x_steps"].shape[0]
            self.shape = dict(B=B, D=D, tokens=n_tok)
            self.bytes = {"update": update_bytes(B, D, 2, True)}
            self.counts = {"update": n_tok}
            self.desc = ("decode update: B=%d D=%d, %d single-token steps per step, bf16 "
                         "weight+bias, SiLU, state mutated in place (rotating over %d states)"
                         % (B, D, n_tok, DECODE_STATES))
            return
        if self.kind == "decode_tokens":
            n_call, B, D, L = w["x_calls"].shape
            self.shape = dict(B=B, D=D, tokens=n_call * L, tokens_per_call=L)
            self.bytes = {"update": update_tokens_bytes(B, D, L, 2, True)}
            self.counts = {"update": n_call}
            self.desc = synth.VARIANTS[self.kind] + " (rotating over %d states)" % DECODE_STATES
            return
        x = w["x"]
        B, D, T = x.shape
        cu = w["cu_seqlens"]
        R = B if cu is None else cu.numel() - 1
        wb = 4 if w["weight"].dtype == torch.float32 else 2
        bias = w["bias"] is not None
        bb = 4 if bias and w["bias"].dtype == torch.float32 else 2
        init = w["initial_states"] is not None
        W = w["weight"].shape[1]
        self.shape = dict(B=B, D=D, T=T, R=R, W=W)
        seq = B * T * 4 if w.get("seq_idx") is not None else 0   # the int32 ids
        self.bytes = {"fwd": fwd_bytes(B, D, T, R, init, w["return_final_states"], wb, bias,
                                       W, bb) + seq}
        if w["dy"] is not None:
            self.bytes["bwd"] = bwd_bytes(B, D, T, R, init, False, wb, bias, W, bb) + seq
        self.counts = {k: 1 for k in self.bytes}
        self.desc = synth.VARIANTS[self.kind] if variant else synth.WORKLOADS[idx]
        if name.endswith("_tc"):
            self.desc = self.desc.replace("channel-last", "[B,D,T] time-contiguous")

    def step_bytes(self):
        return sum(self.bytes[k] * self.counts[k] for k in self.bytes)

    def cpu_view(self):
        """A copy of this workload without its device tensors (what the
        oracle baseline needs)."""
        import copy
        c = copy.copy(self)
        c.g = {}
        if self.kind == "large_decode":
            c.large, c.decode = self.large.cpu_view(), self.decode.cpu_view()
        return c

    def token_channels(self):
        """(token, channel) pairs one step processes."""
        if self.kind == "large_decode":
            return self.large.token_channels() + self.decode.token_channels()
        sh = self.shape
        return sh["B"] * sh["D"] * (sh["tokens"] if "tokens" in sh else sh["T"])

    def clone(self):
        """The same workload on fresh device copies of its tensors (strides
        kept), for timing with operands that are not in any cache."""
        import copy
        c = copy.copy(self)
        if self.kind == "large_decode":
            c.large, c.decode = self.large.clone(), self.decode.clone()
            c.g = c.large.g
            return c
        c.g = {k: (v.clone() if getattr(v, "is_cuda", False) else v) for k, v in self.g.items()}
        return c


def rotation_count(wl):
    """Operand copies to rotate over: between two uses of one copy, at least
    three times the memory-side cache of other traffic."""
    return max(2, min(16, -(-4 * MALL_BYTES // max(1, wl.step_bytes()))))


class Step:
    """One pass of the hot path: the ops of a step, run in order on the
    current stream."""

    def __init__(self, ops, outputs, flags):
        self.ops = ops            # [(op name, callable)]
        self.outputs = outputs
        self.flags = flags        # cu_seqlens flag words of packed calls

    def __call__(self, ev):
        for name, fn in self.ops:
            ev.begin(name)
            fn()
            ev.end(name)


def make_step(wl, torch):
    """Allocate every output once; return the Step of this workload."""
    from depthwise_causal_conv1d_02_amd import ops

    g, dev = wl.g, wl.dev
    if wl.kind == "large_decode":
        big, dec = make_step(wl.large, torch), make_step(wl.decode, torch)
        outputs = dict(big.outputs, decode_y=dec.outputs["y"])
        return Step(big.ops + dec.ops, outputs, big.flags + dec.flags)
    if wl.kind == "decode":
        states = [g["conv_state"].clone() for _ in range(DECODE_STATES)]
        xs = g["x_steps"]
        ys = torch.empty_like(xs)
        # one step decodes the seeded tokens in order, each in place on a
        # state; the states rotate so that no launch finds its state cached
        calls = [("update", (lambda s=s: ops.update(xs[s], states[s % DECODE_STATES],
                                                     g["weight"], g["bias"], g["activation"],
                                                     y=ys[s])))
                 for s in range(xs.shape[0])]
        return Step(calls, {"y": ys}, [])
    if wl.kind == "decode_tokens":
        states = [g["conv_state"].clone() for _ in range(DECODE_STATES)]
        xs = g["x_calls"]                       # [calls, B, D, L], unit channel stride
        ys = torch.empty_like(xs)
        calls = [("update", (lambda s=s: ops.update(xs[s], states[s % DECODE_STATES],
                                                     g["weight"], g["bias"], g["activation"],
                                                     y=ys[s])))
                 for s in range(xs.shape[0])]
        return Step(calls, {"y": ys}, [])

    x = g["x"]
    y = torch.empty_like(x)
    W = g["weight"].shape[1]
    opts = ops._options(g.get("fp32_weight_bias", False), g.get("deterministic_dbias", False))
    fin = None
    if g["return_final_states"]:
        fin = torch.empty(wl.shape["R"], x.shape[1], W - 1, dtype=x.dtype, device=dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    seq = g.get("seq_idx")
    calls = [("fwd", lambda: ops.fwd(x, g["weight"], g["bias"], g["cu_seqlens"],
                                     g["initial_states"], g["activation"],
                                     final_states_out=fin, y=y, err_flag=flag, seq_idx=seq,
                                     options=opts))]
    outputs = {"y": y}
    if g["dy"] is not None:
        dx = torch.empty_like(x)
        D = x.shape[1]
        # dweight and dbias live in one buffer, cleared by a single fill per step
        grads = torch.zeros(D * (W + 1), dtype=torch.float32, device=dev)
        dw = grads[:D * W].view(D, W)
        db = grads[D * W:] if g["bias"] is not None else None
        dinit = torch.empty_like(g["initial_states"]) if g["initial_states"] is not None else None
        ws = torch.empty(1 << 26, dtype=torch.uint8, device=dev) if g["deterministic"] else None
        calls.append(("zero_grads", grads.zero_))
        calls.append(("bwd", lambda: ops.bwd(x, g["weight"], g["dy"], g["bias"], g["cu_seqlens"],
                                             g["initial_states"], None, g["activation"],
                                             g["deterministic"], False, dx=dx, err_flag=flag,
                                             workspace=ws, dweight=dw, dbias=db, dinit=dinit,
                                             seq_idx=seq, options=opts)))
        outputs.update(dx=dx, dw=dw)
    return Step(calls, outputs, [flag] if g["cu_seqlens"] is not None else [])


class Events:
    """HIP events around each op on the current stream (the one the kernels use).

    With `spacer`, a short GPU spin runs before each start event, so that the
    host has queued the op before the GPU reaches it: the event pair then
    brackets the op's kernels, not host launch latency."""

    def __init__(self, torch, on, spacer=False):
        self.torch, self.on, self.spacer = torch, on, spacer
        self.rec = {}
        self.open = {}

    def begin(self, name):
        if self.on:
            if self.spacer:
                self.torch.cuda._sleep(SPACER_CYCLES)
            e = self.torch.cuda.Event(enable_timing=True)
            e.record()
            self.open[name] = e

    def end(self, name):
        if self.on:
            e = self.torch.cuda.Event(enable_timing=True)
            e.record()
            self.rec.setdefault(name, []).append((self.open.pop(name), e))

    def mean_ms(self):
        return {k: sum(a.elapsed_time(b) for a, b in v) / len(v) for k, v in self.rec.items()}


def _graph_launch_ms(torch, fns, n):
    """Mean ms per launch of n back-to-back launches cycling through fns,
    captured in one HIP graph (no host latency between launches) and timed
    by one event pair after a GPU spin; the median over three replays."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fns[i % len(fns)]()
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(3):
        torch.cuda._sleep(SPACER_CYCLES)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) / n)
    del g
    return sorted(ts)[1]


def op_times(torch, step, wl, reps):
    """Warm per-op times: `reps` back-to-back launches of each op kind on the
    same operands (the memory-side cache may serve part of them)."""
    seen = {}
    for name, fn in step.ops:
        if name in wl.bytes and name not in seen:
            seen[name] = _graph_launch_ms(torch, [fn], reps)
    return seen


def rotated_op_times(torch, steps, wl, rounds):
    """Cold per-op times: back-to-back launches of each op kind rotating over
    the workload's operand copies (one Step per copy), so every launch finds
    its operands in HBM, not in the memory-side cache."""
    res = {}
    for name in wl.bytes:
        fns = [fn for st in steps for (n, fn) in st.ops if n == name]
        res[name] = _graph_launch_ms(torch, fns, max(rounds * len(steps), len(fns)))
    return res


def check_flags(steps):
    """Packed calls report malformed offsets through their flag word, and a
    set word makes every later packed launch return early; a timing taken
    with one set would not be a timing of the op."""
    for st in steps:
        for fl in st.flags:
            v = int(fl.item())
            if v:
                raise RuntimeError("cu_seqlens flag word is %#x: the packed launches did no work"
                                   % v)


def op_kernel_label(wl, op):
    """The kernels one launch of `op` runs (the deterministic backward adds
    the fixed-order reduction of its partials)."""
    k = op_kernels(wl.name)[op]
    w = wl.large.cpu if wl.kind == "large_decode" else wl.cpu
    if op == "bwd" and w.get("deterministic"):
        k += " + k_dw_reduce"
    return k


def per_op_entry(wl, name, t, n_rot):
    gbs = wl.bytes[name] / (t * 1e-3) / 1e9
    return {"ms": round(t, 5), "algorithmic_bytes": wl.bytes[name],
            "launches_per_step": wl.counts[name], "kernels": op_kernel_label(wl, name),
            "GB_s": round(gbs, 1), "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "timing": "cold (rotating over %d operand copies)" % n_rot}


def other_config_ops(torch, dev, names, reps, warm_steps):
    """Cold per-op times of other workloads (their own operand copies), in
    the same run: the dense and packed configurations' forward and backward.
    Each workload first runs `warm_steps` whole steps, as a run of its own
    would before its per-op pass."""
    res = {}
    for name in names:
        print("bench: per-op times of workload %s" % name, file=sys.stderr, flush=True)
        wl = Workload(name, dev)
        n_rot = rotation_count(wl)
        wls = [wl] + [wl.clone() for _ in range(n_rot - 1)]
        steps = [make_step(w, torch) for w in wls]
        quiet = Events(torch, False)
        for i in range(max(1, warm_steps)):
            steps[i % n_rot](quiet)
        torch.cuda.synchronize()
        cold = rotated_op_times(torch, steps, wl, reps)
        check_flags(steps)
        res[name] = {"workload": wl.desc,
                     "ops": {k: per_op_entry(wl, k, t, n_rot) for k, t in cold.items()}}
        del steps, wls, wl
        torch.cuda.empty_cache()
    return res


def host_cpu():
    """The host the oracle baseline ran on: logical CPU count and model name."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "model": model}


class _OneCore:
    """Pin the calling thread to one CPU for the duration (the oracle is
    single-threaded C; pinning keeps the scheduler from moving it)."""

    def __enter__(self):
        self.prev = None
        self.cpu = None
        if hasattr(os, "sched_setaffinity"):
            self.prev = os.sched_getaffinity(0)
            self.cpu = min(self.prev)
            os.sched_setaffinity(0, {self.cpu})
        return self

    def __exit__(self, *exc):
        if self.prev is not None:
            os.sched_setaffinity(0, self.prev)
        return False


def _oracle_decode(wl, budget_s):
    """Oracle decode steps over every batch row, until the 64 tokens are done
    or the budget is spent: (seconds, bytes, steps, rows)."""
    import oracle
    w = wl.cpu
    f = lambda t: None if t is None else t.double().numpy()
    B, D = w["conv_state"].shape[:2]
    st = f(w["conv_state"])
    t0 = time.perf_counter()
    steps = 0
    while steps < w["x_steps"].shape[0] and time.perf_counter() - t0 < budget_s:
        _, st = oracle.update(f(w["x_steps"][steps]), st, f(w["weight"]), f(w["bias"]), "silu")
        steps += 1
    dt = time.perf_counter() - t0
    return dt, steps * update_bytes(B, D, 2, True), steps, B, D


def _oracle_decode_tokens(wl, budget_s):
    """Oracle multi-token updates (each call's L tokens on every batch row),
    until the calls are done or the budget is spent: (seconds, bytes, calls,
    rows, D, L)."""
    import oracle
    w = wl.cpu
    f = lambda t: None if t is None else t.double().numpy()
    n_call, B, D, L = w["x_calls"].shape
    st = f(w["conv_state"])
    t0 = time.perf_counter()
    calls = 0
    while calls < n_call and time.perf_counter() - t0 < budget_s:
        _, st = oracle.update_tokens(f(w["x_calls"][calls]), st, f(w["weight"]), f(w["bias"]),
                                     w["activation"])
        calls += 1
    dt = time.perf_counter() - t0
    return dt, calls * update_tokens_bytes(B, D, L, 2, True), calls, B, D, L


def _oracle_rows(wl, budget_s):
    """Oracle forward (+ backward) of a workload on a leading block of
    channels (all rows and tokens), sized by a short pilot to about
    `budget_s` seconds: (seconds, bytes, channels, D, has_bwd)."""
    import oracle
    w = wl.cpu
    f = lambda t: None if t is None else t.double().numpy()
    x = w["x"]
    B, D, T = x.shape
    cu = w["cu_seqlens"]
    cun = None if cu is None else cu.numpy()
    R = wl.shape["R"]
    wb = 4 if w["weight"].dtype.itemsize == 4 else 2
    has_bwd = w["dy"] is not None

    # Channels are independent, so a block of channels over every row and
    # token is the same workload, narrower.
    def run(nch):
        sub = lambda t: None if t is None else f(t[:, :nch] if t.dim() == 3 else t[:nch])
        xs, ws_, bs = sub(x), sub(w["weight"]), sub(w["bias"])
        init, dy = sub(w["initial_states"]), sub(w["dy"])
        seq = w.get("seq_idx")
        act = w["activation"]
        t0 = time.perf_counter()
        if seq is not None:
            oracle.fwd_seq(xs, ws_, seq.numpy(), bs, act)
            if has_bwd:
                oracle.bwd_seq(xs, ws_, dy, seq.numpy(), bs, act)
        else:
            oracle.fwd(xs, ws_, bs, cun, init, act, return_final_states=True)
            if has_bwd:
                oracle.bwd(xs, ws_, dy, bs, cun, init, None, act)
        dt = time.perf_counter() - t0
        fin = w["return_final_states"]
        W = w["weight"].shape[1]
        bb = 4 if bs is not None and w["bias"].dtype.itemsize == 4 else 2
        nbytes = fwd_bytes(B, nch, T, R, init is not None, fin, wb, bs is not None, W, bb)
        if has_bwd:
            nbytes += bwd_bytes(B, nch, T, R, init is not None, False, wb, bs is not None, W, bb)
        return dt, nbytes

    pilot_dt, _ = run(min(D, 8))
    nch = int(min(D, max(8, budget_s / max(pilot_dt / min(D, 8), 1e-9))))
    dt, nbytes = run(nch)
    return dt, nbytes, nch, D, has_bwd


def cpu_baseline(wl, budget_s=10.0):
    """The fp64 oracle, single-threaded and pinned to one CPU, on a bounded
    sample of the same workload."""
    with _OneCore() as core:
        if wl.kind == "large_decode":
            dt1, b1, nch, D, _ = _oracle_rows(wl.large, budget_s)
            dt2, b2, steps, rows, Dd = _oracle_decode(wl.decode, budget_s / 2)
            dt, nbytes = dt1 + dt2, b1 + b2
            B, T = wl.large.shape["B"], wl.large.shape["T"]
            sample = ("fwd+bwd on channels 0..%d of %d (all %d rows x %d tokens), then %d decode "
                      "steps on all %d rows x %d channels" % (nch - 1, D, B, T, steps, rows, Dd))
            tc = B * nch * T + steps * rows * Dd
        elif wl.kind == "decode":
            dt, nbytes, steps, rows, D = _oracle_decode(wl, budget_s)
            sample = "%d decode steps on all %d rows x %d channels" % (steps, rows, D)
            tc = steps * rows * D
        elif wl.kind == "decode_tokens":
            dt, nbytes, calls, rows, D, L = _oracle_decode_tokens(wl, budget_s)
            sample = "%d calls of %d tokens on all %d rows x %d channels" % (calls, L, rows, D)
            tc = calls * L * rows * D
        else:
            dt, nbytes, nch, D, has_bwd = _oracle_rows(wl, budget_s)
            B, T = wl.shape["B"], wl.shape["T"]
            sample = "fwd%s on channels 0..%d of %d (all %d rows x %d tokens)" % (
                "+bwd" if has_bwd else "", nch - 1, D, B, T)
            tc = B * nch * T
    return dict(value=nbytes / dt / 1e9, unit="GB/s", cores=1, kind="oracle",
                sample=sample + ", one thread pinned to CPU %s" % core.cpu,
                seconds=round(dt, 3), token_channels_per_s=round(tc / dt, 1),
                host=host_cpu())


def _kernel_rows(csv_path):
    import csv
    rows = list(csv.DictReader(open(csv_path)))
    for r in rows:
        n = r.get("Kernel_Name") or r.get("Name")
        r["_short"] = n.replace("void ccv::(anonymous namespace)::", "").split("(ccv")[0]
    return rows


def _is_kernel(short, kernel):
    """Whether a kernel-trace name is `kernel` (any namespace, template
    arguments or parameter list)."""
    import re
    short = short.replace("(anonymous namespace)::", "")
    base = re.split(r"[<(]", short, maxsplit=1)[0].split("::")[-1].split(" ")[-1]
    return base == kernel


def _counter_per_launch(pmc_dir, counter, kernel=None, name_part=None):
    """Mean of a counter over the dispatches of `kernel` (or, for library
    kernels, of the names containing name_part)."""
    import glob
    vals = []
    for f in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in _kernel_rows(f):
            hit = _is_kernel(r["_short"], kernel) if kernel else name_part in r["_short"]
            if r["Counter_Name"] == counter and hit:
                vals.append(float(r["Counter_Value"]))
    return sum(vals) / len(vals) if vals else None, len(vals)


def summarize(args):
    """Write profiles/<kernel>_<workload>.md from rocprofv3 output directories
    (kernel trace, FETCH_SIZE pass, WRITE_SIZE pass, and the same two counters
    for a plain copy of known size)."""
    import glob
    wl_bytes = WORKLOAD_BYTES[
        args.workload[:-3] if args.workload.endswith("_tc") else args.workload]
    trace_dir, fetch_dir, write_dir, cfetch_dir, cwrite_dir = args.summarize
    stats = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)[0]
    rows = _kernel_rows(stats)
    copy_bytes = args.copy_calibration << 20
    c_fetch, _ = _counter_per_launch(cfetch_dir, "FETCH_SIZE", name_part="copyBuffer")
    c_write, _ = _counter_per_launch(cwrite_dir, "WRITE_SIZE", name_part="copyBuffer")
    f_scale = copy_bytes / (c_fetch * 1024.0)   # counter KiB -> bytes read
    w_scale = copy_bytes / (c_write * 1024.0)
    h = source_hash()
    for op, kernel in op_kernels(args.workload).items():
        if op not in wl_bytes:
            continue
        # the update op is whichever update kernel the workload's shape takes
        family = (UPDATE_KERNELS if kernel == "k_update" else (kernel,))
        kernels = [k for k in family if any(_is_kernel(r["_short"], k) for r in rows)]
        if not kernels:
            continue
        # An op of several launches counts all of them (time and traffic are
        # their sums per launch): the deterministic backward's fixed-order
        # reduction of its partials; on packed time lanes, the boundary repair
        # after the chunks, and the validation kernel before them when there
        # are too many offsets for the chunk waves to check.
        if kernel in ("k_fwd_tcp", "k_bwd_tcp"):
            kernels = ["k_validate", kernel, kernel + "_fix"]
        if op == "bwd":
            kernels.append("k_dw_reduce")
        kernels = [k for k in kernels if any(_is_kernel(r["_short"], k) for r in rows)]
        fetch = write = 0.0
        nf = nw = 0
        for k in kernels:
            f_, n_ = _counter_per_launch(fetch_dir, "FETCH_SIZE", kernel=k)
            w_, m_ = _counter_per_launch(write_dir, "WRITE_SIZE", kernel=k)
            fetch += f_
            write += w_
            nf, nw = nf + n_, nw + m_
        hbm = int(fetch * 1024 * f_scale + write * 1024 * w_scale)
        alg = wl_bytes[op]
        lines = ["# %s on the %s workload" % (kernel, args.workload), "",
                 "Commands (one MI355X, repository root as $REPO, `cd /tmp && export TMPDIR=/tmp` first):", "",
                 "```"]
        lines += args.commands.split(";;")
        lines += ["```", "", "Kernel trace (`--kernel-trace --stats`):", "",
                  "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
        for r in rows:
            lines.append("| `%s` | %s | %.2f | %.2f | %.2f |" % (
                r["_short"][:70], r["Calls"], float(r["AverageNs"]) / 1e3,
                float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
        avg_us = 0.0
        for k in kernels:
            ks = [r for r in rows if _is_kernel(r["_short"], k)]
            avg_us += sum(float(r["AverageNs"]) * int(r["Calls"]) for r in ks) / \
                sum(int(r["Calls"]) for r in ks) / 1e3
        lines += ["", "Counters per launch of `%s` (means over %d and %d dispatches):"
                  % (" + ".join(kernels), nf, nw), "",
                  "| quantity | value |", "|---|---|",
                  "| FETCH_SIZE (KiB) | %.1f |" % fetch, "| WRITE_SIZE (KiB) | %.1f |" % write,
                  "| copy calibration: %d MiB copy reads FETCH_SIZE KiB | %.1f (factor %.4f) |" % (
                      args.copy_calibration, c_fetch, f_scale),
                  "| copy calibration: %d MiB copy reads WRITE_SIZE KiB | %.1f (factor %.4f) |" % (
                      args.copy_calibration, c_write, w_scale),
                  "| HBM bytes per launch (scaled) | %d |" % hbm,
                  "| algorithmic bytes per launch | %d |" % alg,
                  "| traffic / algorithmic | %.4f |" % (hbm / alg),
                  "| average duration per launch of the op (us) | %.2f |" % avg_us,
                  "| algorithmic bytes / average duration (GB/s) | %.1f |" % (alg / (avg_us * 1e-6) / 1e9),
                  "",
                  "<!-- traffic " + json.dumps({"kernel": kernel, "kernels": kernels,
                                                 "workload": args.workload,
                                                 "hbm_bytes_per_launch": hbm,
                                                 "algorithmic_bytes": alg,
                                                 "avg_kernel_us": round(avg_us, 3),
                                                 "source_hash": h}) + " -->"]
        path = profile_path(kernel, args.workload)
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        print("wrote", path)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large_decode",
                    choices=WORKLOADS)
    ap.add_argument("--no-other-configs", action="store_true",
                    help="with large_decode: skip timing the dense and packed workloads' ops")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-events", action="store_true",
                    help="skip the per-op event pass")
    ap.add_argument("--op-reps", type=int, default=10,
                    help="back-to-back launches per event pair in the per-op pass")
    ap.add_argument("--no-warm-pass", action="store_true",
                    help="skip the warm per-op pass (same operands every launch)")
    ap.add_argument("--graph", dest="graph", action="store_true", default=True,
                    help="replay the step as a captured HIP graph in the timed region (default)")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="launch every op eagerly in the timed region")
    ap.add_argument("--no-cycle-graph", dest="cycle_graph", action="store_false", default=True,
                    help="replay one graph per step instead of one per rotation of R steps")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the workload, run a plain device copy of MIB MiB "
                         "(counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--summarize", nargs=5, metavar="DIR",
                    help="(no GPU) write profiles/<kernel>_<workload>.md from rocprofv3 output: "
                         "TRACE FETCH WRITE COPY_FETCH COPY_WRITE directories")
    ap.add_argument("--commands", default="", help="with --summarize: the commands run, ';;'-separated")
    args = ap.parse_args()
    if args.summarize:
        summarize(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the op shards over channels or batch rows with no communication, each "
              "GPU running the same kernels on its share)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from depthwise_causal_conv1d_02_amd import _abi
    _abi.lib()
    dev = torch.device("cuda", 0)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).random_()
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": 2 * n, "launches":
                          args.warmup + args.steps}))
        return

    print("bench: building workload %s" % args.workload, file=sys.stderr, flush=True)
    wl = Workload(args.workload, dev)
    # R copies of every operand; the timed steps and the cold per-op pass
    # rotate over them, so that no launch finds its operands in the 256 MB
    # memory-side cache (HBM-bound, "cold" timing).
    n_rot = rotation_count(wl)
    wls = [wl] + [wl.clone() for _ in range(n_rot - 1)]
    steps = [make_step(w, torch) for w in wls]
    quiet = Events(torch, False)
    for _ in range(args.warmup):
        for st in steps:
            st(quiet)
    torch.cuda.synchronize()

    graphs = cycle = None
    if args.graph:
        # Each copy's step captured once and replayed: no host launch latency
        # between kernels (HIP graphs under torch.cuda.CUDAGraph).  A second
        # graph holds one whole rotation (the R steps in order), so the timed
        # loop launches one graph per R steps and a host launch never stands
        # between two steps.
        graphs = []
        for st in steps:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                st(quiet)
            gr.replay()
            graphs.append(gr)
        if args.cycle_graph:
            cycle = torch.cuda.CUDAGraph()
            with torch.cuda.graph(cycle):
                for st in steps:
                    st(quiet)
            cycle.replay()
        torch.cuda.synchronize()

    # Timed region: exactly K steps between two synchronisations; step i runs
    # on operand copy i mod R.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while i < args.steps:
        if cycle is not None and i + n_rot <= args.steps:
            cycle.replay()          # steps i .. i+R-1 (i is a multiple of R here)
            i += n_rot
        elif graphs is not None:
            graphs[i % n_rot].replay()
            i += 1
        else:
            steps[i % n_rot](quiet)
            i += 1
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    check_flags(steps)
    ms = (t1 - t0) * 1e3 / args.steps
    step_bytes = wl.step_bytes()
    value = step_bytes / (ms * 1e-3) / 1e9
    print("bench: timed %d steps, %.4f ms/step (%s over %d operand copies)" % (
        args.steps, ms, "graph replay" if graphs is not None else "eager", n_rot),
        file=sys.stderr, flush=True)

    per_op = {}
    roof = None
    if not args.no_events:
        # Per-op times, on the stream the kernels run on, each from one event
        # pair around many back-to-back launches replayed from a HIP graph
        # after a GPU spin (the pair's own latency is spread over the
        # launches, as a kernel trace would not count it).  Cold: the
        # launches rotate over the operand copies (the headline, HBM-bound).
        # Warm: the same operands every launch, so the memory-side cache can
        # serve part of them (reported beside it).
        cold = rotated_op_times(torch, steps, wl, args.op_reps)
        warm = {} if args.no_warm_pass else op_times(torch, steps[0], wl, args.op_reps)
        for k, t in cold.items():
            per_op[k] = per_op_entry(wl, k, t, n_rot)
            if k in warm:
                wg = wl.bytes[k] / (warm[k] * 1e-3) / 1e9
                per_op[k].update(warm_ms=round(warm[k], 5), warm_GB_s=round(wg, 1),
                                 warm_pct_of_peak=round(100 * wg / PEAK_HBM_GBS, 2))
        check_flags(steps)
        dom = max(cold, key=lambda k: cold[k] * wl.counts[k])
        kernel = op_kernel_label(wl, dom)
        ach = wl.bytes[dom] / (cold[dom] * 1e-3) / 1e9
        rec = recorded_traffic(op_kernels(wl.name)[dom], profile_workload(wl.name, dom))
        roof = {"bound": "hbm", "kernel": kernel, "op": dom, "achieved": round(ach, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                "traffic": None if rec is None else rec["hbm_bytes_per_launch"],
                "bytes_per_launch": wl.bytes[dom], "avg_launch_ms": round(cold[dom], 5),
                "timing": "cold: back-to-back launches rotating over %d operand copies" % n_rot}
        if rec is not None:
            roof["traffic_over_algorithmic"] = round(rec["hbm_bytes_per_launch"] / wl.bytes[dom], 4)
        if dom in warm:
            ach_w = wl.bytes[dom] / (warm[dom] * 1e-3) / 1e9
            roof.update(achieved_warm=round(ach_w, 1), frac_warm=round(ach_w / PEAK_HBM_GBS, 4),
                        avg_launch_ms_warm=round(warm[dom], 5))

    shape = wl.shape
    tc = wl.token_channels()
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.desc, "io_dtype": "bf16", **shape,
                   "ops_per_step": wl.counts, "step_algorithmic_bytes": step_bytes,
                   "timing": ("graph replay, one graph per %d steps" % n_rot if cycle is not None
                              else "graph replay, one graph per step" if graphs is not None
                              else "eager launches") +
                             " rotating over %d operand copies (cold caches)" % n_rot},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "token_channels_per_s": round(tc / (ms * 1e-3), 1),
        "ops": per_op, "roofline": roof,
    }
    if wl.kind == "large_decode" and not args.no_events and not args.no_other_configs:
        # the large workload's operands and graphs are released first, so the
        # smaller workloads are timed on a device holding only their own data
        cpu_wl = wl.cpu_view()
        del graphs, cycle, steps, wls, wl
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        out["other_configs"] = other_config_ops(torch, dev, ("dense", "packed"), args.op_reps,
                                                args.warmup + args.steps)
        wl = cpu_wl
    if not args.no_cpu_baseline:
        print("bench: timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
