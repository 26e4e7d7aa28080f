#!/usr/bin/env python3
"""Achieved HBM GB/s of the depthwise causal conv1d (fwd, bwd, update) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dense|packed|decode|large|tiny]

One step is one pass of the whole hot path over one batch of seeded synthetic
input already resident in HBM:

  dense  (default)  B=4 D=4096 T=2048, [B,T,D] storage behind a transpose view,
                    BF16 weight + bias, initial states, SiLU:
                    forward (returns final states) + backward (FP32 atomics,
                    dinit) + one decode update from the final states.
  packed            16 sequences, T=33,280, D=5120, FP32 weight, no bias,
                    initial states: forward + backward.
  decode            B=256 D=8192 single-token update; a step is one token
                    (the 64 seeded tokens are cycled).
  large             B=8 D=8192 T=8192, no bias: forward + deterministic backward.
  tiny              B=1 D=64 T=128 [B,D,T]: forward (launch-bound).

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
METRIC = "achieved HBM GB/s (% of MI355X peak) for fwd, bwd and update at 1 GPU"


def act_bytes(B, D, T):
    return B * D * T * 2


def fwd_bytes(B, D, T, R, init, final, w_bytes, bias):
    return (2 * act_bytes(B, D, T) + (R * D * 6 if init else 0) + (R * D * 6 if final else 0)
            + D * 4 * w_bytes + (D * 2 if bias else 0))


def bwd_bytes(B, D, T, R, init, dfinal, w_bytes, bias):
    return (3 * act_bytes(B, D, T) + (2 * R * D * 6 if init else 0) + (R * D * 6 if dfinal else 0)
            + D * 4 * w_bytes + D * 4 * 4 + ((D * 2 + D * 4) if bias else 0))


def update_bytes(B, D, w_bytes, bias):
    return B * D * 16 + D * 4 * w_bytes + (D * 2 if bias else 0)


class Workload:
    """Device tensors of one named workload and its per-op byte counts."""

    def __init__(self, name, dev):
        import torch
        from depthwise_causal_conv1d_02_amd import synth

        self.name, self.dev = name, dev
        to = lambda t: None if t is None else t.to(dev)
        idx = {"tiny": 1, "dense": 2, "packed": 3, "decode": 4, "large": 5}[name]
        self.cpu = synth.workload(idx)
        w = self.cpu
        self.g = {k: to(v) if isinstance(v, torch.Tensor) else v for k, v in w.items()}
        self.ops = []
        if name == "decode":
            B, D = w["conv_state"].shape[:2]
            self.shape = dict(B=B, D=D)
            self.bytes = {"update": update_bytes(B, D, 2, True)}
            self.desc = ("decode update: B=%d D=%d, one token per step (64 seeded tokens), "
                         "bf16 weight+bias, SiLU, state mutated in place" % (B, D))
            return
        x = w["x"]
        B, D, T = x.shape
        cu = w["cu_seqlens"]
        R = B if cu is None else cu.numel() - 1
        wb = 4 if w["weight"].dtype == torch.float32 else 2
        bias = w["bias"] is not None
        init = w["initial_states"] is not None
        self.shape = dict(B=B, D=D, T=T, R=R)
        self.bytes = {"fwd": fwd_bytes(B, D, T, R, init, w["return_final_states"], wb, bias)}
        if w["dy"] is not None:
            self.bytes["bwd"] = bwd_bytes(B, D, T, R, init, False, wb, bias)
        if name == "dense":
            self.bytes["update"] = update_bytes(B, D, 2, bias)
        self.desc = synth.WORKLOADS[idx]


def make_step(wl, torch):
    """Allocate every output once; return step() running all ops of one pass."""
    from depthwise_causal_conv1d_02_amd import ops

    g, dev = wl.g, wl.dev
    if wl.name == "decode":
        state = g["conv_state"].clone()
        y = torch.empty_like(g["x_steps"][0])
        n = [0]

        def step(ev):
            xt = g["x_steps"][n[0] % g["x_steps"].shape[0]]
            n[0] += 1
            ev.begin("update")
            ops.update(xt, state, g["weight"], g["bias"], g["activation"], y=y)
            ev.end("update")
        return step

    x = g["x"]
    y = torch.empty_like(x)
    fin = None
    if g["return_final_states"] or wl.name == "dense":
        fin = torch.empty(wl.shape["R"], x.shape[1], 3, dtype=x.dtype, device=dev)
    has_bwd = g["dy"] is not None
    if has_bwd:
        dx = torch.empty_like(x)
        dw = torch.zeros(x.shape[1], 4, dtype=torch.float32, device=dev)
        db = torch.zeros(x.shape[1], dtype=torch.float32, device=dev) if g["bias"] is not None else None
        dinit = torch.empty_like(g["initial_states"]) if g["initial_states"] is not None else None
        ws = torch.empty(1 << 26, dtype=torch.uint8, device=dev) if g["deterministic"] else None
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    if wl.name == "dense":
        state = torch.empty_like(fin)
        xt = g["x"][:, :, -1].contiguous()
        yt = torch.empty_like(xt)

    def step(ev):
        ev.begin("fwd")
        ops.fwd(x, g["weight"], g["bias"], g["cu_seqlens"], g["initial_states"], g["activation"],
                final_states_out=fin, y=y, err_flag=flag)
        ev.end("fwd")
        if has_bwd:
            dw.zero_()
            if db is not None:
                db.zero_()
            ev.begin("bwd")
            ops.bwd(x, g["weight"], g["dy"], g["bias"], g["cu_seqlens"], g["initial_states"], None,
                    g["activation"], g["deterministic"], False, dx=dx, err_flag=flag,
                    workspace=ws, dweight=dw, dbias=db, dinit=dinit)
            ev.end("bwd")
        if wl.name == "dense":
            state.copy_(fin)
            ev.begin("update")
            ops.update(xt, state, g["weight"], g["bias"], g["activation"], y=yt)
            ev.end("update")
    return step


class Events:
    """HIP events around each op on the current stream (the one the kernels use)."""

    def __init__(self, torch, on):
        self.torch, self.on = torch, on
        self.rec = {}
        self.open = {}

    def begin(self, name):
        if self.on:
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


def cpu_baseline(wl, budget_s=10.0):
    """The fp64 oracle, single-threaded, on a channel sample of the same workload."""
    import oracle

    w = wl.cpu
    f = lambda t: None if t is None else t.double().numpy()
    if wl.name == "decode":
        B, D = w["conv_state"].shape[:2]
        nb = 16
        st = f(w["conv_state"][:nb])
        t0 = time.perf_counter()
        steps = 0
        while steps < 64 and time.perf_counter() - t0 < budget_s:
            _, st = oracle.update(f(w["x_steps"][steps][:nb]), st, f(w["weight"]), f(w["bias"]),
                                  "silu")
            steps += 1
        dt = time.perf_counter() - t0
        nbytes = steps * update_bytes(nb, D, 2, True)
        return dict(value=nbytes / dt / 1e9, unit="GB/s", cores=1, kind="oracle",
                    sample="%d decode steps on %d of %d batch rows (all %d channels)"
                           % (steps, nb, B, D),
                    seconds=dt, token_channels_per_s=steps * nb * D / dt)
    x = w["x"]
    B, D, T = x.shape
    cu = w["cu_seqlens"]
    cun = None if cu is None else cu.numpy()
    R = wl.shape["R"]
    wb = 4 if w["weight"].dtype.itemsize == 4 else 2
    has_bwd = w["dy"] is not None

    # Channels are independent, so a block of channels over every row and
    # token is the same workload, narrower.  A short pilot sizes the sample
    # to about `budget_s` seconds of oracle time.
    def run(nch):
        sub = lambda t: None if t is None else f(t[:, :nch] if t.dim() == 3 else t[:nch])
        xs, ws_, bs = sub(x), sub(w["weight"]), sub(w["bias"])
        init, dy = sub(w["initial_states"]), sub(w["dy"])
        t0 = time.perf_counter()
        oracle.fwd(xs, ws_, bs, cun, init, "silu", return_final_states=True)
        if has_bwd:
            oracle.bwd(xs, ws_, dy, bs, cun, init, None, "silu")
        dt = time.perf_counter() - t0
        nbytes = fwd_bytes(B, nch, T, R, init is not None, True, wb, bs is not None)
        if has_bwd:
            nbytes += bwd_bytes(B, nch, T, R, init is not None, False, wb, bs is not None)
        return dt, nbytes

    pilot_dt, _ = run(min(D, 8))
    nch = int(min(D, max(8, budget_s / max(pilot_dt / min(D, 8), 1e-9))))
    dt, nbytes = run(nch)
    return dict(value=nbytes / dt / 1e9, unit="GB/s", cores=1, kind="oracle",
                sample="fwd%s on channels 0..%d of %d (all %d rows x %d tokens), one thread"
                       % ("+bwd" if has_bwd else "", nch - 1, D, B, T),
                seconds=round(dt, 3), token_channels_per_s=round(B * nch * T / dt, 1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dense",
                    choices=["dense", "packed", "decode", "large", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-events", action="store_true",
                    help="time the steps without per-op events")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the workload, run a plain device copy of MIB MiB "
                         "(counter calibration for rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the op shards with no communication over channels; see the design notes)",
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
    step = make_step(wl, torch)
    warm = Events(torch, False)
    for _ in range(args.warmup):
        step(warm)
    ev = Events(torch, not args.no_events)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(ev)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    step_bytes = sum(wl.bytes.values())
    value = step_bytes / (ms * 1e-3) / 1e9
    print("bench: timed %d steps, %.4f ms/step" % (args.steps, ms), file=sys.stderr, flush=True)

    per_op = {}
    roof = None
    if not args.no_events:
        means = ev.mean_ms()
        for k, t in means.items():
            gbs = wl.bytes[k] / (t * 1e-3) / 1e9
            per_op[k] = {"ms": round(t, 5), "algorithmic_bytes": wl.bytes[k],
                         "GB_s": round(gbs, 1), "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2)}
        dom = max(means, key=lambda k: means[k])
        kernel = {"fwd": "k_fwd_chan", "bwd": "k_bwd_chan", "update": "k_update"}[dom]
        ach = wl.bytes[dom] / (means[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": kernel, "op": dom, "achieved": round(ach, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                "traffic": None, "bytes_per_launch": wl.bytes[dom],
                "avg_launch_ms": round(means[dom], 5)}

    shape = wl.shape
    tc = shape["B"] * shape["D"] * shape.get("T", 1)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.desc, "io_dtype": "bf16", **shape,
                   "ops_per_step": list(wl.bytes), "step_algorithmic_bytes": step_bytes},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "token_channels_per_s": round(tc / (ms * 1e-3), 1),
        "ops": per_op, "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print("bench: timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
