"""Seeded synthetic inputs for the depthwise causal conv1d.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic.  The tests (for both the GPU path and the CPU oracle)
and the benchmark use it so that both sides see the same inputs.

Recipe (shapes and distributions of the Mamba-style mixer workloads):

* one ``torch.Generator`` on the CPU, ``manual_seed(seed)``; tensors drawn in
  the order they are listed; each drawn in float32 and rounded to bfloat16
  (round to nearest even) unless stated otherwise;
* N(0,1): ``randn``;  U(-0.5,0.5): ``rand - 0.5``;  bias: ``randn * 0.1``
  (a standard deviation of 0.1);
* "channel-last" inputs are drawn as ``[B,T,D]`` storage and exposed as the
  ``[B,D,T]`` view ``storage.transpose(1, 2)``, which is how a model that owns
  ``[B,T,D]`` storage hands them over (cuDNN FE "Causal Conv1d", the paragraph
  on transpose views).
"""
import torch

BF16 = torch.bfloat16


def _normal(g, shape, scale=1.0):
    t = torch.randn(*shape, generator=g, dtype=torch.float32)
    if scale != 1.0:
        t = t * scale
    return t.to(BF16)


def _uniform_half(g, shape, dtype=BF16):
    return (torch.rand(*shape, generator=g, dtype=torch.float32) - 0.5).to(dtype)


def activation_tensor(g, B, D, T, layout):
    """x or dy: [B,D,T] logical view; layout 'cl' draws [B,T,D] storage."""
    if layout == "cl":
        return _normal(g, (B, T, D)).transpose(1, 2)
    if layout == "tc":
        return _normal(g, (B, D, T))
    raise ValueError(layout)


def weight_tensor(g, D, W=4, dtype=BF16):
    return _uniform_half(g, (D, W), dtype)


def bias_tensor(g, D, dtype=BF16):
    """randn * 0.1, rounded to BF16, or kept in FP32 for an FP32 filter."""
    t = torch.randn(D, generator=g, dtype=torch.float32) * 0.1
    return t.to(dtype)


def state_tensor(g, R, D, W=4):
    return _normal(g, (R, D, W - 1))


def packed_lengths(n_seq=16, lo=64, hi=4096, target=None, tol=0.01):
    """Sequence lengths ~U[lo, hi] from a generator of their own.

    The seed is the smallest one whose total lies within ``tol`` of the
    expected total ``n_seq * (lo + hi) / 2`` (33,280 for 16 x U[64,4096]).
    Returns (seed, lengths list).
    """
    if target is None:
        target = n_seq * (lo + hi) / 2.0
    seed = 0
    while True:
        g = torch.Generator().manual_seed(seed)
        lens = torch.randint(lo, hi + 1, (n_seq,), generator=g)
        if abs(int(lens.sum()) - target) <= tol * target:
            return seed, [int(v) for v in lens]
        seed += 1


def seq_idx_tensor(g, B, T, kind="runs", max_run=64, n_ids=3, min_run=1):
    """seq_idx [B,T] int32 ids: 'runs' = contiguous runs of U[min_run, max_run]
    tokens with increasing ids (packed sequences), 'random' = iid ids from
    {0..n_ids-1} (ids recur inside the window), 'periodic' = t mod n_ids,
    'constant' = 0."""
    if kind == "runs":
        rows = []
        for _ in range(B):
            ids, cur = [], 0
            while len(ids) < T:
                n = int(torch.randint(min_run, max_run + 1, (1,), generator=g))
                ids.extend([cur] * n)
                cur += 1
            rows.append(ids[:T])
        return torch.tensor(rows, dtype=torch.int32)
    if kind == "random":
        return torch.randint(0, n_ids, (B, T), generator=g, dtype=torch.int32)
    if kind == "periodic":
        return (torch.arange(T, dtype=torch.int32) % n_ids).repeat(B, 1)
    if kind == "constant":
        return torch.zeros(B, T, dtype=torch.int32)
    raise ValueError(kind)


def cu_from_lengths(lengths):
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def random_inputs(seed, B, D, T, *, layout="cl", W=4, bias=True, init=False, dy=True,
                  dfinal=False, weight_dtype=BF16, cu_seqlens=None):
    """General seeded inputs for parity tests (CPU tensors).

    Draw order: x, weight, bias, initial_states, dy, dfinal_states.
    With ``cu_seqlens`` (B must be 1) the states have N = len(cu)-1 rows.
    The bias takes the weight's dtype.
    """
    g = torch.Generator().manual_seed(seed)
    R = B if cu_seqlens is None else int(cu_seqlens.numel()) - 1
    out = {"x": activation_tensor(g, B, D, T, layout)}
    out["weight"] = weight_tensor(g, D, W, weight_dtype)
    out["bias"] = bias_tensor(g, D, weight_dtype) if bias else None
    out["initial_states"] = state_tensor(g, R, D, W) if init else None
    out["dy"] = activation_tensor(g, B, D, T, layout) if dy else None
    out["dfinal_states"] = state_tensor(g, R, D, W) if dfinal else None
    out["cu_seqlens"] = cu_seqlens
    return out


# ---- the five named workloads ---------------------------------------------

WORKLOADS = {
    1: "tiny dense fwd: B=1 D=64 T=128, [B,D,T] contiguous, bf16 weight+bias, SiLU, "
       "no initial state, final_states returned",
    2: "dense fwd+bwd with state: B=4 D=4096 T=2048, channel-last, bf16 weight+bias, "
       "initial_states, SiLU, final_states returned",
    3: "packed varlen fwd+bwd: N=16 U[64,4096] lengths (T=33280), D=5120, channel-last, "
       "fp32 weight, no bias, initial_states, SiLU",
    4: "decode update: B=256 D=8192, 64 single-token steps, bf16 weight+bias, SiLU",
    5: "large dense fwd+bwd: B=8 D=8192 T=8192, channel-last, bf16 weight, no bias, SiLU, "
       "deterministic dweight",
    6: "seq_idx fwd+bwd: B=4 D=4096 T=2048, channel-last, bf16 weight+bias, SiLU, each row "
       "packs sequences of U[64,1024] tokens marked by seq_idx (no states)",
}


def workload(idx):
    """Inputs of workload ``idx`` (1..6) as CPU tensors, seed = idx."""
    g = torch.Generator().manual_seed(idx)
    if idx == 1:
        B, D, T = 1, 64, 128
        return dict(x=activation_tensor(g, B, D, T, "tc"), weight=weight_tensor(g, D),
                    bias=bias_tensor(g, D), initial_states=None, dy=None, cu_seqlens=None,
                    activation="silu", return_final_states=True, deterministic=False)
    if idx == 2:
        B, D, T = 4, 4096, 2048
        return dict(x=activation_tensor(g, B, D, T, "cl"), weight=weight_tensor(g, D),
                    bias=bias_tensor(g, D), initial_states=state_tensor(g, B, D),
                    dy=activation_tensor(g, B, D, T, "cl"), cu_seqlens=None,
                    activation="silu", return_final_states=True, deterministic=False)
    if idx == 3:
        _, lens = packed_lengths()
        cu = cu_from_lengths(lens)
        D, T = 5120, int(cu[-1])
        N = len(lens)
        return dict(x=activation_tensor(g, 1, D, T, "cl"),
                    weight=weight_tensor(g, D, dtype=torch.float32), bias=None,
                    initial_states=state_tensor(g, N, D), dy=activation_tensor(g, 1, D, T, "cl"),
                    cu_seqlens=cu, activation="silu", return_final_states=True,
                    deterministic=False)
    if idx == 4:
        B, D, steps = 256, 8192, 64
        return dict(conv_state=_normal(g, (B, D, 3)), x_steps=_normal(g, (steps, B, D)),
                    weight=weight_tensor(g, D), bias=bias_tensor(g, D), activation="silu")
    if idx == 5:
        B, D, T = 8, 8192, 8192
        return dict(x=activation_tensor(g, B, D, T, "cl"), weight=weight_tensor(g, D),
                    bias=None, initial_states=None, dy=activation_tensor(g, B, D, T, "cl"),
                    cu_seqlens=None, activation="silu", return_final_states=False,
                    deterministic=True)
    if idx == 6:
        B, D, T = 4, 4096, 2048
        x = activation_tensor(g, B, D, T, "cl")
        weight, bias = weight_tensor(g, D), bias_tensor(g, D)
        dy = activation_tensor(g, B, D, T, "cl")
        return dict(x=x, weight=weight, bias=bias, initial_states=None, dy=dy, cu_seqlens=None,
                    seq_idx=seq_idx_tensor(g, B, T, "runs", max_run=1024, min_run=64),
                    activation="silu", return_final_states=False, deterministic=False)
    raise ValueError("workload index must be 1..6")


# ---- variants of the dense and decode workloads (the optional features) -----

VARIANTS = {
    "dense_w2": "dense fwd+bwd with state, filter width 2: B=4 D=4096 T=2048, channel-last, "
                "bf16 weight+bias, initial_states [B,D,1], SiLU, final_states returned",
    "dense_w3": "dense fwd+bwd with state, filter width 3: B=4 D=4096 T=2048, channel-last, "
                "bf16 weight+bias, initial_states [B,D,2], SiLU, final_states returned",
    "dense_noact": "dense fwd+bwd with state, no activation: B=4 D=4096 T=2048, channel-last, "
                   "bf16 weight+bias, initial_states, final_states returned",
    "dense_f32bias": "dense fwd+bwd with state, fp32 weight + fp32 bias (opt-in): B=4 D=4096 "
                     "T=2048, channel-last, initial_states, SiLU, final_states returned, "
                     "deterministic dweight and dbias (opt-in)",
    "dense_odd": "dense fwd+bwd with state, an odd length: B=4 D=4096 T=2047, channel-last, "
                 "bf16 weight+bias, initial_states, SiLU, final_states returned",
    "decode_tokens": "multi-token decode update: B=256 D=8192, 64 tokens as 8 calls of 8 "
                     "tokens ([B,D,8] over [B,8,D] storage), bf16 weight+bias, SiLU, state "
                     "mutated in place",
}


def variant(name):
    """Inputs of variant ``name`` (a key of VARIANTS) as CPU tensors; the seed
    is 100 + the variant's position in VARIANTS."""
    g = torch.Generator().manual_seed(100 + list(VARIANTS).index(name))
    if name == "decode_tokens":
        B, D, L, calls = 256, 8192, 8, 8
        return dict(conv_state=_normal(g, (B, D, 3)),
                    x_calls=_normal(g, (calls, B, L, D)).transpose(2, 3),
                    weight=weight_tensor(g, D), bias=bias_tensor(g, D), activation="silu")
    B, D, T = 4, 4096, 2047 if name == "dense_odd" else 2048
    W = {"dense_w2": 2, "dense_w3": 3}.get(name, 4)
    f32 = name == "dense_f32bias"
    dt = torch.float32 if f32 else BF16
    return dict(x=activation_tensor(g, B, D, T, "cl"), weight=weight_tensor(g, D, W, dt),
                bias=bias_tensor(g, D, dt), initial_states=state_tensor(g, B, D, W),
                dy=activation_tensor(g, B, D, T, "cl"), cu_seqlens=None,
                activation=None if name == "dense_noact" else "silu",
                return_final_states=True, deterministic=f32,
                fp32_weight_bias=f32, deterministic_dbias=f32)
