"""The seeded input recipe reproduces the packed workload's lengths."""
import torch

from depthwise_causal_conv1d_02_amd import synth


def test_packed_lengths_rule():
    seed, lens = synth.packed_lengths()
    assert seed == 4
    assert lens == [742, 732, 1021, 3741, 4008, 2506, 2232, 372, 1896, 182, 3277, 511, 1182,
                    3773, 3892, 3213]
    cu = synth.cu_from_lengths(lens)
    assert cu.dtype == torch.int32 and int(cu[-1]) == 33280 and cu.numel() == 17


def test_channel_last_is_transpose_view():
    inp = synth.random_inputs(0, 2, 16, 5, layout="cl")
    x = inp["x"]
    assert x.shape == (2, 16, 5) and x.stride() == (80, 1, 16)
    assert x.dtype == torch.bfloat16


def test_seeded_reproducible():
    a = synth.random_inputs(3, 1, 8, 4, layout="tc", init=True)
    b = synth.random_inputs(3, 1, 8, 4, layout="tc", init=True)
    for k in ("x", "weight", "bias", "initial_states", "dy"):
        assert torch.equal(a[k], b[k])
