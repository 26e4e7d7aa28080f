"""The comparison helpers themselves (CPU): exact BF16 rounding and the
one-step ordering used by the GPU parity tests."""
import numpy as np
import torch

from parity import bf16_bits, bf16_ord, bf16_rne, check_bf16


def test_bf16_rne_matches_single_rounding_from_float32():
    g = torch.Generator().manual_seed(0)
    f = torch.randn(200000, generator=g, dtype=torch.float32) * 3
    f = torch.cat([f, torch.tensor([1.00390625, 1.01171875, -1.00390625, 0.0, -0.0,
                                    1e-40, 3.0e38, -3.3e38])])
    want = f.to(torch.bfloat16).double().numpy()   # float32 -> bf16 is one RNE rounding
    got = bf16_rne(f.double().numpy())
    assert np.array_equal(got, want)


def test_bf16_rne_ties_from_double():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins (1.0);
    # 1 + 2^-8 + 2^-40 is above the tie and rounds up -- a float32 detour
    # would lose the 2^-40 and round down.
    assert bf16_rne([1 + 2 ** -8])[0] == 1.0
    assert bf16_rne([1 + 2 ** -8 + 2 ** -40])[0] == 1 + 2 ** -7
    assert bf16_rne([1 + 3 * 2 ** -8])[0] == 1 + 2 ** -6


def test_ordering_and_tolerance():
    t = torch.tensor([1.0, -1.0, 0.0, -0.0], dtype=torch.bfloat16)
    o = bf16_ord(bf16_bits(t))
    assert o[2] == o[3] == 0 and o[0] > 0 > o[1]
    g = torch.tensor([1.0 + 2 ** -7], dtype=torch.bfloat16)   # one step above 1.0
    check_bf16("one step", g, np.array([1.0]))
    g2 = torch.tensor([1.0 + 2 ** -6], dtype=torch.bfloat16)  # two steps
    try:
        check_bf16("two steps", g2, np.array([1.0]))
        raise RuntimeError("should have failed")
    except AssertionError:
        pass
    # near zero the absolute escape applies
    check_bf16("abs", torch.tensor([5e-4], dtype=torch.bfloat16), np.array([-4e-4]))
