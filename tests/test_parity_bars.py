"""The parity bars the GPU tests apply (tests/parity.py), checked on the CPU:
1e-2 on O everywhere for fp32 outputs and below |O| = 4 for bf16 outputs, one
bf16 ulp at and beyond 4, 1e-3 on lse."""
import numpy as np
import pytest

import parity


def test_o_bar_values():
    ref = np.array([0.0, 0.3, -1.99, 3.999, 4.0, -5.5, 8.0, 100.0])
    fp32 = parity.o_tolerance(ref, bf16_out=False)
    assert np.all(fp32 == 1e-2)
    bf = parity.o_tolerance(ref, bf16_out=True)
    assert np.all(bf[:4] == 1e-2)
    # one ulp of an 8-significant-bit number: 2^(e - 7)
    assert list(bf[4:]) == [2.0 ** -5, 2.0 ** -5, 2.0 ** -4, 2.0 ** -1]


def test_bf16_rounding_alone_fits_the_bar_beyond_four():
    """Beyond |O| = 4 rounding to nearest moves a value by at most half an ulp,
    so a correctly rounded result always passes; below 4 the bar stays 1e-2."""
    g = np.random.default_rng(0)
    x = g.uniform(4.0, 64.0, 10000) * g.choice([-1, 1], 10000)
    import torch
    r = torch.from_numpy(x.astype(np.float32)).bfloat16().float().numpy().astype(np.float64)
    assert np.all(np.abs(r - x) <= parity.o_tolerance(x, True))


def test_check_o_flags_an_error_just_over_the_bar():
    ref = np.zeros((2, 512))
    ref[1, 7] = 5.0
    ok = ref.copy()
    ok[0, 3] += 0.0099
    ok[1, 7] += 2.0 ** -5
    parity.check_o(ok, ref, bf16_out=True)
    bad = ref.copy()
    bad[0, 3] += 0.0101
    with pytest.raises(AssertionError):
        parity.check_o(bad, ref, bf16_out=True)
    bad = ref.copy()
    bad[1, 7] += 2.0 ** -5 + 1e-6
    with pytest.raises(AssertionError):
        parity.check_o(bad, ref, bf16_out=True)
    with pytest.raises(AssertionError):
        parity.check_o(ok, ref, bf16_out=False)  # fp32 outputs: 1e-2 at 5 too


def test_lse_bar():
    ref = np.array([1.0, -np.inf, 3.0])
    parity.check_lse(np.array([1.0009, -np.inf, 3.0]), ref)
    with pytest.raises(AssertionError):
        parity.check_lse(np.array([1.0011, -np.inf, 3.0]), ref)
    with pytest.raises(AssertionError):
        parity.check_lse(np.array([1.0, 0.0, 3.0]), ref)
