"""Pins of the CPU oracle's elementwise pieces: bf16 rounding, RMSNorm and the
fp32-specified router sigmoid.  Each check uses something other than the oracle
itself: a library routine (torch, scipy), a closed form or exact constants."""
import math

import numpy as np
import pytest
import torch
from scipy.special import expit

from oracle import moe_oracle as o

F32 = np.float32


def test_bf16_round_matches_torch_conversion():
    rng = np.random.default_rng(1)
    a = np.concatenate([
        rng.standard_normal(200_000).astype(F32) * F32(3.0),
        rng.standard_normal(1000).astype(F32) * F32(1e-30),
        rng.standard_normal(1000).astype(F32) * F32(1e30),
    ])
    # exact ties: bf16 value plus half a bf16 ulp
    base = torch.from_numpy(a[:1000]).to(torch.bfloat16).float().numpy()
    ties = (base.astype(np.float64) + np.spacing(base.astype(F32)).astype(np.float64) * 2 ** 15).astype(F32)
    a = np.concatenate([a, ties])
    want = torch.from_numpy(a).to(torch.bfloat16).double().numpy()
    got = o.bf16_round(a)
    np.testing.assert_array_equal(got, want)


def test_bf16_round_ties_to_even():
    one = 1.0
    assert o.bf16_round(one + 2 ** -8) == 1.0                  # mantissa 0 is even
    assert o.bf16_round(one + 3 * 2 ** -8) == 1.0 + 2 ** -6    # 1+2^-7 is odd -> up
    assert o.bf16_round(-(one + 2 ** -8)) == -1.0
    assert o.bf16_round(one + 2 ** -8 + 2 ** -20) == 1.0 + 2 ** -7


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 96))
    g = rng.standard_normal(96)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(o.rmsnorm(x, g, 1e-6), want, rtol=1e-13, atol=1e-13)


def test_rmsnorm_constant_row_closed_form():
    # x = c * ones  ->  h = gamma * c / sqrt(c^2 + eps)
    g = np.linspace(0.5, 2.0, 16)
    for c in (-3.0, 0.25, 7.0):
        h = o.rmsnorm(np.full((1, 16), c), g, 1e-6)
        np.testing.assert_allclose(h[0], g * c / math.sqrt(c * c + 1e-6), rtol=1e-14)


def test_rmsnorm_scale_invariance():
    """RMSNorm output does not depend on the input scale (up to eps): the
    demo's 'scaling compensation before RMSNorm' (Tab 5) is the identity."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((8, 128))
    g = np.ones(128)
    for alpha in (0.5, 4.0, 1e3):
        np.testing.assert_allclose(o.rmsnorm(alpha * x, g, 1e-6), o.rmsnorm(x, g, 1e-6), rtol=1e-5)


def test_sigmoid_constants_from_math():
    ln2 = math.log(2.0)
    assert o.LOG2E == F32(1.0 / ln2)
    hi = float(o.LN2_HI)
    # at most 16 significant bits, and below ln 2
    assert hi * 2 ** 16 == int(hi * 2 ** 16) and hi < ln2
    assert abs(hi + float(o.LN2_LO) - ln2) < 2 ** -40
    # n * LN2_HI is exact for every n the clamp allows (|n| <= 44)
    for n in range(-44, 45):
        assert float(F32(n) * o.LN2_HI) == n * hi
    assert [float(t) for t in o._TAYLOR] == [float(F32(1.0 / math.factorial(i))) for i in range(8)]


def _ulp_err(s, x):
    ref = expit(x.astype(np.float64))
    return np.abs(s.astype(np.float64) - ref) / np.spacing(s.astype(F32)).astype(np.float64)


def test_sigmoid_r_accuracy_sweep():
    """Error against the fp64 logistic function (scipy.special.expit).

    Measured on this sweep: max 2.46 ulp, mean 0.367 ulp.  The bounds are set
    so that dropping the degree-7 term (max 3.38, mean 0.402), flipping the
    sign of the low part of ln 2, or truncating instead of rounding n fails."""
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.uniform(-30, 30, 4_000_000).astype(F32),
        np.linspace(-1, 1, 2_000_001).astype(F32),
        rng.standard_normal(2_000_000).astype(F32) * F32(3.0),
    ])
    e = _ulp_err(o.sigmoid_r(x), x)
    assert e.max() <= 3.0
    assert e.mean() <= 0.385


def test_sigmoid_r_special_values():
    assert o.sigmoid_r(np.array([0.0], F32))[0] == F32(0.5)
    big = o.sigmoid_r(np.array([30.0, 31.0, 1e6, -30.0, -1e6], F32))
    assert big[0] == big[1] == big[2] == F32(1.0)
    assert big[3] == big[4]
    assert abs(float(big[3]) - math.exp(-30.0)) / math.exp(-30.0) < 1e-6
    x = np.linspace(-8, 8, 1001).astype(F32)
    s = o.sigmoid_r(x).astype(np.float64)
    assert np.all(np.diff(s) >= 0)                      # monotone
    np.testing.assert_allclose(s + s[::-1], 1.0, atol=2e-7)  # sigma(-x) = 1 - sigma(x)
