"""Pins of the oracle's MXFP8 rounding (low-precision experts).

E4M3 element rounding is checked against torch's own float8_e4m3fn
conversion (an independent implementation) over every representable
neighbourhood, ties included; saturation, the E8M0 block scale and the
round-trip error bound against their closed forms; the MXFP8 expert path
against the bf16 one where MXFP8 is exact."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as o
from sparse_moe_layer_rmsnorm_amd import workloads as wl

F32 = np.float32


def _all_e4m3():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    return np.unique(b[np.isfinite(b)].astype(np.float64))


def test_e4m3_round_matches_torch_below_saturation():
    vals = _all_e4m3()
    assert vals.max() == 448.0 and len(vals) == 253          # 126 magnitudes each sign, one zero
    mids = (vals[1:] + vals[:-1]) / 2                         # exact ties
    rng = np.random.default_rng(0)
    rand = rng.uniform(-460, 460, 20000) * np.exp2(rng.integers(-14, 1, 20000))
    x = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9), rand])
    x = x[np.abs(x) < 464].astype(np.float32)                 # torch turns |x| >= 480 into NaN
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(o.e4m3_round(x.astype(np.float64)), want)


def test_e4m3_saturates():
    x = np.array([464.0, 470.0, 480.0, 511.9, 1e6, -464.0, -1e9])
    np.testing.assert_array_equal(o.e4m3_round(x), np.sign(x) * 448.0)


def test_mx_scale_closed_form():
    """Block scale 2^(floor(log2 amax) - 8): amax 1 -> byte 119; amax just
    under 2 -> 119; amax 2 -> 120; zero block -> 0; amax 2^-125 -> clamped 0."""
    cases = [(1.0, 119), (1.9999, 119), (2.0, 120), (0.0, 0), (2.0 ** -125, 0), (448.0, 127 + 8 - 8)]
    for amax, byte in cases:
        blk = np.zeros(32)
        blk[7] = -amax
        assert o.mx_scale_bytes(blk[None, :])[0, 0] == byte, amax
    q, sb = o.mx_quantize(np.full((1, 32), 3.0))                # 3 = 1.5 * 2^1: scale 2^-7, element 384
    assert sb[0, 0] == 120 and np.all(q == 384.0)


def test_mx_round_trip_error_bound():
    """Every element of a block lands in [256, 512) * scale at most for the
    block maximum, so the relative error is <= 2^-4 for elements >= 2^-6 of
    the scaled range and the clipped maximum loses < 12.5%."""
    rng = np.random.default_rng(3)
    a = rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    r = o.mx_round(a)
    q, sb = o.mx_quantize(a)
    assert np.all(np.abs(q) <= 448)
    scale = np.repeat(np.ldexp(1.0, sb - 127), 32, axis=1)
    norm = np.abs(a) / scale >= 2.0 ** -6
    rel = np.abs(r - a) / np.abs(a)
    assert np.all(rel[norm & (np.abs(a) / scale < 464)] <= 2.0 ** -4 + 1e-12)
    assert np.all(rel[np.abs(a) / scale >= 464] < 0.125)
    np.testing.assert_array_equal(o.mx_round(r), r)            # idempotent


def test_mx_experts_equal_bf16_where_exact():
    """With W_g, W_u, W_d made of {0, +-1/2, +-1, +-2} and a 2 in every
    block, MXFP8 holds the weights exactly; the MXFP8 layer then differs
    from the bf16 one only through the rounding of the activations z and H,
    by less than the MXFP8 error, and never in which hidden units are zero."""
    shape = wl.LayerShape("mx", 23, "bf16", T=40, d=128, l=128, E=4, k=2, f=128, f_s=0, B=256)
    W = wl.make_weights(shape)
    rng = np.random.default_rng(1)
    for n in ("W_g", "W_u", "W_d"):
        v = rng.choice([0.0, 0.5, -0.5, 1.0, -1.0, 2.0], size=W[n].shape)
        v[..., ::32] = 2.0
        W[n] = (v * 2.0 ** -4).astype(F32)
        np.testing.assert_array_equal(o.mx_round(W[n]), W[n])
    x = wl.make_x(shape)
    fb = o.forward(x, W, np.zeros(4, F32), k=2, dtype="bf16")
    fm = o.forward(x, W, np.zeros(4, F32), k=2, dtype="bf16", logits=fb["logits"], experts="mxfp8")
    den = np.abs(fb["out"]).max()
    assert 0 < np.abs(fm["out"] - fb["out"]).max() / den < 0.1
    np.testing.assert_array_equal(fm["H"] != 0, fb["H"] != 0)


# ---------------------------------------------------------------- MXFP4 --
def _e2m1_codes():
    """(value, mantissa bit) of the 16 E2M1 codes, decoded from the bit
    fields: sign, 2 exponent bits (bias 1, 0 = subnormal), 1 mantissa bit."""
    out = []
    for code in range(16):
        s = -1.0 if code & 8 else 1.0
        e, m = (code >> 1) & 3, code & 1
        v = m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1)
        out.append((s * v, m))
    return out


def _e2m1_brute(x):
    """Nearest code value by search; ties to the code whose mantissa bit is
    0; beyond the largest value, saturate."""
    codes = _e2m1_codes()
    res = np.empty(len(x))
    for i, v in enumerate(x):
        v = float(np.clip(v, -6.0, 6.0))
        d = [abs(v - c) for c, _ in codes]
        best = min(d)
        cands = [(c, m) for (c, m), dd in zip(codes, d) if dd == best]
        even = [c for c, m in cands if m == 0]
        res[i] = (even or [cands[0][0]])[0]
    return res


def test_e2m1_round_matches_brute_force():
    vals = np.unique([c for c, _ in _e2m1_codes()])
    assert len(vals) == 15 and vals.max() == 6.0            # +-0 coincide
    mids = (vals[1:] + vals[:-1]) / 2
    rng = np.random.default_rng(4)
    rand = rng.uniform(-9, 9, 4000)
    x = np.concatenate([vals, mids, np.nextafter(mids, -1e9), np.nextafter(mids, 1e9), rand, [7.0, -7.5, 1e9]])
    np.testing.assert_array_equal(o.e2m1_round(x), _e2m1_brute(x))


def test_e2m1_ties_table():
    x = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 5.0001, 6.9, 7.0, 100.0])
    want = np.array([0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, 6.0, 6.0])
    np.testing.assert_array_equal(o.e2m1_round(x), want)
    np.testing.assert_array_equal(o.e2m1_round(-x), -want)


def test_mx4_scale_closed_form():
    """Block scale 2^(floor(log2 amax) - 2): amax 6 and 4 -> byte 127, amax
    just under 4 -> 126, amax 1 -> 125, zero block -> 0."""
    for amax, byte in [(6.0, 127), (4.0, 127), (3.999, 126), (1.0, 125), (0.0, 0), (2.0 ** -130, 0)]:
        blk = np.zeros(32)
        blk[3] = amax
        assert o.mx4_scale_bytes(blk[None, :])[0, 0] == byte, amax
    q, sb = o.mx4_quantize(np.full((1, 32), 3.0))            # 3 = 1.5 * 2^1: scale 2^-1, element 6
    assert sb[0, 0] == 126 and np.all(q == 6.0)


def test_mx4_round_trip_error_bound():
    """Elements of a block lie in [4, 8) * scale at most for the block
    maximum: relative error <= 1/4 inside the normal range (|a| / scale >=
    1, below the 6 -> 7 saturation edge), and the clipped maximum loses
    < 25%."""
    rng = np.random.default_rng(5)
    a = rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    r = o.mx4_round(a)
    q, sb = o.mx4_quantize(a)
    assert np.all(np.abs(q) <= 6)
    scale = np.repeat(np.ldexp(1.0, sb - 127), 32, axis=1)
    u = np.abs(a) / scale
    rel = np.abs(r - a) / np.abs(a)
    assert np.all(rel[(u >= 1) & (u < 7)] <= 0.25 + 1e-12)
    assert np.all(rel[u >= 7] < 0.25)
    np.testing.assert_array_equal(o.mx4_round(r), r)


def test_mxfp4_layer_equals_mxfp8_where_both_exact():
    """Weights from {0, +-1/2, +-1, +-3/2, +-2, +-3, +-4, +-6} * 2^-4 with a 6
    in every block are exact in MXFP4 and in MXFP8; the two expert formats
    then give the same layer bit for bit (the activations are MXFP8 in both).
    Random weights: the MXFP4 layer differs from the MXFP8 one."""
    shape = wl.LayerShape("mx4", 29, "bf16", T=48, d=128, l=128, E=4, k=2, f=128, f_s=0, B=256)
    W = wl.make_weights(shape)
    x = wl.make_x(shape)
    f8 = o.forward(x, W, np.zeros(4, F32), k=2, dtype="bf16", experts="mxfp8")
    f4 = o.forward(x, W, np.zeros(4, F32), k=2, dtype="bf16", logits=f8["logits"], experts="mxfp4")
    assert not np.array_equal(f4["out"], f8["out"])
    rng = np.random.default_rng(2)
    for n in ("W_g", "W_u", "W_d"):
        v = rng.choice([0.0, 0.5, -0.5, 1.0, -1.0, 1.5, -1.5, 2.0, 3.0, -3.0, 4.0, -4.0, 6.0, -6.0], size=W[n].shape)
        v[..., ::32] = 6.0
        W[n] = (v * 2.0 ** -4).astype(F32)
        np.testing.assert_array_equal(o.mx4_round(W[n]), W[n])
        np.testing.assert_array_equal(o.mx_round(W[n]), W[n])
    f8 = o.forward(x, W, np.zeros(4, F32), k=2, dtype="bf16", experts="mxfp8")
    f4 = o.forward(x, W, np.zeros(4, F32), k=2, dtype="bf16", logits=f8["logits"], experts="mxfp4")
    for n in ("H", "Y", "out"):
        np.testing.assert_array_equal(f4[n], f8[n])
