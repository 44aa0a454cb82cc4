"""Pins of the oracle's backward pass.

The oracle writes every gradient out by hand (chain rule, permutation and
combine transposes).  It is checked against torch.autograd in fp64 on an
independent dense formulation of the layer (every token's selected experts
evaluated in place, no permutation, torch's own sigmoid and SiLU), with the
routing decisions fixed to the oracle's; plus special cases the mathematics
fixes: a zero upstream gradient, E = k = 1 (gates are constant, so the router
gets no gradient), the bias never receiving a gradient, and bf16 rounding
staying within bf16 error of the unrounded chain."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as o
from sparse_moe_layer_rmsnorm_amd import workloads as wl

F32 = np.float32


def _shape(T, d, l, E, k, f, f_s, dtype="f32"):
    return wl.LayerShape("case", 11, dtype, T=T, d=d, l=l, E=E, k=k, f=f, f_s=f_s, B=256)


def _setup(shape, seed=0, bias_scale=0.1):
    W = wl.make_weights(shape)
    x = wl.make_x(shape)
    rng = np.random.default_rng(seed)
    W["gamma"] = (1.0 + 0.2 * rng.standard_normal(shape.d)).astype(F32)
    bias = (rng.standard_normal(shape.E) * bias_scale).astype(F32)
    dout = rng.standard_normal((shape.T, shape.d)).astype(F32)
    return W, x, bias, dout


def _torch_grads(shape, W, x, idx, dout, eps, rs=1.0, gates=None):
    """Gradients of sum(out * dout) by torch.autograd (fp64), dense form;
    res["out"] is torch's forward output.  ``gates`` (fp32 [T,k]) replaces
    the gates computed from torch's sigmoid (the forward check then isolates
    the assembly of the output from the score function)."""
    t = {n: torch.tensor(np.asarray(v, np.float64), requires_grad=True) for n, v in W.items() if v is not None}
    xt = torch.tensor(np.asarray(x, np.float64), requires_grad=True)
    it = torch.tensor(idx.astype(np.int64))
    r = torch.rsqrt((xt * xt).mean(1, keepdim=True) + eps)
    h = t["gamma"] * xt * r
    lg = h @ t["W_r"].T
    s = torch.sigmoid(lg)
    s_sel = s.gather(1, it)
    g = rs * s_sel / s_sel.sum(1, keepdim=True)
    if gates is not None:
        g = torch.tensor(np.asarray(gates, np.float64))
    z = h @ t["W_dn"].T
    y_lat = torch.zeros(shape.T, shape.l, dtype=torch.float64)
    for j in range(shape.k):
        e = it[:, j]
        A = torch.einsum("tl,tfl->tf", z, t["W_g"][e])
        U = torch.einsum("tl,tfl->tf", z, t["W_u"][e])
        Hj = torch.nn.functional.silu(A) * U
        Yj = torch.einsum("tf,tlf->tl", Hj, t["W_d"][e])
        y_lat = y_lat + g[:, j:j + 1] * Yj
    out = y_lat @ t["W_up"].T
    if shape.f_s > 0:
        G = torch.nn.functional.silu(h @ t["W_sg"].T) * (h @ t["W_su"].T)
        out = out + G @ t["W_sd"].T
    (out * torch.tensor(np.asarray(dout, np.float64))).sum().backward()
    res = {n: v.grad.numpy() for n, v in t.items() if v.grad is not None}
    res["x"] = xt.grad.numpy()
    res["out"] = out.detach().numpy()
    return res


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    den = np.abs(b).max()
    return float(np.abs(a - b).max() / (den if den > 0 else 1.0))


NAMES = ["x", "gamma", "W_r", "W_sg", "W_su", "W_sd", "W_dn", "W_g", "W_u", "W_d", "W_up"]


@pytest.mark.parametrize("dims", [
    (64, 64, 32, 8, 2, 32, 64),      # T, d, l, E, k, f, f_s
    (37, 64, 64, 5, 3, 64, 0),       # no shared expert, ragged T
    (50, 32, 16, 16, 16, 16, 32),    # k = E
])
def test_backward_matches_autograd(dims):
    T, d, l, E, k, f, f_s = dims
    shape = _shape(T, d, l, E, k, f, f_s)
    W, x, bias, dout = _setup(shape, seed=T)
    fwd = o.forward(x, W, bias, k=k, dtype="f32", eps=shape.rms_eps)
    got = o.backward(x, W, dout, fwd, dtype="f32", eps=shape.rms_eps)
    want = _torch_grads(shape, W, x, fwd["idx"], dout, shape.rms_eps)
    # the forward output itself: torch's dense formulation (its own sigmoid,
    # SiLU and per-token expert evaluation, no permutation) against the
    # oracle's dispatch path in f32 mode (nothing rounded)
    assert _rel(fwd["out"], want["out"]) < 1e-6
    for n in NAMES:
        if n in ("W_sg", "W_su", "W_sd") and f_s == 0:
            continue
        # the oracle's scores come from the fp32-specified sigmoid, torch's from
        # its fp64 one: agreement to ~1e-7 relative, far below any dropped term
        assert _rel(got[n], want[n]) < 1e-5, n


@pytest.mark.parametrize("dims", [
    (64, 64, 32, 8, 2, 32, 64),      # T, d, l, E, k, f, f_s
    (37, 64, 64, 5, 3, 64, 0),       # no shared expert, ragged T
    (50, 32, 16, 16, 16, 16, 32),    # k = E
    (96, 128, 64, 1, 1, 64, 0),      # E = k = 1: a dense GLU at width l
])
def test_forward_output_matches_torch(dims):
    """out = shared GLU + up-projection of the gate-weighted combine, with
    the oracle's own gates fed to torch: the two fp64 evaluations (dispatch
    through the permutation against every token's experts in place) agree
    to rounding, 1e-12 relative, which a dropped term, a wrong gate or a
    transposed weight would break by many orders of magnitude."""
    T, d, l, E, k, f, f_s = dims
    shape = _shape(T, d, l, E, k, f, f_s)
    W, x, bias, dout = _setup(shape, seed=T + 1)
    fwd = o.forward(x, W, bias, k=k, dtype="f32", eps=shape.rms_eps)
    want = _torch_grads(shape, W, x, fwd["idx"], dout, shape.rms_eps, gates=fwd["gates"])
    assert _rel(fwd["out"], want["out"]) < 1e-12
    assert _rel(fwd["y_r"] + fwd["sh"], want["out"]) < 1e-12


def test_backward_routed_scale_matches_autograd():
    shape = _shape(40, 64, 32, 8, 3, 32, 64)
    W, x, bias, dout = _setup(shape, seed=5)
    fwd = o.forward(x, W, bias, k=3, dtype="f32", eps=shape.rms_eps, routed_scale=2.5)
    got = o.backward(x, W, dout, fwd, dtype="f32", eps=shape.rms_eps, routed_scale=2.5)
    want = _torch_grads(shape, W, x, fwd["idx"], dout, shape.rms_eps, rs=2.5)
    for n in NAMES:
        assert _rel(got[n], want[n]) < 1e-5, n


def test_backward_special_cases():
    """Zero upstream gradient -> every gradient is exactly 0.  E = k = 1: the
    single gate is routed_scale whatever the score, so the router weight
    gets exactly 0."""
    shape = _shape(30, 64, 32, 4, 2, 32, 64)
    W, x, bias, dout = _setup(shape)
    fwd = o.forward(x, W, bias, k=2, dtype="f32", eps=shape.rms_eps)
    zero = o.backward(x, W, np.zeros_like(dout), fwd, dtype="f32", eps=shape.rms_eps)
    for n in NAMES:
        assert np.all(zero[n] == 0), n
    one = _shape(30, 64, 32, 1, 1, 32, 0)
    W1, x1, b1, d1 = _setup(one)
    fwd1 = o.forward(x1, W1, b1, k=1, dtype="f32", eps=one.rms_eps)
    g1 = o.backward(x1, W1, d1, fwd1, dtype="f32", eps=one.rms_eps)
    assert np.all(g1["W_r"] == 0)
    assert np.abs(g1["W_g"]).max() > 0


def test_backward_bias_only_reroutes():
    """Two biases that select the same experts give identical gradients (the
    bias appears nowhere in the chain)."""
    shape = _shape(30, 64, 32, 6, 2, 32, 64)
    W, x, bias, dout = _setup(shape, bias_scale=0.0)
    f0 = o.forward(x, W, bias, k=2, dtype="f32", eps=shape.rms_eps)
    f1 = o.forward(x, W, bias + F32(1e-7), k=2, dtype="f32", eps=shape.rms_eps)
    assert np.array_equal(f0["idx"], f1["idx"])
    g0 = o.backward(x, W, dout, f0, dtype="f32", eps=shape.rms_eps)
    g1 = o.backward(x, W, dout, f1, dtype="f32", eps=shape.rms_eps)
    for n in NAMES:
        np.testing.assert_array_equal(g0[n], g1[n])


def test_backward_bf16_rounding_stays_within_bf16_error():
    """The bf16 chain (operands rounded where the device stores them) stays
    within a few bf16 ulps, relative to each gradient's scale, of the same
    chain unrounded on the same bf16 inputs."""
    shape = _shape(64, 64, 32, 8, 2, 64, 64, dtype="bf16")
    W, x, bias, dout = _setup(shape, seed=9)
    W = {n: (o.bf16_round(v).astype(F32) if n not in ("gamma",) else v) for n, v in W.items()}
    x = o.bf16_round(x).astype(F32)
    dout = o.bf16_round(dout).astype(F32)
    fb = o.forward(x, W, bias, k=2, dtype="bf16", eps=shape.rms_eps)
    gb = o.backward(x, W, dout, fb, dtype="bf16", eps=shape.rms_eps)
    ff = o.forward(x, W, bias, k=2, dtype="f32", eps=shape.rms_eps, logits=fb["logits"])
    gf = o.backward(x, W, dout, ff, dtype="f32", eps=shape.rms_eps)
    assert np.array_equal(fb["idx"], ff["idx"])
    for n in NAMES:
        assert _rel(gb[n], gf[n]) < 3e-2, n
