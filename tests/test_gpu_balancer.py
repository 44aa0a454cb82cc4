"""GPU parity of the sign-rule balancer (capsule 16 of the "Pretraining a Mini
Kimi K3" review: b_e += gamma * sign(mean load - load_e)), through the C ABI.

Given injected logits the accumulated loads, the token count and the new bias
equal the oracle's bit for bit; on the full load-skew workload the GPU logits
are fed to the oracle step by step and the bias is compared every step."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as o
from sparse_moe_layer_rmsnorm_amd import workloads as wl

from gpu_util import assert_routing_equal, compare_full, make_layer, oracle_routing, say, to_np, x_on_gpu

pytestmark = pytest.mark.gpu
F32 = np.float32
GAMMA = 1e-2


def _shape(E, k, d=64, l=64, f=64, f_s=64, dtype="bf16", B=256):
    return wl.LayerShape("case", 9, dtype, T=1, d=d, l=l, E=E, k=k, f=f, f_s=f_s, B=B)


@pytest.mark.parametrize("E,k,Ts", [(16, 2, (256, 100)), (256, 6, (8192, 4097)), (1024, 32, (700, 3)),
                                    (100, 7, (333, 1))])
def test_sign_rule_accumulates_and_updates_bitexact(E, k, Ts):
    """Two routing calls accumulate loads and the token count (no histogram);
    qb_update moves the bias one gamma step and clears both; the next call
    routes with the new bias."""
    say(f"sign E={E} k={k} T={Ts}")
    rng = np.random.default_rng(E + 5 * k)
    shape = _shape(E, k)
    W = wl.make_weights(shape)
    layer = make_layer(shape, W, max_tokens=max(Ts), balancer="sign", sign_gamma=GAMMA)
    bias = (rng.standard_normal(E) * 0.05).astype(F32)
    layer.set_bias(bias)
    load = np.zeros(E, np.int64)
    for T in Ts:
        logits = (rng.standard_normal((T, E)) + np.linspace(0, 2, E)).astype(F32)   # skewed loads
        r = layer.route(T, logits=torch.from_numpy(logits).cuda())
        torch.cuda.synchronize()
        ref = oracle_routing(logits, bias, k, E, shape.B)
        assert_routing_equal(r, ref, T)
        load += ref["counts"]
        st = layer.state_views()
        np.testing.assert_array_equal(to_np(st["load"]), load)
        assert int(st["count"].item()) == int(sum(Ts[:Ts.index(T) + 1]))
        assert int(st["hist_slices"].abs().sum().item()) == 0       # the sign rule builds no histogram
    layer.qb_update()
    torch.cuda.synchronize()
    bias = o.sign_update(load, bias, GAMMA)
    np.testing.assert_array_equal(to_np(layer.get_bias()).view(np.uint32), bias.view(np.uint32))
    st = layer.state_views()
    assert int(st["load"].abs().sum().item()) == 0 and int(st["count"].item()) == 0
    T = Ts[-1]
    logits = rng.standard_normal((T, E)).astype(F32)
    r = layer.route(T, logits=torch.from_numpy(logits).cuda())
    torch.cuda.synchronize()
    assert_routing_equal(r, oracle_routing(logits, bias, k, E, shape.B), T)
    layer.close()


def test_sign_rule_frozen_and_empty():
    """Frozen: nothing accumulates and the update keeps the bias.  Training
    with no token since the last update: every sign is 0, the bias stays."""
    E, k, T = 64, 4, 500
    shape = _shape(E, k)
    layer = make_layer(shape, wl.make_weights(shape), max_tokens=T, balancer="sign", sign_gamma=GAMMA)
    b = np.random.default_rng(1).standard_normal(E).astype(F32)
    layer.set_bias(b)
    layer.qb_update()                                              # nothing accumulated
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(layer.get_bias()).view(np.uint32), b.view(np.uint32))
    layer.set_qb_mode(frozen=True)
    logits = np.random.default_rng(2).standard_normal((T, E)).astype(F32)
    layer.route(T, logits=torch.from_numpy(logits).cuda())
    layer.qb_update()
    torch.cuda.synchronize()
    st = layer.state_views()
    assert int(st["load"].abs().sum().item()) == 0 and int(st["count"].item()) == 0
    np.testing.assert_array_equal(to_np(layer.get_bias()).view(np.uint32), b.view(np.uint32))
    layer.close()


def test_sign_rule_skew_workload_loop():
    """Full load-skew workload (T=32768, Zipf logit offsets), 12 training
    forwards with the sign rule, fresh x each step: routing and bias bit-exact
    every step; max/mean load from > 10 to < 3 by step 6 and < 2 from step 8
    (the oracle shows the same walk; one QB step reaches < 1.6)."""
    shape = wl.workload("skew")
    T = shape.T
    W = wl.make_weights(shape)
    c = wl.zipf_logit_offset(shape)
    W = dict(W, c=c)
    layer = make_layer(shape, W, max_tokens=T, c=c, balancer="sign", sign_gamma=GAMMA)
    bias = np.zeros(shape.E, F32)
    r = layer.route_buffers(T)
    ratios = []
    for step in range(12):
        say(f"sign skew step {step}")
        x = wl.make_x(shape, step)
        out = layer.forward(x_on_gpu(x, layer), route=r)
        layer.qb_update()
        torch.cuda.synchronize()
        lg = to_np(r["logits"])
        ref = oracle_routing(lg, bias, shape.k, shape.E, shape.B)
        assert_routing_equal(r, ref, T)
        ref_bias = bias
        st = o.load_stats(ref["counts"])
        ratios.append(st["max_over_mean"])
        say(f"  max/min {st['max_over_min']:.2f} max/mean {st['max_over_mean']:.2f} dead {st['dead']}")
        bias = o.sign_update(ref["counts"], bias, GAMMA)
        np.testing.assert_array_equal(to_np(layer.get_bias()).view(np.uint32), bias.view(np.uint32))
        if step in (0, 11):                             # every element, with the bias of this step
            compare_full(shape, W, x, lg, r, out, layer.ws_views(T), ref_bias)
    assert ratios[0] > 10
    assert ratios[6] < 3
    assert max(ratios[8:]) < 2
    layer.close()
