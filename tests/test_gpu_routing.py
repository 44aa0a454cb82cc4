"""GPU parity of the routing path and the QB update, through the C ABI.

Given bit-identical fp32 logits (injected), the scores, biased top-k, gates,
counts, offsets, permutation, histogram and QB bias must equal the oracle's
bit for bit."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as o
from sparse_moe_layer_rmsnorm_amd import workloads as wl

from gpu_util import assert_routing_equal, make_layer, oracle_routing, say, to_np

pytestmark = pytest.mark.gpu
F32 = np.float32


def _shape(E, k, d=64, l=64, f=64, f_s=64, dtype="bf16", B=256):
    return wl.LayerShape("case", 9, dtype, T=1, d=d, l=l, E=E, k=k, f=f, f_s=f_s, B=B)


CASES = [  # (E, k, T, logit scale, bias scale)
    (16, 2, 256, 1.0, 0.0),        # tiny workload shape
    (16, 2, 1000, 1.0, 0.1),
    (256, 6, 8192, 1.0, 0.05),     # replica shape
    (256, 6, 4097, 3.0, 0.05),     # ragged tail
    (896, 16, 2048, 1.0, 0.05),    # K3 routing shape
    (100, 7, 333, 2.0, 0.2),       # E not a multiple of 64
    (8, 8, 130, 1.0, 0.0),         # k = E
    (64, 1, 1, 1.0, 0.0),          # one token
    (1024, 32, 700, 1.0, 0.01),    # largest E and k
]


@pytest.mark.parametrize("E,k,T,ls,bs", CASES)
def test_route_injected_logits_bitexact(E, k, T, ls, bs):
    say(f"route E={E} k={k} T={T}")
    rng = np.random.default_rng(E * 7 + T)
    shape = _shape(E, k)
    W = wl.make_weights(shape)
    layer = make_layer(shape, W, max_tokens=T)
    logits = (rng.standard_normal((T, E)) * ls).astype(F32)
    logits[: min(T, 8)] = np.round(logits[: min(T, 8)] * 2) / 2      # exact ties in a few rows
    bias = (rng.standard_normal(E) * bs).astype(F32)
    layer.set_bias(bias)
    lg = torch.from_numpy(logits).cuda()
    r = layer.route(T, logits=lg)
    torch.cuda.synchronize()
    ref = oracle_routing(logits, bias, k, E, shape.B)
    assert_routing_equal(r, ref, T)
    st = layer.state_views()
    np.testing.assert_array_equal(to_np(st["hist"]), ref["hist"])
    assert int(st["count"].item()) == T
    layer.close()


def test_sigmoid_bitexact_sweep():
    """Scores over a dense sweep of logits: the GPU's bins and gates match the
    oracle's fp32-specified sigmoid exactly (k = 2 gates = s_a / (s_a + s_b))."""
    say("sigmoid sweep")
    E, k, T = 64, 2, 16384
    rng = np.random.default_rng(3)
    logits = np.concatenate([rng.uniform(-31, 31, (T // 2, E)), rng.standard_normal((T // 2, E)) * 2]).astype(F32)
    shape = _shape(E, k)
    layer = make_layer(shape, wl.make_weights(shape), max_tokens=T)
    r = layer.route(T, logits=torch.from_numpy(logits).cuda())
    torch.cuda.synchronize()
    ref = oracle_routing(logits, np.zeros(E, F32), k, E, shape.B)
    assert_routing_equal(r, ref, T)
    np.testing.assert_array_equal(to_np(layer.state_views()["hist"]), ref["hist"])
    layer.close()


@pytest.mark.parametrize("E,k,T,B", [(16, 2, 256, 256), (256, 6, 8192, 256), (896, 16, 4096, 256), (33, 3, 999, 64),
                                     (8, 2, 100, 2), (1024, 32, 700, 3)])
def test_qb_update_bitexact(E, k, T, B):
    say(f"qb_update E={E} k={k} T={T} B={B}")
    rng = np.random.default_rng(E + T)
    shape = _shape(E, k, B=B)
    layer = make_layer(shape, wl.make_weights(shape), max_tokens=T)
    off = (rng.standard_normal(E) * 0.7).astype(F32)
    bias = np.zeros(E, F32)
    hist_acc = np.zeros((E, B), np.int64)
    N = 0
    for step in range(3):                     # accumulate over two batches, then update; then one more
        logits = (rng.standard_normal((T, E)) + off[None, :]).astype(F32)
        r = layer.route(T, logits=torch.from_numpy(logits).cuda())
        ref = oracle_routing(logits, bias, k, E, B)
        torch.cuda.synchronize()
        assert_routing_equal(r, ref, T)
        hist_acc += ref["hist"]
        N += T
        if step >= 1:
            layer.qb_update()
            bias = o.qb_update(hist_acc, N, k, bias)
            hist_acc[:] = 0
            N = 0
            torch.cuda.synchronize()
            st = layer.state_views()
            np.testing.assert_array_equal(to_np(layer.get_bias()).view(np.uint32), bias.view(np.uint32))
            assert int(st["count"].item()) == 0
            assert int(st["hist"].abs().sum().item()) == 0
    layer.close()


def test_qb_frozen_and_empty():
    say("qb frozen / empty")
    E, k, T = 32, 4, 512
    shape = _shape(E, k)
    layer = make_layer(shape, wl.make_weights(shape), max_tokens=T)
    b0 = (np.random.default_rng(0).standard_normal(E) * 0.1).astype(F32)
    layer.set_bias(b0)
    layer.qb_update()                          # no tokens yet: bias kept
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(layer.get_bias()), b0)
    layer.set_qb_mode(True)
    logits = np.random.default_rng(1).standard_normal((T, E)).astype(F32)
    r = layer.route(T, logits=torch.from_numpy(logits).cuda())
    layer.qb_update()                          # frozen: no-op
    torch.cuda.synchronize()
    assert_routing_equal(r, oracle_routing(logits, b0, k, E, shape.B), T)
    st = layer.state_views()
    assert int(st["count"].item()) == 0 and int(st["hist"].abs().sum().item()) == 0
    np.testing.assert_array_equal(to_np(layer.get_bias()), b0)
    layer.close()
