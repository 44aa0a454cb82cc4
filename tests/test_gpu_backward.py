"""GPU parity of the backward pass (moe_backward through the C ABI) against the
oracle's hand-derived chain, which is itself pinned to torch.autograd.

The forward runs on the GPU first; its router logits are injected into the
oracle forward so both sides route identically, then every gradient (dx and
all weights) is compared at the layer tolerance: max|GPU - oracle| /
max|oracle| <= 2e-2 in bf16 mode, 1e-4 in fp32 mode."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as o
from sparse_moe_layer_rmsnorm_amd import workloads as wl

from gpu_util import OUT_TOL, make_layer, rel_err, say, to_np, x_on_gpu

pytestmark = pytest.mark.gpu
F32 = np.float32
NAMES = ["gamma", "W_r", "W_sg", "W_su", "W_sd", "W_dn", "W_g", "W_u", "W_d", "W_up"]

CASES = [  # name, dtype, T, d, l, E, k, f, f_s
    ("tiny", "f32", 256, 256, 64, 16, 2, 128, 256),
    ("replica-widths", "bf16", 1000, 1024, 256, 256, 6, 512, 2048),
    ("odd", "bf16", 203, 192, 64, 100, 7, 192, 0),
    ("single-expert", "bf16", 130, 128, 64, 1, 1, 64, 64),
    ("k32", "bf16", 70, 128, 64, 64, 32, 64, 128),
    ("replica", "bf16", 8192, 1024, 256, 256, 6, 512, 2048),   # the benchmarked size
    ("wide", "bf16", 300, 128, 64, 1024, 32, 64, 64),          # most experts and slots: router rows up to Epad
    ("deep", "bf16", 4096, 256, 128, 8, 2, 256, 256),          # 1024 rows per expert: block-wide tile tables
]


@pytest.mark.parametrize("keep", [False, True], ids=["recompute", "kept"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(case, keep):
    """keep: the forward stores the GLU pre-activations (keep_preact) and the
    backward reads them instead of recomputing them."""
    name, dtype, T, d, l, E, k, f, f_s = case
    say(f"backward {name}: T={T} d={d} l={l} E={E} k={k} f={f} f_s={f_s} {dtype} keep={keep}")
    shape = wl.LayerShape(name, 21, dtype, T=T, d=d, l=l, E=E, k=k, f=f, f_s=f_s, B=256)
    W = wl.make_weights(shape)
    rng = np.random.default_rng(T + E)
    W["gamma"] = (1.0 + 0.2 * rng.standard_normal(d)).astype(F32)
    x = wl.make_x(shape)
    dout = rng.standard_normal((T, d)).astype(F32)
    if dtype == "bf16":
        dout = o.bf16_round(dout).astype(F32)
    bias = (rng.standard_normal(E) * 0.05).astype(F32)
    layer = make_layer(shape, W, max_tokens=T, keep_preact=keep)
    layer.set_bias(bias)
    r = layer.route_buffers(T)
    xg = x_on_gpu(x, layer)
    layer.forward(xg, route=r)
    dx, grads = layer.backward(xg, x_on_gpu(dout, layer), route=r)
    torch.cuda.synchronize()
    fwd = o.forward(x, W, bias, k=k, dtype=dtype, eps=shape.rms_eps, logits=to_np(r["logits"]))
    np.testing.assert_array_equal(to_np(r["topk_idx"]), fwd["idx"])
    ref = o.backward(x, W, dout, fwd, dtype=dtype, eps=shape.rms_eps)
    tol = OUT_TOL[dtype]
    errs = {"x": rel_err(to_np(dx), ref["x"])}
    for n in NAMES:
        if n in grads:
            errs[n] = rel_err(to_np(grads[n]), ref[n])
    say("  " + " ".join(f"{n}:{v:.2e}" for n, v in errs.items()))
    for n, v in errs.items():
        assert v <= tol, (n, v)
    layer.close()


def test_backward_is_deterministic_and_leaves_qb_state():
    shape = wl.LayerShape("det", 22, "bf16", T=300, d=256, l=64, E=32, k=4, f=128, f_s=256, B=256)
    W = wl.make_weights(shape)
    x = wl.make_x(shape)
    dout = o.bf16_round(np.random.default_rng(1).standard_normal((shape.T, shape.d))).astype(F32)
    layer = make_layer(shape, W, max_tokens=shape.T)
    xg = x_on_gpu(x, layer)
    layer.forward(xg)
    st0 = {n: v.clone() for n, v in layer.state_views().items()}
    dx1, g1 = layer.backward(xg, x_on_gpu(dout, layer))
    torch.cuda.synchronize()
    dx1, g1 = dx1.clone(), {n: v.clone() for n, v in g1.items()}
    dx2, g2 = layer.backward(xg, x_on_gpu(dout, layer))
    torch.cuda.synchronize()
    assert torch.equal(dx1, dx2)
    for n in g1:
        assert torch.equal(g1[n], g2[n]), n
    for n, v in layer.state_views().items():
        assert torch.equal(v, st0[n]), n
    layer.close()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kept_preactivations(dtype):
    """keep_preact changes no output bit of the forward, and the stored P, Q,
    A, U are the products of the GPU's own h and dispatched z rows with the
    weights (oracle in fp64, rounded to the storage dtype) at the layer
    tolerance."""
    shape = wl.LayerShape("keep", 23, dtype, T=1000, d=1024, l=256, E=256, k=6, f=512, f_s=2048, B=256)
    if dtype == "f32":
        shape = wl.LayerShape("keep", 23, dtype, T=300, d=256, l=128, E=32, k=4, f=192, f_s=128, B=256)
    W = wl.make_weights(shape)
    x = wl.make_x(shape)
    T = shape.T
    say(f"kept pre-activations {dtype}: T={T}")
    plain = make_layer(shape, W, max_tokens=T, frozen=True)
    kept = make_layer(shape, W, max_tokens=T, frozen=True, keep_preact=True)
    out0 = plain.forward(x_on_gpu(x, plain)).clone()
    r = kept.route_buffers(T)
    out1 = kept.forward(x_on_gpu(x, kept), route=r)
    torch.cuda.synchronize()
    assert torch.equal(out0, out1)
    v = kept.ws_views(T)
    h = to_np(v["h"]).astype(np.float64)
    st = o.bf16_round if dtype == "bf16" else (lambda a: a.astype(F32).astype(np.float64))
    tol = OUT_TOL[dtype]
    for n, w in (("P", "W_sg"), ("Q", "W_su")):
        want = st(h @ W[w].astype(np.float64).T)
        assert rel_err(to_np(v[n]), want) <= tol, n
    X = to_np(v["z"]).astype(np.float64)[to_np(r["perm_src"])]
    offs = to_np(r["offsets"])
    for n, w in (("A", "W_g"), ("U", "W_u")):
        got = to_np(v[n]).astype(np.float64)
        want = np.zeros_like(got)
        for e in range(shape.E):
            a, b = int(offs[e]), int(offs[e + 1])
            want[a:b] = st(X[a:b] @ W[w][e].astype(np.float64).T)
        assert rel_err(got, want) <= tol, n
    plain.close()
    kept.close()


def test_training_step_graph_replay():
    """forward (pre-activations kept) + backward + qb_update captured in one
    graph: every replay, with eager work and synchronisation between
    replays, equals the eager step bit for bit (out, dx, every gradient, bias)."""
    shape = wl.LayerShape("graph", 24, "bf16", T=1024, d=1024, l=256, E=256, k=6, f=512, f_s=2048, B=256)
    T = shape.T
    say(f"training-step graph replay: T={T}")
    W = wl.make_weights(shape)
    layer = make_layer(shape, W, max_tokens=T, keep_preact=True)
    xt = x_on_gpu(wl.make_x(shape), layer)
    dout = x_on_gpu(o.bf16_round(np.random.default_rng(3).standard_normal((T, shape.d))).astype(F32), layer)
    r = layer.route_buffers(T)
    out = torch.empty(T, shape.d, dtype=layer.tdtype, device="cuda")

    def step(grads=None):
        layer.forward(xt, out=out, route=r)
        dx, g = layer.backward(xt, dout, route=r, grads=grads)
        layer.qb_update()
        return dx, g

    dx1, grads = step()                                  # bias 0, then the QB bias
    dx2, _ = step(grads)                                 # the converged bias: a fixed point
    torch.cuda.synchronize()
    ref = {"out": out.clone(), "dx": dx2.clone(), "bias": layer.get_bias().clone()}
    ref.update({n: v.clone() for n, v in grads.items()})
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(grads)                                      # warm the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dxc, _ = step(grads)
    for i in range(4):
        out.zero_()
        dxc.zero_()
        for v in grads.values():
            v.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = {"out": out, "dx": dxc, "bias": layer.get_bias()}
        got.update(grads)
        for n, v in ref.items():
            assert torch.equal(got[n], v), (i, n)
        _ = (xt.float() * 2).sum().item()               # unrelated eager work between replays
    layer.close()
