"""GPU parity of the whole layer forward through the C ABI.

The GPU's router logits are checked against the oracle's own (tolerance),
then injected into the oracle so that routing is compared bit for bit and the
outputs (and intermediates) within max|d|/max|ref| <= 1e-4 (fp32) / 2e-2
(bf16)."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as o
from sparse_moe_layer_rmsnorm_amd import workloads as wl

from gpu_util import (LOGIT_TOL, OUT_TOL, assert_routing_equal, compare_full, make_layer, rel_err, say,
                      stored_intermediates, to_np, x_on_gpu)

pytestmark = pytest.mark.gpu
F32 = np.float32


def _run(shape, T, *, bias=None, c=None, step=0, compare_inner=True, layer=None, W=None):
    W = wl.make_weights(shape) if W is None else W
    if c is not None:
        W = dict(W, c=c)
    x = wl.make_x(shape.with_tokens(T), step)
    own = layer is None
    if own:
        layer = make_layer(shape, W, max_tokens=T, c=c)
        if bias is not None:
            layer.set_bias(bias)
    b = to_np(layer.get_bias())
    r = layer.route_buffers(T)
    out = layer.forward(x_on_gpu(x, layer), route=r)
    torch.cuda.synchronize()
    lg = to_np(r["logits"])
    ref_own = o.forward(x, W, b, k=shape.k, dtype=shape.dtype, eps=shape.rms_eps, B=shape.B)
    assert rel_err(lg, ref_own["logits"]) <= LOGIT_TOL[shape.dtype]
    ref = o.forward(x, W, b, k=shape.k, dtype=shape.dtype, eps=shape.rms_eps, B=shape.B, logits=lg)
    assert_routing_equal(r, ref, T)
    if compare_inner:  # intermediates first: a failure then names the first wrong step
        v = layer.ws_views(T)
        for name in stored_intermediates(shape, v):
            e = rel_err(to_np(v[name]), ref[name])
            say(f"  {name} rel err {e:.3e}")
            assert e <= OUT_TOL[shape.dtype], name
    err = rel_err(to_np(out), ref["out"])
    say(f"  out rel err {err:.3e}")
    assert err <= OUT_TOL[shape.dtype]
    if own:
        layer.close()
    return ref, out


def _small(dtype, **kw):
    base = dict(T=1, d=128, l=64, E=16, k=2, f=64, f_s=128)
    base.update(kw)
    return wl.LayerShape("case", 9, dtype, **base)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 77, 300])
def test_forward_small(dtype, T):
    say(f"forward small {dtype} T={T}")
    _run(_small(dtype), T, bias=(np.random.default_rng(T).standard_normal(16) * 0.05).astype(F32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_no_shared_expert(dtype):
    say(f"forward no shared {dtype}")
    _run(_small(dtype, f_s=0, E=40, k=5, l=128, f=192), 150)


def test_tiny_workload_train_update_train():
    """The tiny fp32 workload: forward (b = 0), QB update, second forward."""
    shape = wl.workload("tiny")
    say("tiny workload")
    W = wl.make_weights(shape)
    layer = make_layer(shape, W, max_tokens=shape.T)
    ref0, _ = _run(shape, shape.T, layer=layer, W=W, step=0)
    layer.qb_update()
    torch.cuda.synchronize()
    b1 = o.qb_update(ref0["hist"], shape.T, shape.k, np.zeros(shape.E, F32))
    np.testing.assert_array_equal(to_np(layer.get_bias()).view(np.uint32), b1.view(np.uint32))
    _run(shape, shape.T, layer=layer, W=W, step=1)
    layer.close()


def test_replica_shape_ragged():
    shape = wl.workload("replica")
    say("replica shape T=1000")
    _run(shape, 1000, bias=(np.random.default_rng(5).standard_normal(shape.E) * 0.02).astype(F32))


def test_replica_full_size_all_elements():
    """The replica workload at full size (T=8192), as the benchmark runs it:
    the oracle's whole forward with the GPU logits injected; routing and the
    QB histogram bit-exact; every element of h, z, G, H, Y, y_lat and out
    compared (64 m-tiles x 36 n-tiles of the h GEMM: the persistent blocks'
    cross-tile DMA ring and tile switches are all in play)."""
    shape = wl.workload("replica")
    T = shape.T
    say(f"replica full T={T}")
    W = wl.make_weights(shape)
    x = wl.make_x(shape)
    layer = make_layer(shape, W, max_tokens=T)
    r = layer.route_buffers(T)
    out = layer.forward(x_on_gpu(x, layer), route=r)
    torch.cuda.synchronize()
    ref, _ = compare_full(shape, W, x, to_np(r["logits"]), r, out, layer.ws_views(T), np.zeros(shape.E, F32),
                          with_hist=True)
    np.testing.assert_array_equal(to_np(layer.state_views()["hist"]), ref["hist"])
    # the update's histogram quantiles (the state's q) against the exact,
    # sort-based quantiles of the same scores: within one bin width
    layer.qb_update()
    torch.cuda.synchronize()
    q = to_np(layer.state_views()["q"])
    np.testing.assert_array_equal(q, o.qb_quantiles(ref["hist"], T, shape.k))
    exact = np.array([o.exact_quantile(ref["s"][:, e], T, shape.k, shape.E) for e in range(shape.E)])
    qerr = float(np.abs(q - exact).max())
    say(f"  histogram quantile vs exact: max |q - q*| = {qerr:.5f} (bin width {1 / shape.B:.5f})")
    assert qerr <= 1.0 / shape.B
    layer.close()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_tall_expert_tiles(dtype):
    """T*k/E = 1024 rows per expert (>= 512): expert_up takes the 128-row
    tile table and pipeline (the path of the load-skew and decode-like
    workloads); every element of z, G, H, Y, y_lat and out compared.  With
    f_s = 1024 the h GEMM has 32 x 18 tiles, more than its 512 block slots, so
    the fp32 persistent loop crosses tiles as well."""
    say(f"forward tall expert tiles {dtype}")
    shape = wl.LayerShape("tall", 15, dtype, T=1, d=256, l=128, E=8, k=2, f=256, f_s=1024)
    _run(shape, 4096, bias=(np.random.default_rng(15).standard_normal(8) * 0.02).astype(F32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_odd_widths(dtype):
    """Widths that are multiples of 64 but not of the tiles: d=192, l=64,
    f=192, f_s=320, E=96 (partial router and latent tiles, 96 experts over
    64-lane columns), k=7, and a ragged T."""
    say(f"forward odd widths {dtype}")
    shape = wl.LayerShape("odd", 10, dtype, T=1, d=192, l=64, E=96, k=7, f=192, f_s=320)
    _run(shape, 203, bias=(np.random.default_rng(3).standard_normal(96) * 0.03).astype(F32))


@pytest.mark.parametrize("l,k", [(512, 6), (1024, 16), (1024, 3)])
def test_forward_wide_latent_rows(l, k):
    """Latent widths 512 and 1024 in bf16, whose combine reads whole rows per
    wavefront load (k = 16 in four batches of four slots; k = 3 leaves a
    partial batch), with a ragged T."""
    say(f"forward wide latent l={l} k={k}")
    shape = wl.LayerShape("wide", 11, "bf16", T=1, d=256, l=l, E=32, k=k, f=128, f_s=256)
    _run(shape, 301, bias=(np.random.default_rng(l + k).standard_normal(32) * 0.05).astype(F32))


def test_forward_k_max_and_single_expert():
    """k = 32 of E = 64 (the largest k), then E = k = 1 (one expert takes every token)."""
    say("forward k=32 of 64")
    _run(wl.LayerShape("kmax", 11, "bf16", T=1, d=128, l=64, E=64, k=32, f=64, f_s=64), 96)
    say("forward E=k=1")
    _run(wl.LayerShape("one", 12, "bf16", T=1, d=128, l=64, E=1, k=1, f=128, f_s=0), 130)


def test_forward_is_deterministic():
    """Two forwards of the same batch give bit-identical outputs and routing
    (no order-dependent atomics anywhere on the path)."""
    shape = wl.workload("replica", 2048)
    W = wl.make_weights(shape)
    layer = make_layer(shape, W, max_tokens=shape.T, frozen=True)
    xt = x_on_gpu(wl.make_x(shape), layer)
    r1, r2 = layer.route_buffers(shape.T), layer.route_buffers(shape.T)
    o1 = layer.forward(xt, route=r1).clone()
    o2 = layer.forward(xt, route=r2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    for key in r1:
        assert torch.equal(r1[key], r2[key]), key
    layer.close()


def test_forward_many_experts():
    """E = 1024 experts, k = 32 (the ABI's limits), small widths."""
    say("forward E=1024 k=32")
    _run(wl.LayerShape("wide", 13, "bf16", T=1, d=128, l=64, E=1024, k=32, f=64, f_s=64), 300,
         bias=(np.random.default_rng(13).standard_normal(1024) * 0.02).astype(F32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_route_from_x_odd_shape(dtype):
    """The routing-only pass from x (RMSNorm + the router-only GEMM) on odd
    widths: routing bit-exact from its own logits, logits by tolerance."""
    shape = wl.LayerShape("odd", 14, dtype, T=1, d=320, l=64, E=96, k=5, f=64, f_s=0)
    T = 257
    W = wl.make_weights(shape)
    x = wl.make_x(shape.with_tokens(T))
    layer = make_layer(shape, W, max_tokens=T)
    r = layer.route(T, x=x_on_gpu(x, layer))
    torch.cuda.synchronize()
    lg = to_np(r["logits"])
    ref_own = o.forward(x, W, np.zeros(96, F32), k=shape.k, dtype=dtype, eps=shape.rms_eps, B=shape.B)
    assert rel_err(lg, ref_own["logits"]) <= LOGIT_TOL[dtype]
    ref = o.forward(x, W, np.zeros(96, F32), k=shape.k, dtype=dtype, eps=shape.rms_eps, B=shape.B, logits=lg)
    assert_routing_equal(r, ref, T)
    layer.close()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_two_shared_experts(dtype):
    """n_shared = 2 shared experts of hidden 64 each, their weights stacked
    along the hidden axis: the layer equals the oracle's single shared GLU of
    hidden 128 (the stacking identity is pinned on the CPU)."""
    say(f"forward two shared experts {dtype}")
    shape = _small(dtype, f_s=128)
    T = 150
    W = wl.make_weights(shape)
    x = wl.make_x(shape.with_tokens(T))
    layer = make_layer(shape, W, max_tokens=T, n_shared=2)
    r = layer.route_buffers(T)
    out = layer.forward(x_on_gpu(x, layer), route=r)
    torch.cuda.synchronize()
    compare_full(shape, W, x, to_np(r["logits"]), r, out, layer.ws_views(T), np.zeros(shape.E, F32))
    layer.close()
