"""The no-alloc forward (moe_forward_noalloc), through the C ABI: its
workspace is the library's fixed per-GPU array instead of a caller's buffer.
It must give what moe_forward gives on the same inputs -- bit for bit, since
both run the same kernels on the same data -- on two calls in a row, the
second with fewer tokens (the array keeps the first call's contents), and
reject a batch whose workspace exceeds the array before enqueueing anything."""
import numpy as np
import pytest
import torch

from sparse_moe_layer_rmsnorm_amd import binding as Bd
from sparse_moe_layer_rmsnorm_amd import workloads as wl

from gpu_util import compare_full, make_layer, say, to_np, x_on_gpu

pytestmark = pytest.mark.gpu
F32 = np.float32


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _noalloc(layer, xt, T):
    out = torch.empty(T, layer.dims["d"], dtype=layer.tdtype, device="cuda")
    r = layer.route_buffers(T)
    Bd.moe_forward_noalloc(layer.ctx, xt.data_ptr(), T, out.data_ptr(), layer._route_struct(r), _stream())
    return out, r


@pytest.mark.parametrize("name,dtype", [("replica", "bf16"), ("tiny", "f32")])
def test_noalloc_forward_equals_forward(name, dtype):
    shape = wl.workload(name)
    T1 = shape.T
    T2 = T1 // 2 - 37                                  # second call: fewer tokens, ragged
    say(f"no-alloc forward {name}: T={T1} then T={T2}")
    W = wl.make_weights(shape)
    layer = make_layer(shape, W, max_tokens=T1, frozen=True)   # frozen: both paths see the same bias
    layer.set_bias((np.random.default_rng(7).standard_normal(shape.E) * 0.02).astype(F32))
    for step, T in enumerate((T1, T2)):
        x = wl.make_x(shape.with_tokens(T), step)
        xt = x_on_gpu(x, layer)
        got, r_got = _noalloc(layer, xt, T)
        torch.cuda.synchronize()
        r_want = layer.route_buffers(T)
        want = layer.forward(xt, route=r_want)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"call {step}: out differs from moe_forward"
        for key in r_want:
            assert torch.equal(r_got[key], r_want[key]), f"call {step}: {key}"
        if step == 1:                                  # and the oracle's bar on the second, smaller call
            compare_full(shape, W, x, to_np(r_got["logits"]), r_got, got, layer.ws_views(T),
                         to_np(layer.get_bias()), names=())
    layer.close()


def test_noalloc_training_forward_accumulates_like_forward():
    """In training mode the no-alloc forward adds the same histogram and
    token count as moe_forward (the statistics live in the state, not in the
    scratch)."""
    shape = wl.workload("replica", 1000)
    W = wl.make_weights(shape)
    a = make_layer(shape, W, max_tokens=shape.T)
    b = make_layer(shape, W, max_tokens=shape.T)
    xt = x_on_gpu(wl.make_x(shape), a)
    out_a, _ = _noalloc(a, xt, shape.T)
    out_b = b.forward(xt)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    assert torch.equal(a.state_views()["hist"], b.state_views()["hist"])
    assert int(a.state_views()["count"].item()) == shape.T
    a.qb_update()
    b.qb_update()
    torch.cuda.synchronize()
    assert torch.equal(a.get_bias(), b.get_bias())
    a.close()
    b.close()


def test_noalloc_rejects_batches_beyond_the_array():
    shape = wl.workload("replica", 16384)
    layer = make_layer(shape, wl.make_weights(shape), max_tokens=shape.T)
    assert Bd.moe_workspace_bytes(layer.cfg, shape.T) > Bd.MOE_NOALLOC_SCRATCH_BYTES
    assert Bd.moe_workspace_bytes(layer.cfg, 8192) <= Bd.MOE_NOALLOC_SCRATCH_BYTES
    xt = torch.zeros(shape.T, shape.d, dtype=layer.tdtype, device="cuda")
    out = torch.empty_like(xt)
    st0 = layer.state.clone()
    with pytest.raises(Bd.MoeError, match="MOE_ERR_WORKSPACE.*MOE_NOALLOC_SCRATCH_BYTES"):
        Bd.moe_forward_noalloc(layer.ctx, xt.data_ptr(), shape.T, out.data_ptr(), None, _stream())
    with pytest.raises(Bd.MoeError, match="MOE_ERR_SHAPE"):
        Bd.moe_forward_noalloc(layer.ctx, xt.data_ptr(), shape.T + 1, out.data_ptr(), None, _stream())
    Bd.moe_forward_noalloc(layer.ctx, xt.data_ptr(), 0, out.data_ptr(), None, _stream())   # T = 0: nothing
    torch.cuda.synchronize()
    assert torch.equal(layer.state, st0)               # nothing was enqueued
    layer.close()
