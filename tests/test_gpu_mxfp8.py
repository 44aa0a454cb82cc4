"""GPU parity of the block-scaled expert paths (low-precision experts) through
the C ABI: MXFP8 weights and activations, and MXFP4 weights against MXFP8
activations, each against the oracle's rounding (MXFP8 pinned to torch's E4M3
conversion, MXFP4 to a brute-force E2M1 search).

The quantised weights in the state buffer must equal the oracle's element
for element (bytes or nibbles decoded to values, scales bit for bit); a
forward routes bit-exactly given its logits, and z, H, Y, y_lat and out agree
with the oracle: the quantisation of z and H bit for bit given the same bf16
input, each expert GEMM on the GPU's own input within the layer tolerance
(2e-2 of the largest magnitude), and the whole chain end to end within 5e-2
(a one-ulp bf16 difference upstream can move an element by one E4M3 step)."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as o
from sparse_moe_layer_rmsnorm_amd import binding as Bd
from sparse_moe_layer_rmsnorm_amd import workloads as wl

from gpu_util import OUT_TOL, assert_routing_equal, compare_full, make_layer, rel_err, say, to_np, x_on_gpu

pytestmark = pytest.mark.gpu
F32 = np.float32
# end-to-end bound of the MXFP8 layer against the oracle's own chain (see the
# comment in the test): one E4M3 step on isolated elements, 2.5x the bf16 bound
MX_E2E_TOL = 5e-2


def _e4m3_values(b: np.ndarray) -> np.ndarray:
    b = b.astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 15
    m = b & 7
    v = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    return s * v


def _e2m1_values(b: np.ndarray) -> np.ndarray:
    """Bytes holding two E2M1 codes (low nibble first) -> 2 values each."""
    b = b.astype(np.int64)
    codes = np.stack([b & 15, b >> 4], axis=-1).reshape(-1)
    s = np.where(codes & 8, -1.0, 1.0)
    e, m = (codes >> 1) & 3, codes & 1
    return s * np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))


FORMATS = {  # name: (decode of the weight bytes, weight rounding, bytes per element)
    "mxfp8": (_e4m3_values, o.mx_quantize, 1.0),
    "mxfp4": (_e2m1_values, o.mx4_quantize, 0.5),
}


def _state_mx(layer, shape, fmt):
    E, f, l = shape.E, shape.f, shape.l
    w = E * f * l
    dec, _, bpe = FORMATS[fmt]
    wb = int(w * bpe)
    raw = to_np(layer.state[layer.sl.mx:layer.sl.mx + 3 * wb + 3 * (w // 32)])
    q = [dec(raw[i * wb:(i + 1) * wb]) for i in range(3)]
    sc = [raw[3 * wb + i * (w // 32): 3 * wb + (i + 1) * (w // 32)].astype(np.int64) for i in range(3)]
    return q, sc


def _wround(fmt):
    return o.mx4_round if fmt == "mxfp4" else o.mx_round


SHAPES = [  # name, T, d, l, E, k, f, f_s
    ("small", 300, 256, 128, 16, 2, 128, 256),
    ("ragged", 203, 192, 256, 24, 5, 384, 0),
    ("replica-widths", 1000, 1024, 256, 256, 6, 512, 2048),
    ("deep", 4096, 256, 128, 8, 2, 128, 0),          # 1024 rows per expert: block-wide tile tables
    ("long", 65600, 128, 128, 16, 2, 128, 0),        # 2050 chunks: the per-block scatter copies the scale rows
]


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("case", SHAPES, ids=[c[0] for c in SHAPES])
def test_mxfp8_weights_and_forward_match_oracle(case, fmt):
    name, T, d, l, E, k, f, f_s = case
    say(f"{fmt} {name}: T={T} d={d} l={l} E={E} k={k} f={f} f_s={f_s}")
    shape = wl.LayerShape(name, 31, "bf16", T=T, d=d, l=l, E=E, k=k, f=f, f_s=f_s, B=256)
    W = wl.make_weights(shape)
    layer = make_layer(shape, W, max_tokens=T, experts=fmt)
    torch.cuda.synchronize()
    q, sc = _state_mx(layer, shape, fmt)
    wq = FORMATS[fmt][1]
    rw = _wround(fmt)
    for i, n in enumerate(("W_g", "W_u", "W_d")):
        rq, rs = wq(W[n].reshape(-1, W[n].shape[-1]))
        np.testing.assert_array_equal(sc[i], rs.reshape(-1), err_msg=n)
        np.testing.assert_array_equal(q[i], rq.reshape(-1), err_msg=n)
    x = wl.make_x(shape)
    r = layer.route_buffers(T)
    out = layer.forward(x_on_gpu(x, layer), route=r)
    torch.cuda.synchronize()
    lg = to_np(r["logits"])
    ref = o.forward(x, W, np.zeros(E, F32), k=k, dtype="bf16", eps=shape.rms_eps, logits=lg, experts=fmt)
    assert_routing_equal(r, ref, T)
    v = layer.ws_views(T)
    z, H, Y = to_np(v["z"]).astype(np.float64), to_np(v["H"]).astype(np.float64), to_np(v["Y"]).astype(np.float64)
    assert rel_err(z, ref["z"]) <= OUT_TOL["bf16"]
    # quantisation of the activations: bit-exact given the same bf16 input
    _check_quant(to_np(v["z8"])[:T * l], to_np(v["zs"])[:T * l // 32], z)
    _check_quant(to_np(v["H8"])[:T * k * f], to_np(v["Hs"])[:T * k * f // 32], H)
    # each expert GEMM against the oracle on the GPU's own input (stage by stage)
    offs = ref["offsets"]
    H_ref = np.zeros_like(H)
    Y_ref = np.zeros_like(Y)
    Xq = o.mx_round(z[ref["perm_src"]])
    for e in range(E):
        a, b = int(offs[e]), int(offs[e + 1])
        if a < b:
            H_ref[a:b] = o.bf16_round(o.glu(Xq[a:b], rw(W["W_g"][e]), rw(W["W_u"][e])))
            Y_ref[a:b] = o.bf16_round(o.mx_round(H[a:b]) @ rw(W["W_d"][e]).T)
    for n, got, want in (("H", H, H_ref), ("Y", Y, Y_ref)):
        err = rel_err(got, want)
        say(f"  {n} (on the GPU's input) rel err {err:.3e}")
        assert err <= OUT_TOL["bf16"], n
    # end to end against the oracle's own chain: a 1-ulp bf16 difference in z or
    # H can move an element to the next E4M3 value (a 2^-3 relative step), so
    # the bound is looser than the bf16 layer's
    for n in ("H", "Y", "y_lat"):
        say(f"  {n} end-to-end rel err {rel_err(to_np(v[n]), ref[n]):.3e}")
    e2e = rel_err(to_np(out), ref["out"])
    say(f"  out end-to-end rel err {e2e:.3e}")
    assert e2e <= MX_E2E_TOL
    ref_bf = o.forward(x, W, np.zeros(E, F32), k=k, dtype="bf16", eps=shape.rms_eps, logits=lg)
    say(f"  vs bf16 experts {rel_err(ref['out'], ref_bf['out']):.3e}")
    layer.close()


def _check_quant(q8, qs, a):
    rq, rs = o.mx_quantize(a)
    np.testing.assert_array_equal(qs.astype(np.int64), rs.reshape(-1))
    np.testing.assert_array_equal(_e4m3_values(q8), rq.reshape(-1))


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_mxfp8_replica_full_and_requantize(fmt):
    """Full replica size (T=8192): routing bit-exact and every element of the
    output within the end-to-end bound; moe_requantize_experts after changing
    W_d picks up the change."""
    shape = wl.workload("replica")
    T = shape.T
    say(f"{fmt} replica T={T}")
    W = wl.make_weights(shape)
    layer = make_layer(shape, W, max_tokens=T, experts=fmt)
    x = wl.make_x(shape)
    r = layer.route_buffers(T)
    out = layer.forward(x_on_gpu(x, layer), route=r)
    torch.cuda.synchronize()
    zero = np.zeros(shape.E, F32)
    compare_full(shape, W, x, to_np(r["logits"]), r, out, layer.ws_views(T), zero, experts=fmt, names=("h", "z"),
                 out_tol=MX_E2E_TOL)
    layer.w["W_d"].mul_(2)                                   # exact in bf16 and in MX formats (scale + 1)
    Bd.moe_requantize_experts(layer.ctx, torch.cuda.current_stream().cuda_stream)
    out2 = layer.forward(x_on_gpu(x, layer), route=r)
    torch.cuda.synchronize()
    W2 = dict(W, W_d=W["W_d"] * 2)
    compare_full(shape, W2, x, to_np(r["logits"]), r, out2, layer.ws_views(T), zero, experts=fmt, names=(),
                 out_tol=MX_E2E_TOL)
    layer.close()


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_block_scaled_forward_graph_replay(fmt):
    """The block-scaled forward (activation quantisation, fused H
    quantisation) + qb_update captured in a graph: every replay equals the
    eager result bit for bit."""
    shape = wl.workload("replica", 2048)
    T = shape.T
    say(f"{fmt} graph replay T={T}")
    W = wl.make_weights(shape)
    layer = make_layer(shape, W, max_tokens=T, experts=fmt)
    xt = x_on_gpu(wl.make_x(shape), layer)
    r = layer.route_buffers(T)
    out = torch.empty(T, shape.d, dtype=layer.tdtype, device="cuda")
    for _ in range(2):                                   # bias 0, then the converged QB bias
        layer.forward(xt, out=out, route=r)
        layer.qb_update()
    torch.cuda.synchronize()
    want, bias = out.clone(), layer.get_bias().clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward(xt, out=out, route=r)
        layer.qb_update()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(xt, out=out, route=r)
        layer.qb_update()
    for i in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), i
        assert torch.equal(layer.get_bias(), bias), i
        _ = (xt.float() * 2).sum().item()
    layer.close()
