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
    (384, 8, 1500, 1.0, 0.05),     # 8 columns per lane
    (8, 8, 130, 1.0, 0.0),         # k = E
    (64, 1, 1, 1.0, 0.0),          # one token
    (1024, 32, 700, 1.0, 0.01),    # largest E and k
    (256, 6, 16384, 1.0, 0.05),    # 32 super-chunks: the scan splits each expert's over 4 threads
    (48, 3, 30000, 1.5, 0.1),      # 59 super-chunks over 16 threads per expert, one part empty
    (256, 6, 2000, 1.0, 300.0),    # |b| >> s: v = s + b spaced by ulps of a few hundred, many negative
    (896, 16, 1000, 1.0, 40.0),
    (256, 6, 65569, 1.0, 0.05),    # 2050 chunks: the per-block scatter, its last block 2 chunks, a 1-token chunk
    (100, 4, 70001, 1.0, 0.1),     # the per-block scatter with E < 256 (threads without an expert)
    (128, 12, 65601, 1.0, 0.05),   # the per-block scatter with more slots than its prefetched indices
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


def test_fast_score_error_bound():
    """The routing kernels filter with a fast router score (hardware exp2 and
    reciprocal) and compute the exact one only where a decision could depend
    on it; that is exact only while |fast - exact| <= MOE_FAST_SCORE_ERR for
    every fp32 logit, which the library measures over all 2^32 of them."""
    say("fast score error over all fp32 logits")
    from sparse_moe_layer_rmsnorm_amd import binding as B
    err = torch.full((4,), -1.0, dtype=torch.float32, device="cuda")
    B.moe_fast_score_error(err.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    e = float(err[0].item())
    say(f"  max |fast - exact| = {e:.3e} (bound {B.MOE_FAST_SCORE_ERR:.3e})")
    assert 0.0 <= e <= B.MOE_FAST_SCORE_ERR


NEAR_TIE_CASES = [  # (E, k, T, kind)
    (896, 16, 512, "cluster"),   # K3 routing shape
    (256, 6, 1024, "cluster"),   # replica shape
    (256, 6, 1024, "tight"),     # replica shape, cluster of k + 4: ranked among at most 16 candidates
    (128, 8, 700, "tight"),
    (256, 6, 20000, "tight"),    # more than 512 chunks: 16 lanes per token
    (128, 8, 17000, "equal"),
    (100, 7, 257, "cluster"),    # E not a multiple of 64, ragged chunk
    (500, 12, 700, "cluster"),   # 8 columns per lane
    (256, 6, 300, "equal"),      # every expert a candidate: more than 64
    (896, 16, 65, "equal"),
    (64, 8, 256, "equal"),       # 64 candidates, all tied
    (256, 6, 512, "coarse"),     # logits on a grid of 1/4: many exact ties
]


@pytest.mark.parametrize("E,k,T,kind", NEAR_TIE_CASES)
def test_route_near_ties_bitexact(E, k, T, kind):
    """Scores closer together than the fast score resolves.  "cluster": per
    token 2k + 8 random experts get logits within 3 fp32 ulps of 2.0, above
    the rest, so the top-k cut falls inside the cluster and only the exact
    scores (and the lower index on exact ties) order it ("tight": k + 4 such
    experts, few enough for the 16-lane row layout); "equal": half the
    rows hold one logit everywhere (the exact ranking sees every expert);
    "coarse": logits rounded to quarters.  Routing must still equal the
    oracle's bit for bit."""
    say(f"near ties E={E} k={k} T={T} {kind}")
    rng = np.random.default_rng(E * 3 + T)
    logits = (rng.standard_normal((T, E)) * 0.5).astype(F32)
    bias = np.zeros(E, F32)
    if kind in ("cluster", "tight"):
        n = min(E, 2 * k + 8 if kind == "cluster" else k + 4)
        base = np.array([2.0], F32).view(np.int32)[0]
        for t in range(T):
            sel = rng.choice(E, size=n, replace=False)
            logits[t, sel] = (base + rng.integers(-3, 4, n).astype(np.int32)).view(F32)
    elif kind == "equal":
        logits[::2] = F32(0.75)
        bias = (rng.standard_normal(E) * 0.05).astype(F32)
        bias[:] = bias[0]                      # equal biases keep the rows tied
    else:
        logits = (np.round(logits * 4) / 4).astype(F32)
    shape = _shape(E, k)
    layer = make_layer(shape, wl.make_weights(shape), max_tokens=T)
    layer.set_bias(bias)
    r = layer.route(T, logits=torch.from_numpy(logits).cuda())
    torch.cuda.synchronize()
    ref = oracle_routing(logits, bias, k, E, shape.B)
    assert_routing_equal(r, ref, T)
    np.testing.assert_array_equal(to_np(layer.state_views()["hist"]), ref["hist"])
    layer.close()


@pytest.mark.parametrize("lo,hi,B", [(0.0, 1.0, 256), (0.3, 0.9, 100)])
def test_histogram_at_bin_edges_bitexact(lo, hi, B):
    """Scores within a few ulps of every bin edge, where the fast score cannot
    place them and the exact score must decide: the histogram must equal the
    oracle's bit for bit."""
    say(f"histogram bin edges [{lo}, {hi}] B={B}")
    E, k = 64, 2
    p = lo + (hi - lo) * np.arange(1, B) / B
    p = p[(p > 0) & (p < 1)]
    l0 = np.log(p / (1 - p)).astype(F32)
    cols, up, down = [l0], l0, l0
    for _ in range(6):                         # the 6 fp32 neighbours on each side
        up, down = np.nextafter(up, F32(np.inf)), np.nextafter(down, F32(-np.inf))
        cols += [up, down]
    vals = np.stack(cols, axis=1).ravel()
    T = -(-vals.size // E)
    rng = np.random.default_rng(B)
    logits = rng.permutation(np.resize(vals, T * E)).reshape(T, E).astype(F32)
    shape = _shape(E, k, B=B)
    layer = make_layer(shape, wl.make_weights(shape), max_tokens=T, qb_lo=lo, qb_hi=hi)
    r = layer.route(T, logits=torch.from_numpy(logits).cuda())
    torch.cuda.synchronize()
    ref = oracle_routing(logits, np.zeros(E, F32), k, E, B)
    assert_routing_equal(r, ref, T)
    np.testing.assert_array_equal(to_np(layer.state_views()["hist"]), o.histogram(ref["s"], B, lo, hi))
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


@pytest.mark.parametrize("lo,hi,B", [(0.25, 0.75, 256), (0.3, 0.9, 100), (-1.0, 2.0, 7)])
def test_qb_histogram_over_a_score_range(lo, hi, B):
    """The histogram over [qb_lo, qb_hi] (scores beyond it in the end bins)
    and the quantile mapped back onto that range: bit-exact with the oracle."""
    say(f"qb range [{lo}, {hi}] B={B}")
    E, k, T = 40, 4, 3000
    rng = np.random.default_rng(B)
    shape = _shape(E, k, B=B)
    layer = make_layer(shape, wl.make_weights(shape), max_tokens=T, qb_lo=lo, qb_hi=hi)
    logits = (rng.standard_normal((T, E)) * 0.6 + rng.standard_normal(E)[None, :] * 0.3).astype(F32)
    r = layer.route(T, logits=torch.from_numpy(logits).cuda())
    torch.cuda.synchronize()
    ref = oracle_routing(logits, np.zeros(E, F32), k, E, B)
    assert_routing_equal(r, ref, T)
    want = o.histogram(ref["s"], B, lo, hi)
    np.testing.assert_array_equal(to_np(layer.state_views()["hist"]), want)
    layer.qb_update()
    torch.cuda.synchronize()
    b = o.qb_update(want, T, k, np.zeros(E, F32), lo, hi)
    np.testing.assert_array_equal(to_np(layer.get_bias()).view(np.uint32), b.view(np.uint32))
    layer.close()


@pytest.mark.parametrize("balancer", ["qb", "sign"])
def test_window_overflow_guard_on_the_device(balancer):
    """A statistics window past 2^32 - 1 tokens that the host did not see (as
    under graph replay, emulated by writing the device count directly): the
    update keeps the bias, marks every q_e NaN (QB) and clears the window."""
    say(f"window overflow guard ({balancer})")
    E, k, T = 32, 4, 256
    shape = _shape(E, k)
    layer = make_layer(shape, wl.make_weights(shape), max_tokens=T, balancer=balancer)
    b0 = (np.random.default_rng(2).standard_normal(E) * 0.1).astype(F32)
    layer.set_bias(b0)
    st = layer.state_views()
    st["count"].fill_(2 ** 32 - 100)                # tokens the host mirror never counted
    logits = np.random.default_rng(4).standard_normal((T, E)).astype(F32)
    layer.route(T, logits=torch.from_numpy(logits).cuda())
    torch.cuda.synchronize()
    assert int(st["count"].item()) == 2 ** 32 - 100 + T
    layer.qb_update()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(layer.get_bias()).view(np.uint32), b0.view(np.uint32))
    assert int(st["count"].item()) == 0
    assert int(st["hist_slices"].abs().sum().item()) == 0 and int(st["load"].abs().sum().item()) == 0
    if balancer == "qb":
        assert np.all(np.isnan(to_np(st["q"])))
    # the next window starts clean: an ordinary update works again
    r = layer.route(T, logits=torch.from_numpy(logits).cuda())
    layer.qb_update()
    torch.cuda.synchronize()
    ref = oracle_routing(logits, b0, k, E, shape.B)
    assert_routing_equal(r, ref, T)
    if balancer == "qb":
        want = o.qb_update(ref["hist"], T, k, b0)
    else:
        want = o.sign_update(ref["counts"], b0, 1e-2)
    np.testing.assert_array_equal(to_np(layer.get_bias()).view(np.uint32), want.view(np.uint32))
    layer.close()
