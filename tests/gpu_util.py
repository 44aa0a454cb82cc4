"""Helpers of the GPU parity tests: build a layer on the GPU from a seeded
workload, run it through the C ABI, and compare with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import moe_oracle as o
from sparse_moe_layer_rmsnorm_amd import workloads as wl
from sparse_moe_layer_rmsnorm_amd.layer import layer_from_shape

F32 = np.float32

# max|GPU - oracle| / max|oracle| bounds of the layer output
OUT_TOL = {"f32": 1e-4, "bf16": 2e-2}
# router logits against the oracle's own logits (before injection)
LOGIT_TOL = {"f32": 1e-5, "bf16": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.abs(want).max()
    return float(np.abs(got - want).max() / (den if den > 0 else 1.0))


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def make_layer(shape, W, *, max_tokens, c=None, frozen=None, **kw):
    return layer_from_shape(shape, W, max_tokens=max_tokens, logit_offset=c, frozen=frozen, **kw)


def x_on_gpu(x: np.ndarray, layer) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).cuda().to(layer.tdtype)


def assert_routing_equal(r_gpu: dict, ref: dict, T: int) -> None:
    np.testing.assert_array_equal(to_np(r_gpu["topk_idx"]), ref["idx"])
    np.testing.assert_array_equal(to_np(r_gpu["gates"]).view(np.uint32), ref["gates"].view(np.uint32))
    np.testing.assert_array_equal(to_np(r_gpu["counts"]), ref["counts"])
    np.testing.assert_array_equal(to_np(r_gpu["offsets"]), ref["offsets"])
    np.testing.assert_array_equal(to_np(r_gpu["perm_src"]), ref["perm_src"])
    np.testing.assert_array_equal(to_np(r_gpu["inv"]), ref["inv"])


def oracle_routing(logits: np.ndarray, bias: np.ndarray, k: int, E: int, B: int, routed_scale: float = 1.0):
    s = o.sigmoid_r(logits)
    idx = o.topk_select(s, bias, k)
    g = o.gates_from(s, idx, routed_scale)
    counts, offsets, perm_src, inv = o.permutation(idx, E)
    return {"s": s, "idx": idx, "gates": g, "counts": counts, "offsets": offsets, "perm_src": perm_src,
            "inv": inv, "hist": o.histogram(s, B)}


def stored_intermediates(shape, views):
    """The intermediates a forward left in its workspace: h, z, G (with a
    shared expert), H (unless the experts ran fused, keeping H on chip), Y,
    y_lat."""
    return ("h", "z") + (("G",) if shape.f_s else ()) + (("H",) if views["H"].numel() else ()) + ("Y", "y_lat")


def compare_full(shape, W, x, lg, r_gpu, out_gpu, views, bias, *, experts="bf16", with_hist=False,
                 out_tol=None, names=None):
    """Whole-batch parity: the oracle's full forward with the GPU's logits
    injected.  The GPU logits are checked against the oracle's own router
    output on its own h (tolerance); routing is compared bit for bit; every
    element of the stored intermediates (h, z, G, H, Y, y_lat) and of out is
    compared within the layer tolerance.  Returns the oracle's forward and the
    errors."""
    T = x.shape[0]
    ref = o.forward(x, W, np.asarray(bias, F32), k=shape.k, dtype=shape.dtype, eps=shape.rms_eps, B=shape.B,
                    logits=lg, with_hist=with_hist, experts=experts)
    errs = {"logits": rel_err(lg, o.router_logits(ref["h"], W["W_r"], W.get("c")))}
    say(f"  logits rel err {errs['logits']:.3e}")
    assert errs["logits"] <= LOGIT_TOL[shape.dtype]
    assert_routing_equal(r_gpu, ref, T)
    tol = OUT_TOL[shape.dtype]
    if names is None:
        names = stored_intermediates(shape, views)
    for name in names:  # intermediates first: a failure names the first wrong step
        errs[name] = rel_err(to_np(views[name]), ref[name])
        say(f"  {name} rel err {errs[name]:.3e} ({ref[name].size} elements)")
        assert errs[name] <= tol, name
    errs["out"] = rel_err(to_np(out_gpu), ref["out"])
    say(f"  out rel err {errs['out']:.3e} ({ref['out'].size} elements)")
    assert errs["out"] <= (tol if out_tol is None else out_tol)
    return ref, errs
