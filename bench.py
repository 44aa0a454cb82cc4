"""Benchmark: Stable LatentMoE layer forward + QB update on one MI355X.

One step = one training forward of the whole layer (RMSNorm, router, scores,
QB histogram, biased top-k, gates, permutation, shared GLU, experts, combine,
up-projection) over a batch of synthetic tokens, followed by the QB bias
update.  Inputs and weights are resident in HBM before timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload replica]

Prints one JSON line: tokens/s over the K timed steps, the per-kernel times
(HIP events on the launch stream, inside the timed region), the roofline
position of the dominant kernel and of the expert GEMMs / routing kernels, and
the CPU oracle's tokens/s on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
from sparse_moe_layer_rmsnorm_amd.profsum import source_hash  # noqa: E402

METRIC = "MoE-layer fwd tokens/sec on 1 MI355X + % bf16 MFMA peak + routing GB/s"
METRIC_BWD = "MoE-layer fwd+bwd tokens/sec on 1 MI355X (training step: forward, backward, bias update)"


def kernel_work(s, T: int) -> dict:
    """Algorithmic work per launch: FLOPs of the GEMMs, and bytes of the
    memory-bound kernels counted as the layer's own data (each operand read
    once, each result written once), not as the buffers an implementation
    chooses to keep.  Routing bytes follow the per-token figures of the
    routing, permutation and combine steps (scores and top-k read the fp32
    logits and write indices and gates, 4E + 8k per token, plus the E x B
    histogram once; counts, offsets and the stable permutation 16k per token;
    combine 2kl + 8k + 2l per token in bf16)."""
    es = 2 if s.dtype == "bf16" else 4
    Tk = T * s.k
    flops = {
        "gemm_h": 2.0 * T * s.d * (s.E + 2 * s.f_s + s.l),
        "gemm_rz": 2.0 * T * s.d * s.E,
        "gemm_out": 2.0 * T * s.d * (s.f_s + s.l),
        "expert_up": 2.0 * Tk * s.l * 2 * s.f,
        "expert_down": 2.0 * Tk * s.f * s.l,
    }
    bytes_ = {
        "rmsnorm": 2.0 * T * s.d * es + 4 * s.d,
        "topk": 4.0 * T * s.E + 8.0 * Tk + 4.0 * s.E * s.B,
        # count + prefix sum + stable scatter: 16 bytes per (token, slot) in all
        "scan": 4.0 * Tk,
        "scatter": 12.0 * Tk,
        "combine": 1.0 * Tk * s.l * es + 8.0 * Tk + 1.0 * T * s.l * es,
        # read and clear the histogram, write q and the bias
        "qb_update": 8.0 * s.E * s.B + 12.0 * s.E,
        # MXFP8 quantisation of z and H (one launch each): read bf16, write bytes + scales
        "mx_quant": 0.5 * (2.0 + 1.0 + 1.0 / 32) * (T * s.l + Tk * s.f),
        "sign_bias": 16.0 * s.E,
    }
    # bytes the implementation moves beyond those: the histogram's atomic
    # adds from its token parts (32 where the top-k runs 512-thread blocks: a
    # token per 16 lanes, E <= 256, k <= 8, more than 512 chunks; 16 with a
    # token per 32 lanes, E <= 512, k <= 16; else 8), the per-chunk selection
    # masks and the per-super-chunk counts
    nchunks = (T + 31) // 32
    nsuper = (nchunks + 15) // 16
    if s.E <= 256 and s.k <= 8 and nchunks > 512:
        parts = 32
    elif s.E <= 512 and s.k <= 16:
        parts = 16
    else:
        parts = 8
    impl_extra = {
        "topk": 8.0 * parts * s.E * s.B + 4.0 * nchunks * s.E + 8.0 * nsuper * s.E,
        "scan": 8.0 * nsuper * s.E,
        "scatter": 4.0 * 8 * Tk,
    }
    return {"flops": flops, "bytes": bytes_, "impl_extra": impl_extra}


def gemm_groups(s, T: int) -> dict:
    """FLOPs and minimum HBM bytes of each GEMM group (weights, inputs and
    outputs once): the h GEMM, the routed experts (with the expert hidden H
    kept on chip: weights, dispatched rows in, expert rows out) and the output
    GEMM."""
    es = 2 if s.dtype == "bf16" else 4
    Tk = T * s.k
    return {
        "gemm_h": (2.0 * T * s.d * (s.E + 2 * s.f_s + s.l),
                   es * (T * s.d + s.d * (s.E + 2 * s.f_s + s.l) + T * (s.f_s + s.l)) + 4.0 * T * s.E),
        "experts": (2.0 * Tk * s.l * 3 * s.f, es * (3.0 * s.E * s.f * s.l + 2.0 * Tk * s.l)),
        "gemm_out": (2.0 * T * s.d * (s.f_s + s.l), es * (T * (s.f_s + s.l) + s.d * (s.f_s + s.l) + T * s.d)),
    }


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def backward_flops(s, T: int, keep: bool = False) -> dict:
    """GEMM FLOPs of one backward pass per launch group (0: memory-bound
    groups): the dense products (shared pre-activations recomputed unless the
    forward kept them, the output-projection transposes, dh), the grouped
    expert products (dH, A and U recomputed unless kept, dX) and the weight
    gradients (per expert, and the two dense ones split along the tokens)."""
    Tk = T * s.k
    Kc = 2 * s.f_s + s.l + (s.E + 63) // 64 * 64
    rec = 0 if keep else 1
    dense = rec * 2.0 * T * s.d * (2 * s.f_s) + 2.0 * T * s.d * (s.f_s + s.l) + 2.0 * T * Kc * s.d
    expert = 2.0 * Tk * s.l * s.f * (1 + 2 * rec) + 2.0 * Tk * 2 * s.f * s.l
    # weight gradients: the per-expert ones and the two split-K dense ones
    wgrad = 2.0 * Tk * s.l * s.f + 2.0 * Tk * 2 * s.f * s.l + 2.0 * s.d * T * (s.f_s + s.l) + 2.0 * Kc * T * s.d
    return {"bwd_gemm": dense, "bwd_expert": expert, "bwd_wgrad": wgrad, "bwd_eltwise": 0.0}


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash():
        return None
    return t.get("kernels", {}).get(workload, {}).get(kernel)


def cpu_baseline(shape, W, x, seconds: float = 12.0) -> dict:
    """The CPU oracle (as it is) on a bounded sample of the same workload:
    full training forward + QB update on the first T_s tokens, repeated until
    about `seconds` of CPU time."""
    from oracle import moe_oracle as o
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    Ts = min(shape.T, 1024)
    xs = x[:Ts]
    b = np.zeros(shape.E, np.float32)
    reps, t0 = 0, time.perf_counter()
    while True:
        r = o.forward(xs, W, b, k=shape.k, dtype=shape.dtype, eps=shape.rms_eps, B=shape.B)
        o.qb_update(r["hist"], Ts, shape.k, b)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 50:
            break
    res = {"value": reps * Ts / el, "unit": "tokens/s", "cores": int(cores), "cpu_model": host_cpu_model(),
           "kind": "oracle",
           "sample": f"{reps} x full training forward + QB update of the first {Ts} tokens of the {shape.name} "
                     f"workload (numpy fp64, {el:.1f} s)"}
    # the same sample on one host thread, about a third of the time budget
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            r1, t1 = 0, time.perf_counter()
            while True:
                r = o.forward(xs, W, b, k=shape.k, dtype=shape.dtype, eps=shape.rms_eps, B=shape.B)
                o.qb_update(r["hist"], Ts, shape.k, b)
                r1 += 1
                e1 = time.perf_counter() - t1
                if e1 >= seconds / 3 or r1 >= 20:
                    break
        res["value_1_thread"] = r1 * Ts / e1
    except Exception:
        pass
    return res


def cold_forward(layer, x, out, stream, n: int) -> dict:
    """Forward time with the 256 MB MALL flushed first: before each of n
    forwards a 512 MB buffer is written; events bracket the forward alone."""
    import torch
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    ms = []
    for _ in range(n):
        scratch.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        layer.forward(x, out=out)
        e1.record(stream)
        layer.qb_update()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    del scratch
    ms.sort()
    med = ms[len(ms) // 2]
    return {"ms_per_forward_median": round(med, 5), "tokens_per_s": round(x.shape[0] / (med / 1e3), 1),
            "forwards": n, "flush": "512 MB device write before each forward"}


def balance_record(layer, shape, steps: int) -> list:
    """Per-step expert load balance of a training loop that starts from a
    zero bias (fresh x each step, the bias of each step set by the previous
    step's update): max/min and max/mean of the tokens per expert and the
    number of experts with none.  Runs outside the timed region; the layer's
    bias is restored afterwards."""
    import torch
    from sparse_moe_layer_rmsnorm_amd import workloads as wl
    bias0 = layer.get_bias().clone()
    layer.set_bias(torch.zeros_like(bias0))
    T = shape.T
    r = layer.route_buffers(T)
    out = torch.empty(T, shape.d, dtype=layer.tdtype, device="cuda")
    rows = []
    for step in range(steps):
        x = torch.from_numpy(wl.make_x(shape, step)).cuda().to(layer.tdtype)
        layer.forward(x, out=out, route=r)
        layer.qb_update()
        n = r["counts"].double()
        rows.append({"step": step, "max_over_min": round(float(n.max() / n.min()), 3) if n.min() > 0 else None,
                     "max_over_mean": round(float(n.max() / n.mean()), 3), "dead": int((n == 0).sum())})
    layer.set_bias(bias0)
    torch.cuda.synchronize()
    return rows


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="replica")
    ap.add_argument("--tokens", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--graph", action="store_true",
                    help="replay the step as a captured HIP graph (per-kernel times then come from an extra "
                         "eager pass after the timed region)")
    ap.add_argument("--no-profile", action="store_true", help="no per-kernel events in the timed region")
    ap.add_argument("--balancer", choices=("qb", "sign"), default="qb",
                    help="bias update rule of the step: quantile balancing (default) or the sign rule")
    ap.add_argument("--experts", choices=("bf16", "mxfp8", "mxfp4"), default="bf16",
                    help="storage of the routed experts' operands (MXFP8: E4M3 + E8M0 block scales; MXFP4: E2M1 "
                         "weights + E8M0 block scales against MXFP8 activations)")
    ap.add_argument("--backward", action="store_true",
                    help="time the training step with the backward pass: forward, moe_backward (dx and all weight "
                         "gradients) and the bias update")
    ap.add_argument("--keep-preact", action="store_true",
                    help="the forward also stores the GLU pre-activations (keep_preact) and the backward reads them "
                         "instead of recomputing them")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain device copy of 256 MiB (the reference for HBM byte counters)")
    ap.add_argument("--balance-steps", type=int, default=None,
                    help="training steps of the per-step load-balance record (default: 20 for the load-skew "
                         "workload, 3 for the other training workloads)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the layer is built and measured per GPU); --gpus {args.gpus} "
              "is not supported", file=sys.stderr)
        return 2

    import torch
    from sparse_moe_layer_rmsnorm_amd import binding as B
    from sparse_moe_layer_rmsnorm_amd import workloads as wl
    from sparse_moe_layer_rmsnorm_amd.layer import layer_from_shape

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    B.lib()  # fail loudly if the HIP library is missing
    shape = wl.workload(args.workload, args.tokens)
    T = shape.T
    W = wl.make_weights(shape)
    x_np = wl.make_x(shape)
    c = wl.zipf_logit_offset(shape) if shape.name == "skew" else None
    frozen = shape.qb_frozen
    layer = layer_from_shape(shape, W, max_tokens=T, logit_offset=c, frozen=frozen, balancer=args.balancer,
                             experts=args.experts, keep_preact=args.keep_preact)
    if frozen:
        layer.set_bias(wl.frozen_bias(shape))
    x = torch.from_numpy(x_np).cuda().to(layer.tdtype)
    out = torch.empty(T, shape.d, dtype=layer.tdtype, device="cuda")
    stream = torch.cuda.current_stream()
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    grads = None
    if args.backward:
        dout = torch.randn(T, shape.d, generator=torch.Generator().manual_seed(7)).cuda().to(layer.tdtype)
        layer.forward(x, out=out)
        _, grads = layer.backward(x, dout)

    def step():
        layer.forward(x, out=out)
        if args.backward:
            layer.backward(x, dout, grads=grads)
        layer.qb_update()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Per-kernel times: one pass of K steps with every launch bracketed by HIP
    # events on the launch stream (outside the timed region: 24 events a step
    # would add their own cost to it).
    B.moe_profile_begin(layer.ctx, 64 * args.steps + 64)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = B.moe_profile_end(layer.ctx)
    # the roofline object describes the forward's dominant kernel
    dom = max((n for n in prof if prof[n][1] and not n.startswith("bwd_")), key=lambda n: prof[n][0])
    run = step
    if args.graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        for _ in range(3):
            g.replay()
        run = g.replay
    # Timed region: K steps; the dominant kernel's launches alone are bracketed
    # by events (its roofline position is measured live here).
    live = not (args.graph or args.no_profile)
    if live:
        B.moe_profile_begin(layer.ctx, args.steps + 4, [dom])
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        run()
    ev1.record(stream)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    if live:
        prof_dom = B.moe_profile_end(layer.ctx)[dom]
    else:
        prof_dom = prof[dom]
    ms_step = total_ms / args.steps
    tok_s = T / (ms_step / 1e3)
    cold = cold_forward(layer, x, out, stream, min(args.steps, 20)) if not args.backward else None

    work = kernel_work(shape, T)
    peak_mm = PEAK_BF16_TFLOPS if shape.dtype == "bf16" else PEAK_F32_TFLOPS
    kernels = {}
    for name, (ms, n) in prof.items():
        if n == 0:
            continue
        avg_us = ms / n * 1e3
        k = {"avg_us": round(avg_us, 3), "launches": int(n)}
        if name in work["flops"]:
            tf = work["flops"][name] / (avg_us * 1e-6) / 1e12
            k.update(tflops=round(tf, 1), mfma_frac=round(tf / peak_mm, 4))
        elif name in work["bytes"]:
            gbs = work["bytes"][name] / (avg_us * 1e-6) / 1e9
            k.update(gbs=round(gbs, 1), hbm_frac=round(gbs / PEAK_HBM_GBS, 4))
        kernels[name] = k
    dom_us = prof_dom[0] / prof_dom[1] * 1e3
    traffic = traffic_for(dom, shape.name)
    if dom in work["flops"]:
        ach = work["flops"][dom] / (dom_us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "achieved": round(ach, 1), "peak": peak_mm, "unit": "TFLOP/s",
                    "frac": round(ach / peak_mm, 4), "traffic": traffic, "kernel": dom,
                    "avg_us": round(dom_us, 3), "algorithmic": f"{work['flops'][dom]:.6g} FLOP per launch"}
    else:
        ach = work["bytes"][dom] / (dom_us * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic, "kernel": dom,
                    "avg_us": round(dom_us, 3), "algorithmic": f"{work['bytes'][dom]:.6g} bytes per launch"}
    # expert GEMMs together, and routing + permutation + combine together
    ex_names = [n for n in ("expert_up", "expert_down") if n in kernels]
    ex_us = sum(kernels[n]["avg_us"] for n in ex_names)
    ex_tf = (work["flops"]["expert_up"] + work["flops"]["expert_down"]) / (ex_us * 1e-6) / 1e12
    rt_names = [n for n in ("topk", "scan", "scatter", "combine") if n in kernels]
    rt_us = sum(kernels[n]["avg_us"] for n in rt_names)
    rt_bytes = sum(work["bytes"].get(n, 0.0) for n in rt_names)
    rt_impl = sum(work["impl_extra"].get(n, 0.0) for n in rt_names)
    # each GEMM group against the roof that applies to it: the larger of its
    # time at the MFMA peak and its time at the HBM peak, over its time
    groups = gemm_groups(shape, T)
    group_us = {"gemm_h": kernels.get("gemm_h", {}).get("avg_us"), "experts": ex_us or None,
                "gemm_out": kernels.get("gemm_out", {}).get("avg_us")}
    roofs = {}
    for g, (fl, by) in groups.items():
        us = group_us[g]
        if not us:
            continue
        t_mm, t_hbm = fl / (peak_mm * 1e12), by / (PEAK_HBM_GBS * 1e9)
        roofs[g] = {"us": round(us, 3), "gflop": round(fl / 1e9, 2), "min_mbytes": round(by / 1e6, 1),
                    "bound": "mfma" if t_mm >= t_hbm else "hbm",
                    "roof_us": round(max(t_mm, t_hbm) * 1e6, 2),
                    "frac_of_roof": round(max(t_mm, t_hbm) / (us * 1e-6), 4),
                    "mfma_frac": round(fl / (us * 1e-6) / 1e12 / peak_mm, 4)}
    # GEMM FLOPs of one step: the launched forward GEMMs (plus the backward's)
    layer_flops = sum(work["flops"][n] * kernels[n]["launches"] / args.steps for n in kernels if n in work["flops"])
    if args.backward:
        layer_flops += sum(backward_flops(shape, T, args.keep_preact).values())

    bwd = None
    if args.backward:
        bf = backward_flops(shape, T, args.keep_preact)
        bwd = {}
        for n, fl in bf.items():
            ms, cnt = prof.get(n, (0.0, 0))
            if cnt:
                us = ms / args.steps * 1e3
                bwd[n] = {"us_per_step": round(us, 2), "launches_per_step": cnt // args.steps}
                if fl:
                    bwd[n].update(tflops=round(fl / (us * 1e-6) / 1e12, 1),
                                  mfma_frac=round(fl / (us * 1e-6) / 1e12 / peak_mm, 4))
    res = {
        "metric": METRIC_BWD if args.backward else METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.dtype,
        "data": "synthetic: seeded PCG64, x ~ N(0,1), weights ~ N(0,1/fan_in), rounded to bf16; random init",
        "timing": ("graph replay" if args.graph else "eager") + (
            "; dominant kernel bracketed by HIP events in the timed region" if live else "") +
            "; per-kernel table from a separate profiled pass of the same K steps",
        "config": {"workload": f"{shape.name}: T={T} tokens, d={shape.d}, l={shape.l}, E={shape.E}, k={shape.k}, "
                               f"f={shape.f}, f_s={shape.f_s}, B={shape.B}, QB {'frozen' if frozen else 'train'}"
                               + (", sign-rule balancer" if args.balancer == "sign" else "")
                               + {"bf16": "", "mxfp8": ", MXFP8 experts",
                                  "mxfp4": ", MXFP4 expert weights with MXFP8 activations"}[args.experts]
                               + (", GLU pre-activations kept by the forward" if args.keep_preact else ""),
                   "global_batch": T,
                   "step": "training forward + backward + qb_update" if args.backward else
                           "training forward + qb_update"},
        "roofline": roofline,
        "layer_mfma_frac": round(layer_flops / (ms_step * 1e-3) / 1e12 / peak_mm, 4),
        "expert_gemm": {"tflops": round(ex_tf, 1), "mfma_frac": round(ex_tf / peak_mm, 4)},
        "gemm_roofs": roofs,
        "routing_permute_combine": {"gbs": round(rt_bytes / (rt_us * 1e-6) / 1e9, 1),
                                    "hbm_frac": round(rt_bytes / (rt_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                                    "us": round(rt_us, 2), "kernels": rt_names,
                                    "algorithmic_mbytes": round(rt_bytes / 1e6, 2),
                                    "implementation_extra_mbytes": round(rt_impl / 1e6, 2)},
        "kernels": kernels,
    }
    if cold is not None:
        res["cold_mall"] = cold
    if bwd is not None:
        res["backward"] = bwd
    nbal = args.balance_steps if args.balance_steps is not None else (20 if shape.name == "skew" else 3)
    if not frozen and not args.backward and nbal > 0:
        res["balance"] = {"steps": balance_record(layer, shape, nbal),
                          "note": "starts from a zero bias; fresh x per step (seeded by step), each step's bias "
                                  "from the previous step's update; tokens per expert"}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(shape, dict(W, c=c) if c is not None else W, x_np, args.cpu_seconds)
    layer.close()
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
