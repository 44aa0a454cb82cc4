"""Summaries of rocprofv3 output for the layer's kernels (text for profiles/).

    python -m sparse_moe_layer_rmsnorm_amd.profsum trace <kernel_trace.csv> <workload> "<command>"
    python -m sparse_moe_layer_rmsnorm_amd.profsum traffic <fetch.csv> <write.csv> <workload> "<command>" [json]

    python -m sparse_moe_layer_rmsnorm_amd.profsum counters <workload> "<commands>" <pmc.csv> [<pmc.csv> ...]

`trace` prints a markdown table of per-kernel launch counts and durations
from a `--kernel-trace` CSV.  `traffic` reads two `--pmc FETCH_SIZE` and
`--pmc WRITE_SIZE` counter CSVs of the same command, scales each counter by
what it reads for the plain 256 MiB device copy that `bench.py
--copy-calibration` runs first, and prints a markdown table plus the JSON
record (HBM bytes per launch per kernel) that bench.py reports as
`roofline.traffic`; with a fifth argument it also writes that record, keyed
by a hash of the kernel sources' code, comments excluded, to the given JSON
file (bench.py reports the figure only while the sources still hash the same).

`counters` sums each hardware counter of each kernel's launches (the first
launch of a kernel skipped when it has more), over the counter's hardware
instances, from one or more `--pmc` CSVs, and prints them per launch with the
ratios derived from them (each ratio states its counters).

The dense GEMM launches carry a tag template argument: 0 the h GEMM of a
forward (gemm_h), 1 router logits alone (gemm_rz, routing-only pass), 2 the
output GEMM (gemm_out).
Tag 3 is the backward's recomputation of the shared GLU pre-activations
(bwd_pq).  The grouped expert GEMM with the GLU epilogue is expert_up, the
other expert_down (the backward's recomputation of the expert pre-activations
uses that same kernel and is counted there).  The backward's data-gradient
products with K-major weights carry tags too: 4 dout against [W_sd | W_up]
(bwd_dout), 5 dh (bwd_dh), 8 the experts' dH (bwd_dH), 9 their dX (bwd_dX);
k_gemm_wgrad_km is the weight-gradient GEMM (bwd_wgrad, dense and per expert).
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sys
from collections import OrderedDict, defaultdict

COPY_BYTES = 256 << 20
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def strip_comments(text: str) -> str:
    """C/C++ source with // and /* */ comments, trailing blanks and empty lines
    removed (string and character literals are kept as written)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (line.rstrip() for line in "".join(out).split("\n"))
    return "\n".join(line for line in lines if line)


def source_hash(csrc: str = CSRC) -> str:
    """Hash of the HIP/C++ sources' code (comments and blank lines excluded):
    counter figures are valid for one hash."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


def logical_name(symbol: str, dense_seen: int) -> str | None:
    if "k_gemm_dense" in symbol:
        tag = symbol.split(">, ")[-1].split(">")[0].strip()
        return {"0": "gemm_h", "1": "gemm_rz", "2": "gemm_out", "3": "bwd_pq", "4": "bwd_dout", "5": "bwd_dh",
                "6": "bwd_wcat", "7": "bwd_wout"}.get(tag, "gemm_dense")
    if "k_gemm_dgrad" in symbol:
        tag = symbol.split(">(")[0].rsplit(",", 1)[-1].strip()
        return {"4": "bwd_dout", "5": "bwd_dh", "8": "bwd_dH", "9": "bwd_dX"}.get(tag, "bwd_dgrad")
    if "k_gemm_wgrad" in symbol:
        return "bwd_wgrad"
    if "k_gemm_expert" in symbol:  # the KIND argument: 2 GLU, 3 GLU + MXFP8 quantisation -> expert_up
        tail = symbol.rstrip()
        glu = any(tail.endswith(f"{k}>(moe::(anonymous namespace)::ExpertArgs)") for k in (2, 3))
        return "expert_up" if glu or "Li2EEEv" in symbol or "Li3EEEv" in symbol else "expert_down"
    for k in ("rmsnorm_bwd", "dgamma_part", "sum_slices", "glu_bwd", "combine_bwd", "dispatch_bwd", "gates_bwd",
              "mx_quant", "reduce_split"):
        if f"k_{k}" in symbol:
            return k
    for k in ("rmsnorm", "topk", "hist", "scan_local", "scan_global", "scatter", "combine", "qb_update",
              "qb_quantile", "qb_bias", "sign_bias", "zero"):
        if f"k_{k}" in symbol:
            return k
    if "rocclr_copyBuffer" in symbol:
        return "copy"
    return None


def _label(rows):
    """rows: (dispatch id, symbol, ...) in dispatch order -> list of logical names."""
    out, dense = [], 0
    for r in rows:
        name = logical_name(r[1], dense)
        if name in ("gemm_h", "gemm_out"):
            dense += 1
        out.append(name)
    return out


def trace_table(path: str) -> OrderedDict:
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    rows.sort()
    stats: OrderedDict = OrderedDict()
    for (did, sym, t0, t1), name in zip(rows, _label(rows)):
        if name is None:
            continue
        s = stats.setdefault(name, {"calls": 0, "total_ns": 0, "min_ns": None, "max_ns": 0})
        d = t1 - t0
        s["calls"] += 1
        s["total_ns"] += d
        s["min_ns"] = d if s["min_ns"] is None else min(s["min_ns"], d)
        s["max_ns"] = max(s["max_ns"], d)
    return stats


def counter_per_dispatch(path: str) -> list:
    acc: OrderedDict = OrderedDict()
    with open(path) as f:
        for r in csv.DictReader(f):
            did = int(r["Dispatch_Id"])
            e = acc.setdefault(did, [did, r["Kernel_Name"], 0.0])
            e[2] += float(r["Counter_Value"])  # summed over XCD / channel instances
    return sorted(acc.values())


def traffic_table(fetch_csv: str, write_csv: str):
    per = {}
    factors = {}
    for which, path in (("fetch", fetch_csv), ("write", write_csv)):
        rows = counter_per_dispatch(path)
        names = _label(rows)
        copy = [r[2] * 1024 for r, n in zip(rows, names) if n == "copy" and r[2] > 0]
        if not copy:
            raise SystemExit(f"{path}: no calibration copy found (run bench.py with --copy-calibration)")
        factor = COPY_BYTES / copy[-1]
        factors[which] = factor
        sums = defaultdict(list)
        for r, n in zip(rows, names):
            if n and n != "copy":
                sums[n].append(r[2] * 1024 * factor)
        for n, v in sums.items():
            # skip the first (warm-up) launch of each kernel when there are more
            vals = v[1:] if len(v) > 1 else v
            per.setdefault(n, {})[which] = sum(vals) / len(vals)
    return per, factors


def counters_table(paths: list) -> OrderedDict:
    """{kernel: {counter: mean per launch}} over the given --pmc CSVs."""
    out: OrderedDict = OrderedDict()
    for path in paths:
        acc: OrderedDict = OrderedDict()  # dispatch -> [symbol, {counter: value}]
        with open(path) as f:
            for r in csv.DictReader(f):
                did = int(r["Dispatch_Id"])
                e = acc.setdefault(did, [r["Kernel_Name"], defaultdict(float)])
                e[1][r["Counter_Name"]] += float(r["Counter_Value"])
        rows = sorted((did, sym, vals) for did, (sym, vals) in acc.items())
        per = defaultdict(list)
        for (did, sym, vals), name in zip(rows, _label(rows)):
            if name and name != "copy":
                per[name].append(vals)
        for name, launches in per.items():
            use = launches[1:] if len(launches) > 1 else launches
            d = out.setdefault(name, OrderedDict())
            for c in use[0]:
                d[c] = sum(v.get(c, 0.0) for v in use) / len(use)
    return out


def _ratio(d, num, den, scale=1.0):
    if num in d and den in d and d[den] > 0:
        return d[num] / (d[den] * scale)
    return None


def main(argv) -> int:
    if len(argv) >= 4 and argv[0] == "trace":
        path, workload, cmd = argv[1], argv[2], argv[3]
        st = trace_table(path)
        total = sum(s["total_ns"] for s in st.values())
        print(f"# Kernel durations, {workload} workload\n")
        print(f"Command: `{cmd}`\n")
        print("| kernel | launches | avg us | min us | max us | share |")
        print("|---|---:|---:|---:|---:|---:|")
        for n, s in sorted(st.items(), key=lambda kv: -kv[1]["total_ns"]):
            print(f"| {n} | {s['calls']} | {s['total_ns'] / s['calls'] / 1e3:.2f} | {s['min_ns'] / 1e3:.2f} | "
                  f"{s['max_ns'] / 1e3:.2f} | {100.0 * s['total_ns'] / total:.1f}% |")
        return 0
    if len(argv) >= 5 and argv[0] == "traffic":
        fetch, write, workload, cmd = argv[1], argv[2], argv[3], argv[4]
        per, factors = traffic_table(fetch, write)
        print(f"# HBM traffic per launch, {workload} workload\n")
        print(f"Command (one run per counter): `{cmd}`\n")
        print(f"Calibration: a 256 MiB device copy reads FETCH_SIZE x {factors['fetch']:.3f} and "
              f"WRITE_SIZE x {factors['write']:.3f} of its true bytes; the figures below are scaled by those "
              "factors.\n")
        print("| kernel | read MiB | written MiB | total MiB |")
        print("|---|---:|---:|---:|")
        for n, v in per.items():
            r, w = v.get("fetch", 0.0), v.get("write", 0.0)
            print(f"| {n} | {r / 2**20:.1f} | {w / 2**20:.1f} | {(r + w) / 2**20:.1f} |")
        rec = {n: int(v.get("fetch", 0.0) + v.get("write", 0.0)) for n, v in per.items()}
        print("\n```json")
        print(json.dumps({workload: rec}, indent=1))
        print("```")
        if len(argv) >= 6:
            doc = {"source_hash": source_hash(),
                   "note": "HBM bytes per launch (FETCH_SIZE and WRITE_SIZE, each scaled by its 256 MiB device-copy "
                           "factor); source_hash covers the kernel sources the counters were taken on",
                   "kernels": {workload: rec}}
            with open(argv[5], "w") as f:
                json.dump(doc, f, indent=1)
                f.write("\n")
        return 0
    if len(argv) >= 4 and argv[0] == "counters":
        workload, cmd, paths = argv[1], argv[2], argv[3:]
        tab = counters_table(paths)
        print(f"# Hardware counters per launch, {workload} workload\n")
        print(f"Commands (one run per counter group): `{cmd}`\n")
        print("Counter values are summed over their hardware instances and averaged over a kernel's launches (its "
              "first launch skipped). GRBM_GUI_ACTIVE sums 8 XCD instances, so cycles = GRBM_GUI_ACTIVE / 8.\n")
        print("| kernel | cycles | MFMA busy | TA busy | L2 hit | L2 read latency (cycles) | "
              "TCP stalled on L2 |")
        print("|---|---:|---:|---:|---:|---:|---:|")
        for n, d in tab.items():
            cyc = d.get("GRBM_GUI_ACTIVE", 0.0) / 8
            mf = _ratio(d, "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", 1024 / 8)
            ta = _ratio(d, "TA_TA_BUSY_sum", "GRBM_GUI_ACTIVE", 256 / 8)
            hits, miss = d.get("TCC_HIT_sum"), d.get("TCC_MISS_sum")
            hit = hits / (hits + miss) if hits is not None and miss is not None and hits + miss > 0 else None
            lat = _ratio(d, "TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_READ_REQ_sum")
            st = _ratio(d, "TCP_PENDING_STALL_CYCLES_sum", "GRBM_GUI_ACTIVE", 256 / 8)
            f = lambda v, pct=True: "—" if v is None else (f"{100 * v:.0f}%" if pct else f"{v:.0f}")  # noqa: E731
            print(f"| {n} | {cyc:.0f} | {f(mf)} | {f(ta)} | {f(hit)} | {f(lat, False)} | {f(st)} |")
        print("\nRatios: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles); TA busy = TA_TA_BUSY_sum / "
              "(256 x cycles); L2 hit = TCC_HIT / (TCC_HIT + TCC_MISS); L2 read latency = "
              "TCP_TCC_READ_REQ_LATENCY_sum / TCP_TCC_READ_REQ_sum; TCP stalled on L2 = TCP_PENDING_STALL_CYCLES_sum "
              "/ (256 x cycles).")
        return 0
    print(__doc__)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
