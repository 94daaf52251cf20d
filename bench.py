#!/usr/bin/env python3
"""Throughput of shared-prefix, prefill-only branch scoring on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

One step is the whole scoring path over one batch of synthetic input: the
shared prefix is prefilled once into fresh KV pages, every branch is scored
over its own suffix against the prefix pages (label softmax at the last
position), and the prefix pages are released again, so every step is cold.
The default workload is the 2,000-token prefix with 5 branches of 48 tokens
and 2 labels (a 4-block bf16 model at Qwen3-like width), the configuration the
headline metric is quoted on.  Inputs are seeded synthetic data resident in
HBM before the timed region.

Prints one JSON line: scored branches/s (value), effective prefill tokens/s
(logical tokens incl. the shared prefix counted per branch), the phase split,
the roofline of the dominant kernel (algorithmic work per launch / HIP-event
launch time) and the CPU oracle on a bounded sample as a baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
ROOT = os.path.dirname(os.path.abspath(__file__))


def algorithmic(wl, inst):
    """Algorithmic FLOPs of the prefix prefill and bytes of the branch phase.

    What the method needs: a prefill produces the KV cache at every position
    and the logits at the last one only (jdon.com article, prefill-only
    section).  So the last layer needs the K/V projections of every token, and
    the query projection, attention and output projection only at the read-out
    positions (none in the prefix prefill, the last token of each branch)."""
    m = wl.model
    E = 2 if m.dtype == "bf16" else 4
    d, hq, hkv, dh, L = m.d, m.hq, m.hkv, m.dh, m.n_layers
    nqkv = (hq + 2 * hkv) * dh
    nkv = 2 * hkv * dh
    P = sum(len(p) for p in inst.prefixes)
    proj = sum(2 * len(p) * d * nqkv + 2 * len(p) * hq * dh * d for p in inst.prefixes) * (L - 1)
    proj += sum(2 * len(p) * d * nkv for p in inst.prefixes)
    attn = sum(4 * dh * hq * len(p) * (len(p) + 1) / 2 for p in inst.prefixes) * (L - 1)
    br = inst.passes[0]
    tb = sum(len(b.tokens) for b in br)
    w_bytes = L * (nqkv * d + d * hq * dh) * E
    kv_prefix = L * P * 2 * hkv * dh * E            # prefix pages read once per sibling group
    kv_suffix = L * tb * 2 * hkv * dh * E
    emb = tb * d * E
    labels = sum(len(b.labels) for b in br) * d * E
    plen = [len(inst.prefixes[b.request]) for b in br]
    br_flops = (L - 1) * sum(2 * len(b.tokens) * d * nqkv + 2 * len(b.tokens) * hq * dh * d
                             + 4 * dh * hq * len(b.tokens) * (pl + (len(b.tokens) + 1) / 2)
                             for b, pl in zip(br, plen))
    br_flops += sum(2 * len(b.tokens) * d * nkv + 2 * d * hq * dh + 2 * hq * dh * d
                    + 4 * dh * hq * (pl + len(b.tokens)) for b, pl in zip(br, plen))
    return {"prefill_flops": proj + attn, "branch_bytes": w_bytes + kv_prefix + kv_suffix + emb + labels,
            "branch_flops": br_flops}


def tree_flops(wl, inst):
    """Algorithmic FLOPs of a candidate-tree call: projections of every token
    computed once (the trie's nodes) and causal attention of each node's tokens
    over their whole path; in the last layer K/V projections of every token and
    the rest only at the candidates' read-out positions (the leaves' last
    tokens), as in algorithmic()."""
    m = wl.model
    d, hq, hkv, dh, L = m.d, m.hq, m.hkv, m.dh, m.n_layers
    nqkv = (hq + 2 * hkv) * dh
    nkv = 2 * hkv * dh
    t = wl.tree
    nodes = [(t.root_len, 0)]
    leaves = []
    for ci, cl in enumerate(t.child_lens):
        nodes.append((cl, t.root_len))
        nodes += [(t.leaf_len, t.root_len + cl)] * t.leaves_per_child[ci]
        leaves += [(t.leaf_len, t.root_len + cl)] * t.leaves_per_child[ci]
    proj = sum(2 * n * d * nqkv + 2 * n * hq * dh * d for n, _ in nodes) * (L - 1)
    attn = sum(4 * dh * hq * n * (p + (n + 1) / 2) for n, p in nodes) * (L - 1)
    last = sum(2 * n * d * nkv for n, _ in nodes)
    last += sum(2 * d * hq * dh + 2 * hq * dh * d + 4 * dh * hq * (p + n) for n, p in leaves)
    return proj + attn + last


def cpu_baseline(wl, inst, weights, n_branches: int):
    """The oracle as it stands (from scratch per branch) on a bounded sample."""
    import numpy as np
    from oracle import model as om
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    m = om.from_weights(weights)
    seqs = inst.full_sequences(0)[:n_branches]
    t0 = time.perf_counter()
    om.score_from_scratch(m, [s for s, _ in seqs], [l for _, l in seqs])
    dt = time.perf_counter() - t0
    toks = sum(len(s) for s, _ in seqs)
    return {"value": round(n_branches / dt, 4), "unit": "branches/s", "cores": int(threads),
            "kind": "oracle", "effective_tok_s": round(toks / dt, 1),
            "host": {"os_cpu_count": os.cpu_count(), "cpu_model": cpu_model(), "blas_threads": int(threads),
                     "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None},
            "sample": f"{n_branches} of {len(inst.full_sequences(0))} branches of workload "
                      f"'{wl.name}' recomputed from scratch by the numpy oracle ({dt:.1f} s)"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def kernel_fractions(per_key: dict, dtype: str, n_steps: int) -> dict:
    """Each kernel instance against its own binding roofline, each kind timed
    with events on its own launches over untimed steps: the
    prefill projections and every attention against MFMA peak (algorithmic
    FLOPs), the projections of rounds of at most 256 rows (weight streaming)
    and the norm / embedding kernels against HBM peak (algorithmic bytes).
    Kernels whose algorithmic bytes are not recorded (merge, readout) get
    their time only."""
    peak = PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_F32_TFLOPS
    out = {}
    for key, (n, ms, flops, nbytes) in sorted(per_key.items(), key=lambda x: -x[1][1]):
        kind = key.split("[")[0]
        rows = int(key.split("[")[1].split()[0])
        e = {"launches_per_step": n // n_steps, "avg_us": round(1e3 * ms / n, 2)}
        if flops > 0 and not (kind in ("qkv", "qkv_kv", "oproj") and rows <= 256):
            ach = flops / (ms * 1e-3) / 1e12
            e.update({"bound": "mfma", "achieved": round(ach, 1), "unit": "TFLOP/s", "frac": round(ach / peak, 4)})
        elif nbytes > 0:
            ach = nbytes / (ms * 1e-3) / 1e9
            e.update({"bound": "hbm", "achieved": round(ach, 1), "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4)})
        out[key] = e
    return out


def launch_key(rec) -> str:
    """Launches of one kind over the same number of rows run the same kernel
    instance; the K/V-only projection of a last layer without read-outs is
    keyed apart (its FLOPs per row are those of 2 * kv_heads * head_dim
    columns, below the full projection's)."""
    kind = rec["kernel"]
    if kind == "qkv" and rec["rows"] > 0 and _QKV_ROW_FLOPS and rec["flops"] < 0.999 * _QKV_ROW_FLOPS * rec["rows"]:
        kind = "qkv_kv"
    return f"{kind}[{rec['rows']} rows]"


_QKV_ROW_FLOPS = 0.0  # FLOPs per row of the full QKV projection (set by main)


def kernel_sources_sha() -> str:
    import hashlib
    kdir = os.path.join(ROOT, "shared_prefix_kv_amd", "csrc", "kernels")
    h = hashlib.sha256()
    for name in sorted(os.listdir(kdir)):
        with open(os.path.join(kdir, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(key: str):
    """HBM bytes per launch of `key` from the committed counter runs, or None.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are each divided by what the
    same counter read per byte for a plain device copy of known size.  The
    figure is dropped (None) once any kernel source differs from the sources
    the counters were taken on.
    """
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    k = t.get("kernels", {}).get(key)
    if not k or k.get("kernel_sources_sha256") != kernel_sources_sha():
        return None
    c = t["copy"]
    rd = k["fetch_kib"] * c["bytes_read"] / c["fetch_kib"]
    wr = k["write_kib"] * c["bytes_written"] / c["write_kib"]
    return round(rd + wr)


def library_gemms() -> dict:
    """Context for the GEMM rooflines: torch.matmul (the ROCm BLAS library) on
    the projection shapes of the headline workload, bf16 operands drawn like
    the weights (N(0, 0.02)) and the activations (N(0, 1)); the median of 5
    batches of 20 back-to-back calls.  Not part of the scoring path."""
    import numpy as np
    import torch
    g = torch.Generator(device="cuda:0").manual_seed(0)
    res = {}
    for M, N, K, name in ((2000, 5120, 4096, "qkv[2000 rows]"), (2000, 4096, 4096, "oproj[2000 rows]"),
                          (240, 5120, 4096, "qkv[240 rows]"), (240, 4096, 4096, "oproj[240 rows]")):
        a = torch.randn(M, K, device="cuda:0", generator=g).to(torch.bfloat16)
        w = (torch.randn(N, K, device="cuda:0", generator=g) * 0.02).to(torch.bfloat16)
        wt = w.t()
        for _ in range(5):
            torch.matmul(a, wt)
        ts = []
        for _ in range(5):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                torch.matmul(a, wt)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / 20)
        us = float(np.median(ts))
        res[name] = {"us": round(us, 2), "tflop_s": round(2.0 * M * N * K / us / 1e6, 1),
                     "note": "plain GEMM, no RoPE / page-write / residual epilogue"}
    return res


def copy_calibration(mib: int) -> None:
    """A plain device-to-device copy of known size, for the HBM byte counters."""
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copy calibration: 3 copies of {n} bytes", file=sys.stderr)


def summarize(d: str) -> int:
    """Markdown summary of rocprofv3 --stats / --pmc CSV files found under d."""
    import csv
    import glob

    def short(name: str) -> str:
        name = name.split("(")[0]
        return name.replace("void ", "").replace("jev::dev::", "")

    for path in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
        print(f"### kernel time ({os.path.relpath(path, d)})\n")
        print("| kernel | calls | total ms | avg us | min us | max us | % |")
        print("|---|---:|---:|---:|---:|---:|---:|")
        with open(path) as f:
            for r in csv.DictReader(f):
                print(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                      f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                      f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
        print()
    for path in sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
        inst = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                k = (short(r["Kernel_Name"]), int(r["Grid_Size_X"]))
                a = inst.setdefault(k, [])
                a.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        print(f"### kernel instances by grid ({os.path.relpath(path, d)})\n")
        print("| kernel | grid x | calls | avg us | median us |")
        print("|---|---:|---:|---:|---:|")
        for (kn, gx), v in sorted(inst.items(), key=lambda x: -sum(x[1])):
            v = sorted(v)
            print(f"| `{kn}` | {gx} | {len(v)} | {sum(v) / len(v):.2f} | {v[len(v) // 2]:.2f} |")
        print()
    for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        agg = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                k = (short(r["Kernel_Name"]), r.get("Grid_Size", "?"), r["Counter_Name"])
                a = agg.setdefault(k, [0, 0.0])
                a[0] += 1
                a[1] += float(r["Counter_Value"])
        print(f"### counters per dispatch ({os.path.relpath(path, d)})\n")
        print("| kernel | grid | counter | dispatches | mean value |")
        print("|---|---:|---|---:|---:|")
        for (kn, grid, cn), (n, v) in sorted(agg.items()):
            print(f"| `{kn}` | {grid} | {cn} | {n} | {v / n:.1f} |")
        print()
    return 0


def sq_summary(dirs) -> int:
    """Instruction mix and MFMA occupancy per launch of the timed kinds, from
    rocprofv3 --pmc passes (each a directory) that together hold SQ_WAVES,
    SQ_INSTS_{VALU,MFMA,VALU_TRANS_F32,SALU,LDS,VMEM}, SQ_VALU_MFMA_BUSY_CYCLES,
    SQ_VALU_MFMA_COEXEC_CYCLES and GRBM_GUI_ACTIVE.  Per wave: instructions
    issued (VALU without the MFMAs).  MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES
    (cycles summed over the SIMDs) / (GRBM_GUI_ACTIVE / XCDs x SIMDs), the
    share of the kernel's cycles in which an average SIMD's matrix unit
    worked.  Co-issue: SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES."""
    import csv
    import glob

    def short(name: str) -> str:
        return name.split("(")[0].replace("void ", "").replace("jev::dev::", "")

    vals, agent = {}, {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    k = (short(r["Kernel_Name"]), int(r.get("Grid_Size", 0) or 0))
                    a = vals.setdefault(k, {}).setdefault(r["Counter_Name"], [0, 0.0])
                    a[0] += 1
                    a[1] += float(r["Counter_Value"])
        for path in glob.glob(os.path.join(d, "**", "*agent_info.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if r.get("Name", "").startswith("gfx"):
                        agent = r
    simds, xcc = int(agent.get("Simd_Count", 1024)), int(agent.get("Num_Xcc", 8))
    print("| launch | kernel | waves | VALU / wave | MFMA / wave | exp / wave | SALU / wave | LDS / wave | "
          "VMEM / wave | MFMA busy | VALU co-issued with MFMA |")
    print("|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|")
    for key, parts in TRAFFIC_LAUNCHES.items():
        name, grid = parts[0]
        c = {n: v / k for n, (k, v) in vals.get((name, grid), {}).items()}
        if "SQ_WAVES" not in c:
            continue
        w = c["SQ_WAVES"]
        mf = c.get("SQ_INSTS_MFMA", 0.0)
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / xcc
        occ = f"{busy / (cyc * simds):.1%}" if cyc else "—"
        co = f"{c.get('SQ_VALU_MFMA_COEXEC_CYCLES', 0.0) / busy:.1%}" if busy else "—"
        print(f"| `{key}` | `{name}` | {w:.0f} | {(c.get('SQ_INSTS_VALU', 0.0) - mf) / w:.0f} | {mf / w:.0f} | "
              f"{c.get('SQ_INSTS_VALU_TRANS_F32', 0.0) / w:.0f} | {c.get('SQ_INSTS_SALU', 0.0) / w:.0f} | "
              f"{c.get('SQ_INSTS_LDS', 0.0) / w:.0f} | {c.get('SQ_INSTS_VMEM', 0.0) / w:.0f} | {occ} | {co} |")
    return 0


# Kernel instances (name, rocprofv3 counter-run grid size: threads over all
# grid dimensions) that make up one
# launch of each timed kind on the headline workload (the split-K GEMMs of the
# branch round include their epilogue).
TRAFFIC_LAUNCHES = {
    "qkv[2000 rows]": [("gemm_pc_kernel<256, 160, 0>", 131072)],
    "qkv_kv[2000 rows]": [("gemm_pc_kernel<128, 64, 0>", 131072)],
    "oproj[2000 rows]": [("gemm_pc_kernel<256, 128, 1>", 131072)],
    "attn[2000 rows]": [("attn_kernel<bf16s, 128, 2>", 256000)],
    "attn[240 rows]": [("attn_kernel<bf16s, 128, 1>", 122880)],
    "merge[240 rows]": [("merge_kernel<bf16s, 128>", 245760)],
    "qkv[240 rows]": [("gemm_kernel<bf16s, 128, 0, true, 4, 2, 256>", 122880), ("split_epilogue<bf16s, 0>", 153600)],
    "oproj[240 rows]": [("gemm_kernel<bf16s, 128, 1, true, 4, 2, 256>", 98304),
                        ("split_res_norm_kernel<bf16s, 2>", 61440)],
    "attn[5 rows]": [("attn_kernel<bf16s, 128, 1>", 12288)],
    "oproj[5 rows]": [("gemm_kernel<bf16s, 128, 1, true, 1, 4, 64>", 49152), ("split_epilogue<bf16s, 1>", 8192)],
}


def write_traffic(fetch_dir: str, write_dir: str, copy_mib: int = 1024) -> int:
    """profiles/traffic.json from a FETCH_SIZE and a WRITE_SIZE rocprofv3 run of
    `bench.py --copy-calibration MIB`: mean KiB per dispatch of every kernel in
    TRAFFIC_LAUNCHES, and the copy kernel's reading for the calibration."""
    import csv
    import glob

    def short(name: str) -> str:
        return name.split("(")[0].replace("void ", "").replace("jev::dev::", "")

    def means(d: str, counter: str):
        agg = {}
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if r["Counter_Name"] != counter:
                        continue
                    k = (short(r["Kernel_Name"]), int(r.get("Grid_Size", 0) or 0))
                    a = agg.setdefault(k, [0, 0.0])
                    a[0] += 1
                    a[1] += float(r["Counter_Value"])
        return {k: v / n for k, (n, v) in agg.items()}

    fetch, write = means(fetch_dir, "FETCH_SIZE"), means(write_dir, "WRITE_SIZE")
    nbytes = copy_mib << 20
    copy_grid = nbytes // 8192  # the runtime's copy kernel: 8 KiB per workgroup of the 1 GiB copy

    def per_kernel(m, name, grid):
        vals = [v for (kn, g), v in m.items() if kn == name and g == grid]
        if len(vals) != 1:
            raise SystemExit(f"{name} (grid {grid}): {len(vals)} instances in the counter run")
        return vals[0]

    copy_f = [v for (kn, g), v in fetch.items() if kn == "__amd_rocclr_copyBuffer" and g == copy_grid]
    copy_w = [v for (kn, g), v in write.items() if kn == "__amd_rocclr_copyBuffer" and g == copy_grid]
    if not copy_f or not copy_w:
        raise SystemExit("no calibration copy in the counter runs (bench.py --copy-calibration)")
    sha = kernel_sources_sha()
    out = {"about": "HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs of bench.py on the "
                    "headline workload (bench.py --write-traffic); a split-K launch counts the GEMM and its "
                    "epilogue kernel",
           "copy": {"bytes_read": nbytes, "bytes_written": nbytes, "fetch_kib": round(copy_f[0], 1),
                    "write_kib": round(copy_w[0], 1)},
           "kernels": {}}
    for key, names in TRAFFIC_LAUNCHES.items():
        out["kernels"][key] = {"fetch_kib": round(sum(per_kernel(fetch, n, g) for n, g in names), 1),
                               "write_kib": round(sum(per_kernel(write, n, g) for n, g in names), 1),
                               "kernel_sources_sha256": sha}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))
    return 0


# (large, splits, bn) of jev_set_gemm_variant; (0, 0, 0) is the default
GEMM_VARIANTS = [(0, 0, 0), (1, 0, 0), (2, 0, 0), (3, 0, 0), (0, 3, 0), (0, 4, 0), (0, 0, 128)]


def gemm_variants(ctx, step, probs, n_steps: int) -> dict:
    """Each projection kernel variant on the bench step: the step time, every
    projection instance's average launch time (events on the projection
    launches only, over separate steps) and the largest probability change
    against the default variant.  The default's numbers come from the same
    call, so the variants are compared on one box and clock."""
    import numpy as np
    import torch

    from shared_prefix_kv_amd import jev
    res = {}
    ref = None
    try:
        for v in GEMM_VARIANTS:
            jev.set_gemm_variant(*v)
            for _ in range(3):
                step()
            torch.cuda.synchronize()
            got = probs.cpu().numpy().copy()
            if ref is None:
                ref = got
            t0 = time.perf_counter()
            for _ in range(n_steps):
                step()
            torch.cuda.synchronize()
            ms = 1e3 * (time.perf_counter() - t0) / n_steps
            per = {}
            for kind in ("qkv", "oproj"):
                ctx.profile([kind])
                for _ in range(3):
                    step()
                torch.cuda.synchronize()
                for r in ctx.profile_read():
                    a = per.setdefault(launch_key(r), [0, 0.0])
                    a[0] += 1
                    a[1] += r["ms"]
                ctx.profile(())
            res["large=%d splits=%d bn=%d" % v] = {
                "ms_per_step": round(ms, 4),
                "max_abs_dp_vs_default": float(np.max(np.abs(got - ref))),
                "avg_us": {k: round(1e3 * t / n, 2) for k, (n, t) in sorted(per.items())},
            }
    finally:
        jev.set_gemm_variant()
    return res


def config_summary(idx: int, steps: int, warmup: int) -> dict:
    """Throughput of another workload, inputs resident in HBM before the timed
    region; the same one-GPU path as the headline line.

    prefix + branches: a step prefills every prefix into fresh pages, scores
    every branch and frees the pages (cold).  With more than one pass (the
    32,768-token prefix) the prefix stays resident after one cold pass and each
    warm step scores a fresh set of branches on it (the repeated-state case):
    its branches/s is n_branches / t_score.  Tree: a step is one
    jev_score_candidates call over the full candidate sequences (staged rounds
    by depth)."""
    import numpy as np
    import torch
    from shared_prefix_kv_amd import jev
    from synth import make_instance, make_weights, workload

    wl = workload(idx)
    m = wl.model
    inst = make_instance(wl)
    weights = make_weights(wl)
    wdev = jev.upload_weights(weights)
    del weights
    peak = PEAK_BF16_TFLOPS if m.dtype == "bf16" else PEAK_F32_TFLOPS
    out = {"workload": wl.name, "layers": m.n_layers, "dtype": m.dtype}
    stream = torch.cuda.current_stream()

    def med_events(fn, n):
        ts = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    if wl.kind == "tree":
        C, Lb = inst.candidates, inst.cand_labels
        total = sum(len(c) for c in C)
        desc = jev.make_desc(m.n_layers, m.d, m.hq, m.hkv, m.dh, m.vocab, m.dtype, m.rope_theta, m.eps,
                             max(len(c) for c in C) + 16, total)
        ctx = jev.Context(desc, sum((len(c) + 15) // 16 for c in C) + 16, wdev)
        probs = torch.empty(sum(len(l) for l in Lb), dtype=torch.float32, device="cuda:0")
        call = lambda: ctx.score_candidates(C, Lb, probs=probs)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            call()
        torch.cuda.synchronize()
        ms = 1e3 * (time.perf_counter() - t0) / steps
        st = ctx.stats()
        fl = tree_flops(wl, inst)
        out.update({"ms_per_step": round(ms, 3), "branches_per_s": round(len(C) / ms * 1e3, 1),
                    "effective_tok_s": round(total / ms * 1e3, 1),
                    "computed_tok_s": round(st["computed_tokens"] / ms * 1e3, 1), "rounds": st["rounds"],
                    "call_ms_events": round(med_events(call, 3), 4),
                    "mfma_frac": round(fl / (ms * 1e-3) / 1e12 / peak, 4),
                    "algorithmic_gflop": round(fl / 1e9, 2)})
        ctx.close()
        return out

    prefixes = inst.prefixes
    P = sum(len(p) for p in prefixes)
    br_all = inst.passes
    n_br = len(br_all[0])
    max_pos = max(len(prefixes[b.request]) + len(b.tokens) for b in br_all[0]) + 16
    max_tok = max(P, sum(len(b.tokens) for b in br_all[0]))
    n_pages = sum((len(p) + 15) // 16 for p in prefixes) + sum((len(b.tokens) + 15) // 16 for b in br_all[0]) + 16
    desc = jev.make_desc(m.n_layers, m.d, m.hq, m.hkv, m.dh, m.vocab, m.dtype, m.rope_theta, m.eps,
                         max_pos, max_tok)
    ctx = jev.Context(desc, n_pages, wdev)
    probs = torch.empty(sum(len(b.labels) for b in br_all[0]), dtype=torch.float32, device="cuda:0")
    alg = algorithmic(wl, inst)
    logical = sum(len(prefixes[b.request]) + len(b.tokens) for b in br_all[0])
    hs = [None]

    def prefill():
        hs[0] = ctx.prefill_prefix([0] * len(prefixes), prefixes)

    def score(p=0):
        br = br_all[p]
        ctx.score_branches([hs[0][b.request] for b in br], [b.tokens for b in br], [b.labels for b in br],
                           probs=probs)

    def free():
        ctx.free_pages(hs[0])

    if wl.passes == 1:
        def step():
            prefill()
            score()
            free()
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        ms = 1e3 * (time.perf_counter() - t0) / steps
        pre_ms = med_events(lambda: (prefill(), free()), 3)
        prefill()
        sc_ms = med_events(score, 3)
        free()
        out.update({"ms_per_step": round(ms, 3), "branches_per_s": round(n_br / ms * 1e3, 1),
                    "effective_tok_s": round(logical / ms * 1e3, 1),
                    "computed_tok_s": round((P + sum(len(b.tokens) for b in br_all[0])) / ms * 1e3, 1),
                    "prefill_ms": round(pre_ms, 4), "score_ms": round(sc_ms, 4),
                    "prefill_mfma_frac": round(alg["prefill_flops"] / (pre_ms * 1e-3) / 1e12 / peak, 4),
                    "score_hbm_frac": round(alg["branch_bytes"] / (sc_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                    "score_mfma_frac": round(alg["branch_flops"] / (sc_ms * 1e-3) / 1e12 / peak, 4)})
    else:
        # one cold pass (prefill + pass-0 branches), then warm passes on the resident prefix
        t0 = time.perf_counter()
        prefill()
        score(0)
        torch.cuda.synchronize()
        cold_ms = 1e3 * (time.perf_counter() - t0)
        pre_ms = med_events(lambda: (free(), prefill()), 2)
        for _ in range(warmup):
            score(1)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            score(1)
        torch.cuda.synchronize()
        warm_ms = 1e3 * (time.perf_counter() - t0) / steps
        logical_w = sum(len(prefixes[b.request]) + len(b.tokens) for b in br_all[1])
        free()
        out.update({"ms_per_step": round(warm_ms, 3), "branches_per_s": round(n_br / warm_ms * 1e3, 1),
                    "effective_tok_s": round(logical_w / warm_ms * 1e3, 1),
                    "computed_tok_s": round(sum(len(b.tokens) for b in br_all[1]) / warm_ms * 1e3, 1),
                    "timed": "warm passes (prefix resident): n_branches / t_score",
                    "cold_pass_ms": round(cold_ms, 3), "cold_branches_per_s": round(n_br / cold_ms * 1e3, 1),
                    "prefill_ms": round(pre_ms, 4),
                    "prefill_mfma_frac": round(alg["prefill_flops"] / (pre_ms * 1e-3) / 1e12 / peak, 4),
                    "score_hbm_frac": round(alg["branch_bytes"] / (warm_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                    "score_mfma_frac": round(alg["branch_flops"] / (warm_ms * 1e-3) / 1e12 / peak, 4)})
    ctx.close()
    del wdev
    torch.cuda.empty_cache()
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--cpu-branches", type=int, default=4, help="oracle sample size (0 = skip)")
    ap.add_argument("--configs", default="1,3,4,5",
                    help="other workloads summarised under 'configs' in the same line ('' = none)")
    ap.add_argument("--config-steps", type=int, default=5)
    ap.add_argument("--roofline-kernel", default="auto",
                    help="kernel whose roofline is reported, as 'kind[rows]' (auto = largest total time)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the run, copy a MIB-MiB buffer 3 times (counter calibration for traffic)")
    ap.add_argument("--summarize", metavar="DIR", default=None,
                    help="print a summary of the rocprofv3 CSV output under DIR and exit")
    ap.add_argument("--round-invariant", action="store_true",
                    help="run with round-invariant numerics (jev_set_round_invariant); noted in config")
    ap.add_argument("--gemm-variants", action="store_true",
                    help="also time the projection kernel variants (jev_set_gemm_variant) on this workload")
    ap.add_argument("--library-gemms", action="store_true",
                    help="add torch.matmul times of the projection shapes ('library_gemm', context only)")
    ap.add_argument("--sq-summary", nargs="+", metavar="DIR", default=None,
                    help="instruction mix and MFMA occupancy from rocprofv3 --pmc SQ counter passes")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="write profiles/traffic.json from a FETCH_SIZE and a WRITE_SIZE rocprofv3 run and exit")
    args = ap.parse_args(argv)
    if args.summarize:
        return summarize(args.summarize)
    if args.write_traffic:
        return write_traffic(*args.write_traffic)
    if args.sq_summary:
        return sq_summary(args.sq_summary)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the multi-GPU sharding of this path is "
              f"a design note, not built", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from shared_prefix_kv_amd import jev
    from synth import make_instance, make_weights, workload

    wl = workload(args.workload)
    if wl.kind != "prefix_branches":
        print("bench.py times the prefix + branches workloads", file=sys.stderr)
        return 2
    m = wl.model
    global _QKV_ROW_FLOPS
    _QKV_ROW_FLOPS = 2.0 * m.d * (m.hq + 2 * m.hkv) * m.dh
    inst = make_instance(wl)
    weights = make_weights(wl)
    wdev = jev.upload_weights(weights)
    prefixes = inst.prefixes
    br = inst.passes[0]
    max_pos = max(len(inst.prefixes[b.request]) + len(b.tokens) for b in br) + 16
    max_tok = max(sum(len(p) for p in prefixes), sum(len(b.tokens) for b in br))
    n_pages = sum((len(p) + 15) // 16 for p in prefixes) + sum((len(b.tokens) + 15) // 16 for b in br) + 16
    desc = jev.make_desc(m.n_layers, m.d, m.hq, m.hkv, m.dh, m.vocab, m.dtype, m.rope_theta, m.eps,
                         max_pos, max_tok)
    ctx = jev.Context(desc, n_pages, wdev)
    if args.round_invariant:
        ctx.set_round_invariant(True)
    suffixes = [b.tokens for b in br]
    labels = [b.labels for b in br]
    n_lab = sum(len(l) for l in labels)
    probs = torch.empty(n_lab, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        hs = ctx.prefill_prefix([0] * len(prefixes), prefixes)
        if ev:
            ev[1].record(stream)
        ctx.score_branches([hs[b.request] for b in br], suffixes, labels, probs=probs)
        if ev:
            ev[2].record(stream)
        ctx.free_pages(hs)

    # warmup, then the per-kernel timing that also picks the dominant kernel
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    # each kernel kind timed on its own (events on its launches only) over 3
    # untimed steps: time per step by kind and by instance, and the dominant
    # instance (events on every launch of a step would slow the step down)
    n_prof = 3
    per_kind = {}
    per_launch = {}
    per_key = {}
    for kind in jev.KERNELS:
        ctx.profile([kind])
        for _ in range(n_prof):
            step()
        torch.cuda.synchronize()
        for r in ctx.profile_read():
            key = launch_key(r)
            per_kind[r["kernel"]] = per_kind.get(r["kernel"], 0.0) + r["ms"] / n_prof
            per_launch[key] = per_launch.get(key, 0.0) + r["ms"] / n_prof
            a = per_key.setdefault(key, [0, 0.0, 0.0, 0.0])
            a[0] += 1
            a[1] += r["ms"]
            a[2] += r["flops"]
            a[3] += r["bytes"]
        ctx.profile(())
    per_kernel = kernel_fractions(per_key, m.dtype, n_prof)
    key = max(per_launch, key=per_launch.get) if args.roofline_kernel == "auto" else args.roofline_kernel
    kern = key.split("[")[0].replace("qkv_kv", "qkv")

    # timed region: exactly K steps, the dominant kernel event-timed live
    # (events on the launches of its row count only: an event pair idles the
    # stream briefly, and the other instances of the kind need none)
    ctx.profile([kern], rows=int(key.split("[")[1].split()[0]))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    recs = [r for r in ctx.profile_read() if launch_key(r) == key]
    ctx.profile(())
    elapsed = t1 - t0
    st = ctx.stats()

    # phase split (prefill / scoring) from HIP events, on extra untimed steps
    n_ph = min(5, args.steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ph)]
    for i in range(n_ph):
        step(evs[i])
    torch.cuda.synchronize()
    pre_ms = float(np.median([a.elapsed_time(b) for a, b, _ in evs]))
    sc_ms = float(np.median([b.elapsed_time(c) for _, b, c in evs]))
    n_br = len(br)
    logical = sum(len(prefixes[b.request]) + len(b.tokens) for b in br)
    computed = sum(len(p) for p in prefixes) + sum(len(b.tokens) for b in br)
    alg = algorithmic(wl, inst)
    tot_ms = sum(r["ms"] for r in recs)
    flops = sum(r["flops"] for r in recs)
    nbytes = sum(r["bytes"] for r in recs)
    if flops > 0:
        peak = PEAK_BF16_TFLOPS if m.dtype == "bf16" else PEAK_F32_TFLOPS
        ach = flops / (tot_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4), "traffic": None}
    else:
        ach = nbytes / (tot_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None}
    roof["traffic"] = measured_traffic(key)
    roof.update({"kernel": key, "launches": len(recs), "avg_launch_us": round(1e3 * tot_ms / max(1, len(recs)), 2),
                 "work_per_launch": (flops or nbytes) / max(1, len(recs)),
                 "share_of_step": round(per_launch.get(key, 0) / max(1e-9, sum(per_launch.values())), 3)})

    out = {
        "metric": "scored branches/sec + effective prefill tok/s, 2k prefix x 5 branches",
        "value": round(n_br * args.steps / elapsed, 2),
        "unit": "branches/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": m.dtype,
        "data": "synthetic (seeded uniform token ids, N(0,0.02) weights)",
        "config": {"workload": wl.name, "prefix_tokens": [len(p) for p in prefixes], "branches": n_br,
                   "suffix_tokens": len(br[0].tokens), "labels_per_branch": len(labels[0]),
                   "layers": m.n_layers, "d_model": m.d, "q_heads": m.hq, "kv_heads": m.hkv,
                   "head_dim": m.dh, "vocab": m.vocab, "page_tokens": 16,
                   "numerics": "round-invariant" if args.round_invariant else "default"},
        "effective_prefill_tok_s": round(logical * args.steps / elapsed, 1),
        "computed_tok_s": round(computed * args.steps / elapsed, 1),
        "phases": {
            "prefill_ms": round(pre_ms, 4), "score_ms": round(sc_ms, 4),
            "prefill_mfma_frac": round(alg["prefill_flops"] / (pre_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "prefill_algorithmic_gflop": round(alg["prefill_flops"] / 1e9, 2),
            "branch_hbm_frac": round(alg["branch_bytes"] / (sc_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "branch_algorithmic_mb": round(alg["branch_bytes"] / 1e6, 2),
            "kernel_ms_per_step": {k: round(v, 4) for k, v in sorted(per_kind.items(), key=lambda x: -x[1])},
            "per_kernel": per_kernel,
        },
        "stats_last_call": {k: st[k] for k in ("logical_tokens", "computed_tokens", "cached_tokens", "rounds")},
        "roofline": roof,
    }
    if args.gemm_variants:
        out["gemm_variants"] = gemm_variants(ctx, step, probs, max(5, args.steps // 2))
    if args.cpu_branches > 0:
        out["cpu_baseline"] = cpu_baseline(wl, inst, weights, args.cpu_branches)
    else:
        out["cpu_baseline"] = None
    ctx.close()
    del weights, wdev
    torch.cuda.empty_cache()
    cfgs = {}
    for c in [int(x) for x in args.configs.split(",") if x.strip()]:
        if c == args.workload:
            continue
        print(f"config {c}: timing", file=sys.stderr, flush=True)
        cfgs[workload(c).name] = config_summary(c, args.config_steps, 2)
    if cfgs:
        out["configs"] = cfgs
    if args.library_gemms:
        out["library_gemm"] = library_gemms()
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
