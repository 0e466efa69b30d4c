"""Benchmark of the fused chunked KL loss (forward + backward with recompute) on one MI355X.

One step = fkl_forward + fkl_backward over the whole GPT-OSS-20B-like head
workload (N=32768 tokens, d=2880, V=201088, K=100 cached teacher entries,
T=1, chunk=4096), inputs resident in HBM. Prints one JSON line.

  python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--workload gptoss20b]

--workload picks one of the other synthetic workloads instead (llama3b: N=8192,
d=3072, V=128256, chunk 1024; long64k / long256k: N=65536 / 262144 packed rows
with the document ends masked; temp: N=16384, d=4096, V=128256, T=2 with a
perturbed-head teacher).

Throughput: value = tokens/s = N / step time; TFLOP/s counts 8*N*d*V per step
(2NdV forward logits, 2NdV recomputed logits, 2NdV grad_h, 2NdV grad_W).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused KL fwd+bwd tokens/s & TFLOP/s (V=201088,d=2880,N=32K); peak GiB"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0
WORKLOAD = "gptoss20b"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma.json")
TEACHER_RECIPES = {
    "gptoss20b": "zipf(1.1)+uniform top-100, logits N(0,9) sorted",
    "llama3b": "zipf(1.1)+uniform top-100, logits N(0,9) sorted",
    "long64k": "zipf(1.1)+uniform top-100, logits N(0,9) sorted",
    "long256k": "zipf(1.1)+uniform top-100, logits N(0,9) sorted",
    "temp": "exact top-100 of h W_t^T, W_t = W + 0.1 N(0,1/d) (bf16)",
}


def _code_tokens(text: str) -> str:
    """C/C++ source with comments removed and whitespace collapsed (string
    literals kept), so that comment edits leave the hash unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the library's code (kernels and launch plans), comments excluded."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "output_projection_kl_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(csrc, f), encoding="utf-8") as fh:
                h.update(f.encode())
                h.update(_code_tokens(fh.read()).encode())
    return h.hexdigest()


def _profile(path: str):
    try:
        with open(path) as f:
            return json.load(f)
    except (OSError, ValueError):
        return None


def traffic_for(kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if still current."""
    t = _profile(TRAFFIC_FILE)
    if t is None or t.get("source_sha256") != kernel_source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def profile_figures(kernel: str, avg_launch_ms: float) -> dict:
    """MFMA utilisation and HBM GB/s of one kernel from the committed rocprofv3
    counter summaries (profiles/mfma.json, profiles/traffic.json). A figure is
    reported only while the library's code hash matches the one the counters
    were taken on; otherwise it is null and the entry says which summary is stale.
    HBM GB/s = the counted bytes per launch / this run's average launch time."""
    sha = kernel_source_hash()
    out = {"mfma_util": None, "engine_ghz": None, "hbm_gbs": None, "hbm_bytes_per_launch": None, "stale": []}
    m = _profile(MFMA_FILE)
    if m is None:
        out["stale"].append("mfma: no summary")
    elif m.get("source_sha256") != sha:
        out["stale"].append(f"mfma: taken on code {str(m.get('source_sha256'))[:12]}")
    else:
        k = m.get("kernels", {}).get(kernel)
        if k:
            out["mfma_util"] = k.get("mfma_util")
            out["engine_ghz"] = k.get("engine_ghz")
    t = _profile(TRAFFIC_FILE)
    if t is None:
        out["stale"].append("traffic: no summary")
    elif t.get("source_sha256") != sha:
        out["stale"].append(f"traffic: taken on code {str(t.get('source_sha256'))[:12]}")
    else:
        k = t.get("kernels", {}).get(kernel)
        if k and avg_launch_ms:
            out["hbm_bytes_per_launch"] = k.get("bytes_per_launch")
            out["hbm_gbs"] = round(k["bytes_per_launch"] / (avg_launch_ms * 1e-3) / 1e9, 1)
    return out


def _read_counter_csv(path: str):
    """{dispatch id: (kernel name, value)} from a rocprofv3 counter_collection.csv."""
    import csv
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            did = int(r["Dispatch_Id"])
            name, val = r["Kernel_Name"], float(r["Counter_Value"])
            prev = out.get(did)
            out[did] = (name, val + (prev[1] if prev else 0.0))
    return out


def summarize_traffic(fetch_csv: str, write_csv: str, copy_mib: int, command: str) -> dict:
    """HBM bytes per launch of each path kernel from two rocprofv3 --pmc runs.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what they read for
    one plain device copy of copy_mib MiB (the largest copy-kernel dispatch of the
    same run), so the result is in true bytes.
    """
    fetch = _read_counter_csv(fetch_csv)
    write = _read_counter_csv(write_csv)
    n = copy_mib << 20

    def copy_kib(d):
        cands = [v for name, v in d.values() if "copyBuffer" in name or "copy" in name.lower()]
        if not cands:
            raise SystemExit("no copy kernel found in the counter run")
        return max(cands)

    rscale = n / (copy_kib(fetch) * 1024.0)
    wscale = n / (copy_kib(write) * 1024.0)
    kernels = {}
    for tag, d, scale in (("fetch", fetch, rscale), ("write", write, wscale)):
        for name, v in d.values():
            short = name.split("(")[0].split("<")[0].split("::")[-1].replace("void ", "").strip()
            if not short.startswith("k_"):
                continue
            k = kernels.setdefault(short[2:], {"launches_fetch": 0, "launches_write": 0,
                                               "fetch_bytes": 0.0, "write_bytes": 0.0})
            k[f"launches_{tag}"] += 1
            k[f"{tag}_bytes"] += v * 1024.0 * scale
    for k in kernels.values():
        fb = k["fetch_bytes"] / max(k["launches_fetch"], 1)
        wb = k["write_bytes"] / max(k["launches_write"], 1)
        k.update(fetch_bytes=fb, write_bytes=wb, bytes_per_launch=fb + wb)
        del k["launches_write"]
        k["launches"] = k.pop("launches_fetch")
    return {
        "source_sha256": kernel_source_hash(),
        "command": command,
        "copy_calibration": {"bytes": n, "fetch_scale": rscale, "write_scale": wscale},
        "kernels": kernels,
    }


def summarize_stats(stats_csv: str, command: str) -> str:
    """Markdown table from a rocprofv3 --stats kernel_stats.csv."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"Command: `{command}`", "",
             "| kernel | calls | total ms | avg us | min us | max us | share |",
             "|---|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"].split("(")[0].replace("void ", "")
        lines.append(f"| {name} | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f}% |")
    return "\n".join(lines) + "\n"


def _short_kernel_name(name: str) -> str:
    return name.split("(")[0].split("<")[0].split("::")[-1].replace("void ", "").strip()


def summarize_mfma(counter_csv: str, command: str, trace_csv: str | None = None):
    """MFMA utilisation per kernel from a rocprofv3 --pmc run of
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE (GRBM_GUI_ACTIVE is summed over
    the 8 XCDs, MFMA busy cycles over the 1024 SIMDs). With the same run's
    kernel_trace.csv, the engine clock per dispatch is GRBM_GUI_ACTIVE per XCD
    over the dispatch's duration. Returns (markdown, {kernel: figures})."""
    import collections
    import csv
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    act_by_dispatch = {}
    for r in csv.DictReader(open(counter_csv)):
        name = _short_kernel_name(r["Kernel_Name"])
        per[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
        if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
            act_by_dispatch[int(r["Dispatch_Id"])] = (name, float(r["Counter_Value"]))
    durations = collections.defaultdict(list)
    if trace_csv:
        for r in csv.DictReader(open(trace_csv)):
            did = int(r["Dispatch_Id"])
            if did in act_by_dispatch:
                name, act = act_by_dispatch[did]
                ns = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
                if ns > 0:
                    durations[name].append(act / 8.0 / ns)
    lines = [f"Command: `{command}`", "",
             "| kernel | dispatches | MFMA busy SIMD-cycles | active cycles per XCD | MFMA utilisation | engine GHz |",
             "|---|---|---|---|---|---|"]
    figures = {}
    for name, c in per.items():
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES")
        act = c.get("GRBM_GUI_ACTIVE")
        if not busy or not act or sum(busy) == 0:
            continue
        b = sum(busy) / len(busy)
        a = sum(act) / len(act) / 8.0
        ghz = sum(durations[name]) / len(durations[name]) if durations.get(name) else None
        key = name[2:] if name.startswith("k_") else name
        figures[key] = {"dispatches": len(busy), "mfma_util": round(b / (1024.0 * a), 4),
                        "engine_ghz": round(ghz, 3) if ghz else None}
        lines.append(f"| {name} | {len(busy)} | {b:.4g} | {a:.4g} | {b / (1024.0 * a):.3f} | "
                     f"{'%.2f' % ghz if ghz else '-'} |")
    return "\n".join(lines) + "\n", figures


def summarize_counters(counter_csv: str, command: str) -> str:
    """Markdown from a rocprofv3 --pmc run: each kernel's counters averaged per
    dispatch, and the ratios that say where its non-MFMA cycles go, for the
    counters present. GRBM_GUI_ACTIVE is summed over the 8 XCDs; SQ counters
    are summed over the whole chip; SQ_WAVE_CYCLES and SQ_WAIT_* are in units
    of 4 cycles."""
    import collections
    import csv
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    for r in csv.DictReader(open(counter_csv)):
        name = _short_kernel_name(r["Kernel_Name"])
        per[name][r["Counter_Name"]] += float(r["Counter_Value"])
        disp[name].add(int(r["Dispatch_Id"]))
    names = sorted({c for v in per.values() for c in v})
    lines = [f"Command: `{command}`", "", "Per dispatch (averages):", "",
             "| kernel | dispatches | " + " | ".join(names) + " |",
             "|---|---|" + "---|" * len(names)]
    for k, c in per.items():
        n = len(disp[k])
        lines.append(f"| {k} | {n} | " + " | ".join(f"{c[x] / n:.4g}" for x in names) + " |")
    lines += ["", "Ratios:", "",
              "| kernel | LDS bank-conflict cycles / LDS active cycles | LDS active, % of CU cycles | "
              "waves waiting for issue, % of wave cycles | of which for LDS | LDS instr per MFMA | "
              "other VALU instr per MFMA | L2 hit rate |",
              "|---|---|---|---|---|---|---|---|"]

    def ratio(a, b, scale=1.0, fmt="{:.3f}"):
        return fmt.format(scale * a / b) if b else "-"

    for k, c in per.items():
        cu_cycles = c["GRBM_GUI_ACTIVE"] / 8.0 * 256.0
        mf = c["SQ_INSTS_MFMA"]
        lines.append("| " + " | ".join([
            k,
            ratio(c["SQ_LDS_BANK_CONFLICT"], c["SQ_LDS_IDX_ACTIVE"]),
            ratio(c["SQ_LDS_IDX_ACTIVE"], cu_cycles, 100.0, "{:.1f}"),
            ratio(c["SQ_WAIT_INST_ANY"], c["SQ_WAVE_CYCLES"], 100.0, "{:.1f}"),
            ratio(c["SQ_WAIT_INST_LDS"], c["SQ_WAVE_CYCLES"], 100.0, "{:.1f}"),
            ratio(c["SQ_INSTS_LDS"], mf, 1.0, "{:.2f}"),
            ratio(c["SQ_INSTS_VALU"] - mf, mf, 1.0, "{:.2f}"),
            ratio(c["TCC_HIT_sum"], c["TCC_HIT_sum"] + c["TCC_MISS_sum"]),
        ]) + " |")
    return "\n".join(lines) + "\n"


def cpu_baseline(wl, rows: int):
    """The fp64 oracle, as it stands, on the first `rows` rows of the same workload."""
    import numpy as np
    import oracle
    affinity = len(os.sched_getaffinity(0))
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"] or threadpool_info()
        threads = max([p.get("num_threads", 1) for p in info] or [1])
        if info:
            blas = f"{info[0].get('internal_api', '?')} {info[0].get('version', '')}".strip()
    except Exception:  # noqa: BLE001
        threads = affinity
    h = wl.h[:rows].float().cpu().numpy()
    W = wl.W.float().cpu().numpy()
    ti = wl.t_idx_np[:rows]
    tl = wl.t_logit_np[:rows]
    t0 = time.perf_counter()
    oracle.forward(h, W, ti, tl, wl.T, None, chunk=rows)
    oracle.backward(h, W, ti, tl, wl.T, None, chunk=rows)
    dt = time.perf_counter() - t0
    flops = 8.0 * rows * wl.d * wl.V
    return {
        "value": rows / dt,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"first {rows} of {wl.N} rows of the same workload, forward + backward over the full "
                   f"vocabulary in numpy fp64 (BLAS threads={threads}); {dt:.1f} s, "
                   f"{flops / dt / 1e9:.1f} GFLOP/s"),
        "blas": blas,
        "blas_threads": int(threads),
        "affinity_cores": affinity,
        "seconds": round(dt, 2),
    }


def vendor_gemm_context(torch, wl, dev) -> dict:
    """Attainable-peak context: the vendor library's bf16 GEMM (torch.mm, which
    runs hipBLASLt) on one forward chunk's logits shape, chunk x d times d x V.
    Not part of the loss; reported beside it."""
    rows = min(wl.chunk, wl.N)
    a = wl.h[:rows]
    out = torch.empty((rows, wl.V), dtype=torch.bfloat16, device=dev)
    for _ in range(2):
        torch.mm(a, wl.W.t(), out=out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch.mm(a, wl.W.t(), out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del out
    return {"op": f"torch.mm bf16 [{rows} x {wl.d}] x [{wl.d} x {wl.V}] -> bf16", "ms": round(ms, 3),
            "tflops": round(2.0 * rows * wl.d * wl.V / (ms / 1e3) / 1e12, 1)}


def bench_builder(args, torch, fkl, make_device_workload, dev) -> int:
    """fkl_topk on the large-head shape: N=16384 rows, d=4096, V=128256, K=100,
    teacher head W_t = W + 0.1 N(0, 1/d). One step = one full cache build."""
    from workloads.device import perturbed_head
    wl = make_device_workload("temp", dev, teacher="uniform")
    Wt = perturbed_head(wl.W, 4242, dev)
    K = 100
    ws = torch.empty(fkl.topk_workspace_size(wl.N, wl.d, wl.V, K), dtype=torch.uint8, device=dev)
    ti = torch.empty((wl.N, K), dtype=torch.int32, device=dev)
    tl = torch.empty((wl.N, K), dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        fkl.topk(wl.h, Wt, K, workspace=ws, t_idx=ti, t_logit=tl)
    torch.cuda.synchronize()
    trace = not args.no_trace
    if trace:
        fkl.trace_read()
        fkl.trace_enable(True)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        fkl.topk(wl.h, Wt, K, workspace=ws, t_idx=ti, t_logit=tl)
    stop.record()
    torch.cuda.synchronize()
    if trace:
        fkl.trace_enable(False)
    ms = start.elapsed_time(stop) / args.steps
    kernels = {k["name"]: {"launches_per_step": k["launches"] / args.steps,
                           "avg_ms": k["total_ms"] / k["launches"],
                           "tflops": (k["flops"] / k["launches"]) / (k["total_ms"] / k["launches"] / 1e3) / 1e12
                           if k["flops"] else None} for k in (fkl.trace_read() if trace else [])}
    # context: torch fp32 GEMM (no TF32) + torch.topk over the same rows, in 1024-row passes
    prev = torch.backends.cuda.matmul.allow_tf32
    torch.backends.cuda.matmul.allow_tf32 = False
    Wt32 = Wt.float()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for r0 in range(0, wl.N, 1024):
        torch.topk(wl.h[r0:r0 + 1024].float() @ Wt32.t(), K, dim=1)
    e1.record()
    torch.cuda.synchronize()
    torch.backends.cuda.matmul.allow_tf32 = prev
    flops = 2.0 * wl.N * wl.d * wl.V
    out = {
        "metric": "teacher top-100 cache build rows/s (N=16384, d=4096, V=128256)",
        "value": round(wl.N / (ms / 1e3), 1),
        "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 3), "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"teacher cache: N={wl.N} d={wl.d} V={wl.V} K={K}, W_t = W + 0.1 N(0,1/d)"},
        "tflops": round(flops / (ms / 1e3) / 1e12, 1),
        "frac_of_bf16_peak": round(flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "torch_fp32_matmul_topk_ms": round(e0.elapsed_time(e1), 3),
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=WORKLOAD,
                    choices=["gptoss20b", "llama3b", "long64k", "long256k", "temp"],
                    help="synthetic workload (default: the GPT-OSS-20B-like head)")
    ap.add_argument("--cpu-rows", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm-context", action="store_true",
                    help="skip the vendor bf16 GEMM timing reported as context")
    ap.add_argument("--no-trace", action="store_true", help="skip per-kernel event timing")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (reference for HBM counters)")
    ap.add_argument("--builder", action="store_true",
                    help="time the teacher-cache builder (fkl_topk) on the large-head shape instead")
    ap.add_argument("--summarize-stats", metavar="CSV",
                    help="print a markdown summary of a rocprofv3 kernel_stats.csv and exit (no GPU)")
    ap.add_argument("--summarize-mfma", nargs="+", metavar="CSV",
                    help="COUNTER_CSV [KERNEL_TRACE_CSV]: print MFMA utilisation (and engine clock) per kernel "
                         "from a rocprofv3 counter run, write profiles/mfma.json, and exit (no GPU)")
    ap.add_argument("--mfma-json", default=MFMA_FILE,
                    help="where --summarize-mfma writes its figures (default profiles/mfma.json, the file the "
                         "bench line reads)")
    ap.add_argument("--summarize-counters", metavar="CSV",
                    help="markdown of a rocprofv3 counter run: per-kernel averages and cycle ratios (no GPU)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from FETCH_SIZE and WRITE_SIZE counter runs (no GPU)")
    ap.add_argument("--command", default="", help="the profiling command, recorded in summaries")
    args = ap.parse_args()
    if args.summarize_stats:
        print(summarize_stats(args.summarize_stats, args.command), end="")
        return 0
    if args.summarize_mfma:
        md, figures = summarize_mfma(args.summarize_mfma[0], args.command,
                                     args.summarize_mfma[1] if len(args.summarize_mfma) > 1 else None)
        with open(args.mfma_json, "w") as f:
            json.dump({"source_sha256": kernel_source_hash(), "command": args.command, "kernels": figures}, f,
                      indent=1)
        print(md, end="")
        return 0
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters, args.command), end="")
        return 0
    if args.summarize_traffic:
        t = summarize_traffic(*args.summarize_traffic, args.calibrate_copy_mib or 1024, args.command)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t, indent=1))
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported (the path is "
              "single-GPU: no collectives or sharding)", file=sys.stderr)
        return 2

    import torch
    import output_projection_kl_amd as fkl
    from workloads.device import make_device_workload

    dev = torch.device("cuda", 0)
    if args.builder:
        return bench_builder(args, torch, fkl, make_device_workload, dev)
    print(f"[bench] generating {args.workload} inputs on {torch.cuda.get_device_name(dev)}", file=sys.stderr,
          flush=True)
    wl = make_device_workload(args.workload, dev)
    torch.cuda.synchronize()
    fb, bb = fkl.workspace_size(wl.N, wl.d, wl.V, wl.K, wl.T, chunk=wl.chunk)
    plan = fkl.plan_info(wl.N, wl.d, wl.V, wl.K, wl.T, chunk=wl.chunk)
    ws = torch.empty(max(fb, bb), dtype=torch.uint8, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    row_lse = torch.empty(wl.N, dtype=torch.float32, device=dev)
    grad_h = torch.empty((wl.N, wl.d), dtype=torch.float32, device=dev)
    grad_W = torch.empty((wl.V, wl.d), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    in_out_bytes = sum(t.numel() * t.element_size() for t in
                       (wl.h, wl.W, wl.t_idx, wl.t_logit, row_lse, grad_h, grad_W))
    torch.cuda.reset_peak_memory_stats(dev)

    if args.calibrate_copy_mib > 0:
        # A plain copy of n bytes whose source was written long enough ago to
        # have left the 256 MiB last-level cache (a 2 GiB fill comes between).
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        flush = torch.empty(2 << 30, dtype=torch.uint8, device=dev).fill_(2)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy: {n} bytes read, {n} bytes written", file=sys.stderr, flush=True)
        del src, dst, flush
        torch.cuda.reset_peak_memory_stats(dev)

    def step():
        fkl.forward(wl.h, wl.W, wl.t_idx, wl.t_logit, T=wl.T, mask=wl.mask, chunk=wl.chunk, workspace=ws,
                    loss=loss, row_lse=row_lse)
        fkl.backward(wl.h, wl.W, wl.t_idx, wl.t_logit, row_lse, T=wl.T, mask=wl.mask, chunk=wl.chunk,
                     workspace=ws, grad_h=grad_h, grad_W=grad_W)

    def held_outside_torch() -> int:
        # device memory neither free nor in torch's pool (hipMemGetInfo)
        free, total = torch.cuda.mem_get_info(dev)
        return total - free - torch.cuda.memory_reserved(dev)

    outside0 = held_outside_torch()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    outside1 = held_outside_torch()
    print(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps", file=sys.stderr, flush=True)
    trace = not args.no_trace
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    # per-step events: before the forward, between forward and backward, after
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for i in range(args.steps):
        marks[i][0].record()
        fkl.forward(wl.h, wl.W, wl.t_idx, wl.t_logit, T=wl.T, mask=wl.mask, chunk=wl.chunk, workspace=ws,
                    loss=loss, row_lse=row_lse)
        marks[i][1].record()
        fkl.backward(wl.h, wl.W, wl.t_idx, wl.t_logit, row_lse, T=wl.T, mask=wl.mask, chunk=wl.chunk,
                     workspace=ws, grad_h=grad_h, grad_W=grad_W)
        marks[i][2].record()
    stop.record()
    torch.cuda.synchronize()
    outside2 = held_outside_torch()
    fwd_ms = sorted(m[0].elapsed_time(m[1]) for m in marks)
    bwd_ms = sorted(m[1].elapsed_time(m[2]) for m in marks)
    step_ms = sorted(m[0].elapsed_time(m[2]) for m in marks)
    wall = time.perf_counter() - t_wall
    # Per-kernel times come from a second timed run of as many steps with the
    # library's per-launch hipEvents on: two events around every launch cost
    # about 1% of a step, so the headline steps above run without them.
    traced_ms = None
    if trace:
        fkl.trace_read()
        fkl.trace_enable(True)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(args.steps):
            step()
        t1.record()
        torch.cuda.synchronize()
        fkl.trace_enable(False)
        traced_ms = t0.elapsed_time(t1) / args.steps
    ms = start.elapsed_time(stop) / args.steps
    peak = torch.cuda.max_memory_allocated(dev)
    kstats = fkl.trace_read() if trace else []
    flops_step = 8.0 * wl.N * wl.d * wl.V
    tokens_s = wl.N / (ms / 1e3)
    tflops = flops_step / (ms / 1e3) / 1e12

    roofline = None
    kernels = {}
    for k in kstats:
        avg = k["total_ms"] / max(k["launches"], 1)
        kernels[k["name"]] = {
            "launches_per_step": k["launches"] / args.steps,
            "avg_ms": avg,
            "share": k["total_ms"] / (traced_ms * args.steps),
            "tflops": (k["flops"] / k["launches"]) / (avg / 1e3) / 1e12 if k["flops"] else None,
        }
    for name, k in kernels.items():
        k.update({f: v for f, v in profile_figures(name, k["avg_ms"]).items() if f != "stale"})
    mfma = [k for k in kstats if k["flops"] > 0]
    if mfma:
        dom = max(mfma, key=lambda k: k["total_ms"])
        avg_s = dom["total_ms"] / dom["launches"] / 1e3
        achieved = dom["flops"] / dom["launches"] / avg_s / 1e12
        prof = profile_figures(dom["name"], avg_s * 1e3)
        roofline = {
            "bound": "mfma",
            "kernel": dom["name"],
            "achieved": round(achieved, 1),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_for(dom["name"]),
            "avg_launch_ms": round(avg_s * 1e3, 4),
            "flops_per_launch": dom["flops"] / dom["launches"],
            "measured_over": f"{args.steps} further steps with per-launch hipEvents on the library's stream",
            "mfma_util": prof["mfma_util"],
            "engine_ghz": prof["engine_ghz"],
            "hbm_gbs": prof["hbm_gbs"],
            "profile_stale": prof["stale"] or None,
        }

    out = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.describe(), "N": wl.N, "d": wl.d, "V": wl.V, "K": wl.K, "T": wl.T,
                   "chunk": wl.chunk, "teacher": TEACHER_RECIPES[args.workload],
                   "mask": "packed: last token of each of 8 documents" if wl.mask is not None else "none",
                   "passes": {"fwd_rows": plan["fwd_rows"], "bwd_rows": plan["bwd_rows"],
                              "vslab": plan["vslab"], "fwd_passes": plan["fwd_passes"],
                              "bwd_passes": plan["bwd_passes"], "slabs": plan["slabs"]}},
        "tflops": round(tflops, 1),
        "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "step_ms_median": round(step_ms[len(step_ms) // 2], 3),
        "step_ms_min": round(step_ms[0], 3),
        "forward": {"ms_median": round(fwd_ms[len(fwd_ms) // 2], 3),
                    "tflops": round(2.0 * wl.N * wl.d * wl.V / (fwd_ms[len(fwd_ms) // 2] / 1e3) / 1e12, 1)},
        "backward": {"ms_median": round(bwd_ms[len(bwd_ms) // 2], 3),
                     "tflops": round(6.0 * wl.N * wl.d * wl.V / (bwd_ms[len(bwd_ms) // 2] / 1e3) / 1e12, 1)},
        "peak_gib": round(peak / 2**30, 3),
        "extra_gib": round((peak - in_out_bytes) / 2**30, 3),
        # hipMemGetInfo cross-check: device memory taken outside torch's pool
        # by the warmup steps (the library's code objects and static scratch,
        # loaded on first use) and by the timed steps (0: no allocation per call)
        "device_bytes_outside_torch": {"warmup": outside1 - outside0, "timed_steps": outside2 - outside1},
        "inputs_outputs_gib": round(in_out_bytes / 2**30, 3),
        "loss": float(loss.item()),
        "wall_s_timed": round(wall, 3),
        "ms_per_step_traced": round(traced_ms, 3) if traced_ms is not None else None,
        "roofline": roofline,
        "kernels": kernels,
    }
    if not args.no_gemm_context:
        out["vendor_gemm_context"] = vendor_gemm_context(torch, wl, dev)
    if not args.no_cpu_baseline:
        print(f"[bench] timing the fp64 oracle on {args.cpu_rows} rows", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_rows)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
