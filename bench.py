"""LiSA forward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one lisa_forward call (statistics sweeps + fused output pass) over
one batch of synthetic inputs already resident in HBM.  Input sets rotate over
more than twice the 256 MB Infinity Cache so every call starts cold.  Prints
one JSON line: token-heads/s (B*heads*n per second), the roofline of the
dominant kernel (measured with HIP events on the stream it runs on), and the
CPU oracle timed on a bounded sample on the host cores.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LiSA fwd tokens/s (B·heads·n) at T=3, % of HBM roofline, 1 MI355X"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
DEFAULT_WORKLOAD = "pvt_t_stage1"
ROTATE_BYTES = 600 << 20
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
# The sources the forward kernel is built from (its counters go stale when they change).
def _csrc(*names):
    return [os.path.join(ROOT, "vision_transformer_token_amd", "csrc", f) for f in names]


# The sources each forward kernel is built from (with the host planner that
# configures its launch): its counters are current while their hash is.
KERNEL_SOURCES_BY_NAME = {
    "flow_kernel<bf16>": _csrc("lisa_flow.hip", "lisa_flow_schedule.hpp", "lisa_device.hpp", "lisa_kernels.hpp",
                               "lisa_api.hip"),
    "resident_kernel": _csrc("lisa_resident.hip", "lisa_resident.hpp", "lisa_device.hpp", "lisa_kernels.hpp",
                             "lisa_api.hip"),
}
KERNEL_SOURCES = KERNEL_SOURCES_BY_NAME["flow_kernel<bf16>"]
# The backward starts with the resident kernel's statistics launch; the layer
# runs the projections around the resident kernel.
BACKWARD_SOURCES = KERNEL_SOURCES_BY_NAME["resident_kernel"] + _csrc("lisa_backward.hip")
LAYER_SOURCES = KERNEL_SOURCES_BY_NAME["resident_kernel"] + _csrc("lisa_layer.hip", "lisa_layer.hpp")


def kernel_source_hash(sources=None):
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def compulsory_bytes_per_token_head(w):
    """Q, K, V read once, Y written once, adaptive weights read once."""
    esize = 2 if w.dtype == "bf16" else 4
    b = (2 * w.d_h + w.d_v) * esize + w.d_v * esize
    if w.mode == "adaptive":
        b += 4 * w.T
    return b


def cpu_baseline(w, x, budget_s=10.0):
    """The fp64 NumPy oracle, as it stands, on a bounded sample of the workload."""
    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    f64 = lambda t: None if t is None else t.double().numpy()  # noqa: E731
    q, k, v, wt, al = f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["weights"]), f64(x["alpha"])
    # Sample: whole batch entries in turn (cycling), until the time budget is spent.
    nslice = 0
    th = 0
    t0 = time.perf_counter()
    b = 0
    while time.perf_counter() - t0 < budget_s:
        oracle.lisa_forward(q[b:b + 1], k[b:b + 1], v[b:b + 1], H=w.H, W=w.W, T=w.T, alpha=al,
                            weights=None if wt is None else wt[b:b + 1], beta=x["beta"], eps=w.eps)
        nslice += w.heads
        th += w.heads * w.n
        b = (b + 1) % w.B
    dt = time.perf_counter() - t0
    return {
        "value": th / dt,
        "unit": "token-heads/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{nslice} (batch, head) slices of {w.name} ({w.B * w.heads} per step), "
                  f"fp64 NumPy, {dt:.1f} s",
    }


def load_counters(w, kernel):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if current."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    entry = c.get("kernels", {}).get(f"{kernel}@{w.name}")
    if not entry or entry.get("source_hash") != kernel_source_hash(KERNEL_SOURCES_BY_NAME.get(kernel)):
        return None
    return entry.get("hbm_bytes_per_launch")


def _csv_rows(path):
    import csv

    with open(path) as f:
        return list(csv.DictReader(f))


# The one kernel of the path (one launch per forward), by lisa_schedule.
KERNELS = {"streaming": "flow_kernel<bf16>", "resident": "resident_kernel"}


def _short(name):
    if "resident_kernel" in name:
        return "resident_kernel"
    if "flow_kernel" in name:
        t = "bf16" if "BF16" in name else "fp32"
        return f"flow_kernel<{t}, predictor>" if ", true>" in name else f"flow_kernel<{t}>"
    if "mlp_prep" in name:
        return "mlp_prep<bf16>" if "BF16" in name else "mlp_prep<fp32>"
    if "copyBuffer" in name:
        return "copyBuffer"
    if "proj_stream_qkv" in name:
        return "proj_stream_qkv<bf16>"
    m = re.search(r"proj_gemm<(unsigned short|float), (true|false)>", name)
    if m:
        return f"proj_gemm<{'bf16' if m.group(1) == 'unsigned short' else 'fp32'}, " \
               f"{'output' if m.group(2) == 'true' else 'qkv'}>"
    m = re.search(r"(bwd_\w+)(<(unsigned short|float)>)?", name)
    if m:
        return m.group(1) + ({"unsigned short": "<bf16>", "float": "<fp32>"}.get(m.group(3), ""))
    return name[:60]


def compulsory_bytes_backward(w):
    """Q, K, V and dY read once, dQ, dK, dV written once, adaptive weights read
    and their gradient written once."""
    esize = 2 if w.dtype == "bf16" else 4
    b = (2 * w.d_h + 2 * w.d_v) * esize + (2 * w.d_h + w.d_v) * esize
    if w.mode == "adaptive":
        b += 8 * w.T
    return b


def summarize_profiles(outdir, workload, commands):
    """Turn rocprofv3 CSV output (kernel trace + FETCH_SIZE/WRITE_SIZE passes of
    bench.py and of the plain-copy calibration) into profiles/ summaries."""
    w = None
    from vision_transformer_token_amd import workloads

    w = workloads.get(workload)
    stats = _csv_rows(os.path.join(outdir, "prof_trace", "trace_kernel_stats.csv"))
    lines = [f"# rocprofv3 kernel trace, workload {w.describe()}", "",
             f"command: {commands['trace']}", "",
             "| kernel | calls | average ns | min ns | max ns | share |", "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                     f"{r['MinNs']} | {r['MaxNs']} | {float(r['Percentage']):.1f}% |")

    def per_kernel(sub, stem, counter):
        rows = _csv_rows(os.path.join(outdir, sub, f"{stem}_counter_collection.csv"))
        acc = {}
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}

    fetch = per_kernel("pmc_fetch", "fetch", "FETCH_SIZE")
    write = per_kernel("pmc_write", "write", "WRITE_SIZE")
    cfetch = per_kernel("pmc_copy_fetch", "cfetch", "FETCH_SIZE")["copyBuffer"]
    cwrite = per_kernel("pmc_copy_write", "cwrite", "WRITE_SIZE")["copyBuffer"]
    copy_kib = commands["copy_mib"] * 1024
    f_scale, w_scale = copy_kib / cfetch, copy_kib / cwrite
    lines += ["", "# HBM traffic per launch (rocprofv3 --pmc, one counter per pass)", "",
              f"fetch pass: {commands['fetch']}", f"write pass: {commands['write']}",
              f"copy calibration: {commands['copy']} (FETCH_SIZE then WRITE_SIZE)", "",
              f"A plain device copy of {commands['copy_mib']} MiB reads FETCH_SIZE = {cfetch:.0f} KiB "
              f"and WRITE_SIZE = {cwrite:.0f} KiB per dispatch, so FETCH_SIZE is scaled by "
              f"{f_scale:.3f} and WRITE_SIZE by {w_scale:.3f}.", "",
              "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (scaled) |", "|---|---|---|---|"]
    entries = {}
    for k in sorted(set(fetch) & set(write)):
        if k not in KERNEL_SOURCES_BY_NAME:  # the copy, torch's workspace fill
            continue
        hbm = fetch[k] * 1024 * f_scale + write[k] * 1024 * w_scale
        entries[f"{k}@{w.name}"] = {"fetch_kib": fetch[k], "write_kib": write[k],
                                    "hbm_bytes_per_launch": hbm,
                                    "source_hash": kernel_source_hash(KERNEL_SOURCES_BY_NAME[k])}
        lines.append(f"| {k} | {fetch[k]:.0f} | {write[k]:.0f} | {hbm / 1e6:.2f} MB |")
    lines += ["", f"algorithmic bytes per forward: {w.token_heads * compulsory_bytes_per_token_head(w) / 1e6:.2f} MB"]
    lines += [f"source hash of {k.split('@')[0]}: {e['source_hash']}" for k, e in entries.items()]
    # Utilisation and instruction mix (two more passes, when present).
    if os.path.exists(os.path.join(outdir, "pmc_util", "util_counter_collection.csv")):
        avg_ns = {_short(r["Name"]): float(r["AverageNs"]) for r in stats}
        util = {c: per_kernel("pmc_util", "util", c) for c in ("MfmaUtil", "VALUBusy", "SQ_INSTS_VALU_MFMA_MOPS_BF16")}
        inst = {c: per_kernel("pmc_insts", "insts", c)
                for c in ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_MFMA",
                          "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE")}
        lines += ["", "# MFMA and VALU utilisation, instruction mix (rocprofv3 --pmc, two passes)", "",
                  f"utilisation pass: {commands['util']}", f"instruction pass: {commands['insts']}", "",
                  "MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES over (GRBM_GUI_ACTIVE x SIMDs); VALUBusy = SQ_ACTIVE_INST_VALU "
                  "over (GRBM_GUI_ACTIVE x CUs); bf16 MFMA work = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 flops, over "
                  "the trace's average duration; instructions per wave = SQ_INSTS_* / SQ_WAVES; LDS bank conflicts "
                  "= SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE.", "",
                  "| kernel | MfmaUtil | VALUBusy | bf16 MFMA TFLOP/s | waves | VALU / wave | SALU / wave | "
                  "LDS / wave | MFMA / wave | LDS conflict cycles |", "|---|---|---|---|---|---|---|---|---|---|"]
        for k in sorted(util["MfmaUtil"]):
            if k not in KERNEL_SOURCES_BY_NAME:
                continue
            waves = inst["SQ_WAVES"].get(k, 0.0) or float("nan")
            tflops = util["SQ_INSTS_VALU_MFMA_MOPS_BF16"].get(k, 0.0) * 512 / (avg_ns.get(k, float("nan")) * 1e-9) / 1e12
            conflict = inst["SQ_LDS_BANK_CONFLICT"].get(k, 0.0) / max(1.0, inst["SQ_LDS_IDX_ACTIVE"].get(k, 0.0))
            lines.append(f"| {k} | {util['MfmaUtil'][k]:.1f}% | {util['VALUBusy'].get(k, float('nan')):.1f}% | "
                         f"{tflops:.1f} | {waves:.0f} | {inst['SQ_INSTS_VALU'].get(k, 0) / waves:.0f} | "
                         f"{inst['SQ_INSTS_SALU'].get(k, 0) / waves:.0f} | {inst['SQ_INSTS_LDS'].get(k, 0) / waves:.0f} | "
                         f"{inst['SQ_INSTS_MFMA'].get(k, 0) / waves:.0f} | {100 * conflict:.1f}% |")
            if f"{k}@{w.name}" in entries:
                entries[f"{k}@{w.name}"].update({"mfma_util_pct": util["MfmaUtil"][k],
                                                 "valu_busy_pct": util["VALUBusy"].get(k),
                                                 "bf16_mfma_tflops": tflops})
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"lisa_forward_{commands.get('name', w.name)}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        c = {}
    c.pop("source_hash", None)
    c.setdefault("kernels", {})
    c["kernels"] = {k: e for k, e in c["kernels"].items() if "source_hash" in e}
    c["kernels"].update(entries)
    c["copy_calibration"] = {"fetch_scale": f_scale, "write_scale": w_scale}
    with open(COUNTERS, "w") as f:
        json.dump(c, f, indent=1)


def write_phases_profile(w, rec, command):
    """profiles/lisa_forward_phases_<workload>.md from a phases_timing record:
    each stage's median, 90th-percentile and latest end time over the workgroups, the
    interval since the previous stage's median end, and, where a stage moves
    HBM bytes, those bytes over that interval."""
    G, BH = rec["ranks_per_slice"], w.B * w.heads
    esize = 2 if w.dtype == "bf16" else 4
    tok = BH * w.n
    mat = 64 * 64 * 4
    inputs = tok * (3 * 64 * esize + (4 * w.T if w.mode == "adaptive" else 0))
    nstat = 2 if w.T >= 3 else 1
    direct = G == 1
    # (stage, what moves to or from HBM in the interval that ends with it, bytes)
    order = [("start", "", 0),
             ("staged", "Q, K, V, weights read (algorithmic bytes; the halo cells come on top)", inputs),
             ("kvsweep", "", 0),
             ("kv", "partials of s and phi(K)^T V written" if not direct else "s, phi(K)^T V written",
              BH * (G * (mat + 256) if not direct else mat + 256)),
             ("local", "", 0),
             ("s", "s partials read" if not direct else "", BH * G * 256 if not direct else 0),
             ("m", "partials of M written" if not direct else "M written", BH * G * mat if w.T >= 3 else 0),
             ("mwait", "", 0),
             ("cstaged", "every partial read once (by the rank that sums it)", 0 if direct else BH * G * nstat * mat),
             ("csummed", "", 0),
             ("combine", "the statistics written (fp32 rows and bf16 fragments)", 0 if direct else BH * nstat * mat * 3 // 2),
             ("cwait", "", 0),
             ("frags", "the statistics' bf16 fragments read by every rank", 0 if direct else BH * G * nstat * mat // 2),
             ("out", "", 0),
             ("end", "Y written (interval from the fragments' end: the output stage)", tok * 64 * esize)]
    since = {"end": "frags", "cstaged": "mwait"}  # intervals that start earlier than the previous row
    st = rec["stages"]
    lines = [f"# Stage timeline of the resident kernel, workload {w.describe()}", "",
             f"command: {command}", "",
             f"lisa_forward_phases: every workgroup stamps the device's 100 MHz clock (s_memrealtime) as its "
             f"wave 0 reaches each stage of its first slice; times are from the first workgroup's start, "
             f"median, 90th percentile and maximum over the {rec['workgroups']} working workgroups, averaged over "
             f"{rec['calls']} cold calls.  {G} rank(s) per slice.  Wave 0 is the oldest wave and finishes a "
             f"stage first: a stage's end for the whole workgroup is nearer the next stage's start.  The "
             f"interval of a stage runs from the previous listed stage's median; the bytes are those the "
             f"interval moves to or from HBM for the whole launch.", "",
             "| stage | median end us | p90 end us | max end us | interval us | HBM traffic in the interval | MB | GB/s |",
             "|---|---|---|---|---|---|---|---|"]
    prev = None
    for name, what, nbytes in order:
        m = st.get(name, {}).get("median_us")
        if m is None:
            continue
        q, mx = st[name]["p90_us"], st[name].get("max_us")
        mxs = "" if mx is None else f"{mx:.2f}"
        base = st.get(since.get(name, ""), {}).get("median_us")
        dt = None if prev is None else m - (base if base is not None else prev)
        rate = f"{nbytes / (dt * 1e-6) / 1e9:.0f}" if nbytes and dt and dt > 0 else ""
        lines.append(f"| {name} | {m:.2f} | {q:.2f} | {mxs} | {'' if dt is None else f'{dt:.2f}'} | {what} | "
                     f"{nbytes / 1e6:.2f} | {rate} |" if nbytes else
                     f"| {name} | {m:.2f} | {q:.2f} | {mxs} | {'' if dt is None else f'{dt:.2f}'} | {what} | | |")
        prev = m
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"lisa_forward_phases_{w.name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_backward(outdir, workload, command):
    """profiles/ summary of a rocprofv3 kernel trace of bench.py --backward-only."""
    from vision_transformer_token_amd import workloads

    w = workloads.get(workload)
    stats = _csv_rows(os.path.join(outdir, "prof_bwd", "bwd_kernel_stats.csv"))
    calls = None
    lines = [f"# rocprofv3 kernel trace of lisa_backward, workload {w.describe()}", "",
             f"command: {command}", "",
             "| kernel | calls | average ns | min ns | max ns | share |", "|---|---|---|---|---|---|"]
    total_ns = 0.0
    for r in stats:
        name = _short(r["Name"])
        if not (name.startswith("bwd_") or name in KERNEL_SOURCES_BY_NAME):
            continue
        calls = calls or int(r["Calls"])
        total_ns += float(r["AverageNs"])
        lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} | "
                     f"{float(r['Percentage']):.1f}% |")
    bb = compulsory_bytes_backward(w)
    lines += ["", f"sum of the kernels' averages per call: {total_ns / 1e3:.1f} us "
                  f"(the forward kernel, {' or '.join(KERNEL_SOURCES_BY_NAME)}, is the statistics launch the backward starts with)",
              f"algorithmic bytes per call: {w.token_heads * bb / 1e6:.2f} MB ({bb} B per token-head); "
              f"at 8 TB/s: {w.token_heads * bb / 8e12 * 1e6:.1f} us",
              f"kernel source hash (statistics launch and backward sources): {kernel_source_hash(BACKWARD_SOURCES)}"]
    with open(os.path.join(ROOT, "profiles", f"lisa_backward_{w.name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def compulsory_bytes_layer(w):
    """Per token (not token-head): the layer input X read and its output Y
    written once (C = 64 heads channels each), and the adaptive weights read
    (4 T bytes per token-head).  Q, K, V and the heads' outputs, which the
    unfused layer keeps in HBM, are not counted: they count against it."""
    esize = 2 if w.dtype == "bf16" else 4
    C = 64 * w.heads
    return 2 * C * esize + (4 * w.T * w.heads if w.mode == "adaptive" else 0)


def summarize_layer(outdir, workload, command):
    """profiles/ summary of a rocprofv3 kernel trace of bench.py --layer-only."""
    from vision_transformer_token_amd import workloads

    w = workloads.get(workload)
    stats = _csv_rows(os.path.join(outdir, "prof_layer", "layer_kernel_stats.csv"))
    lines = [f"# rocprofv3 kernel trace of lisa_attention_forward (QKV projection, LiSA, output projection), "
             f"workload {w.describe()}, C = {64 * w.heads}", "", f"command: {command}", "",
             "| kernel | calls | average ns | min ns | max ns | share |", "|---|---|---|---|---|---|"]
    total_ns = 0.0
    for r in stats:
        name = _short(r["Name"])
        if not (name in KERNEL_SOURCES_BY_NAME or name.startswith("proj_")):
            continue
        total_ns += float(r["AverageNs"])
        lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} | "
                     f"{float(r['Percentage']):.1f}% |")
    bb = compulsory_bytes_layer(w)
    tok = w.B * w.n
    lines += ["", f"sum of the kernels' averages per call: {total_ns / 1e3:.1f} us",
              f"algorithmic bytes per call: {tok * bb / 1e6:.2f} MB ({bb} B per token: X read, Y written, "
              f"weights); at 8 TB/s: {tok * bb / 8e12 * 1e6:.1f} us",
              f"kernel source hash (operator and projection sources): {kernel_source_hash(LAYER_SOURCES)}"]
    # Counter passes over the same run, when present: utilisation, then HBM
    # bytes scaled by the copy calibration stored with the forward's counters.
    util_csv = os.path.join(outdir, "pmc_layer_util", "util_counter_collection.csv")
    if os.path.exists(util_csv):
        def per_kernel(path, counter):
            acc = {}
            for r in _csv_rows(path):
                if r["Counter_Name"] == counter:
                    acc.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
            return {k: sum(v) / len(v) for k, v in acc.items()}
        avg_ns = {_short(r["Name"]): float(r["AverageNs"]) for r in stats}
        mfma = per_kernel(util_csv, "MfmaUtil")
        valu = per_kernel(util_csv, "VALUBusy")
        mops = per_kernel(util_csv, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
        fetch = per_kernel(os.path.join(outdir, "pmc_layer_fetch", "fetch_counter_collection.csv"), "FETCH_SIZE")
        write = per_kernel(os.path.join(outdir, "pmc_layer_write", "write_counter_collection.csv"), "WRITE_SIZE")
        with open(COUNTERS) as f:
            cal = json.load(f)["copy_calibration"]
        run = "python3 bench.py --layer-only --steps 10 --warmup 2 --no-cpu-baseline --workload " + w.name
        lines += ["", "# Utilisation and HBM traffic per launch (rocprofv3 --pmc, one pass each)", "",
                  f"utilisation pass: rocprofv3 --pmc MfmaUtil VALUBusy SQ_INSTS_VALU_MFMA_MOPS_BF16 --output-format csv "
                  f"-d gpurun_out/pmc_layer_util -o util -- {run}",
                  f"traffic passes: rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv "
                  f"-d gpurun_out/pmc_layer_fetch -o fetch (pmc_layer_write -o write) -- {run}",
                  f"FETCH_SIZE scaled by {cal['fetch_scale']:.3f} and WRITE_SIZE by {cal['write_scale']:.3f} "
                  "(the plain-copy calibration in profiles/counters.json).", "",
                  "| kernel | MfmaUtil | VALUBusy | bf16 MFMA TFLOP/s | HBM bytes (scaled) | GB/s |", "|---|---|---|---|---|---|"]
        for k in sorted(mfma):
            if not (k in KERNEL_SOURCES_BY_NAME or k.startswith("proj_")):
                continue
            ns = avg_ns.get(k, float("nan"))
            hbm = fetch.get(k, float("nan")) * 1024 * cal["fetch_scale"] + write.get(k, float("nan")) * 1024 * cal["write_scale"]
            tflops = mops.get(k, 0.0) * 512 / (ns * 1e-9) / 1e12
            lines.append(f"| {k} | {mfma[k]:.1f}% | {valu.get(k, float('nan')):.1f}% | {tflops:.1f} | "
                         f"{hbm / 1e6:.2f} MB | {hbm / ns:.0f} |")
    with open(os.path.join(ROOT, "profiles", f"lisa_attention_forward_{w.name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_mlp(outdir, workload, command):
    """profiles/ summary of a rocprofv3 kernel trace of bench.py --mlp-only."""
    from vision_transformer_token_amd import workloads

    w = workloads.get(workload)
    stats = _csv_rows(os.path.join(outdir, "prof_mlp", "mlp_kernel_stats.csv"))
    lines = [f"# rocprofv3 kernel trace of lisa_forward_mlp (walk weights predicted, hidden 64), "
             f"workload {w.describe()}", "", f"command: {command}", "",
             "| kernel | calls | average ns | min ns | max ns | share |", "|---|---|---|---|---|---|"]
    total_ns = 0.0
    for r in stats:
        name = _short(r["Name"])
        if not (name.startswith("flow_kernel") or name == "resident_kernel" or name.startswith("mlp_prep")):
            continue
        total_ns += float(r["AverageNs"])
        lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} | "
                     f"{float(r['Percentage']):.1f}% |")
    bb = compulsory_bytes_per_token_head(w) - (4 * w.T if w.mode == "adaptive" else 0)
    lines += ["", f"sum of the kernels' averages per call: {total_ns / 1e3:.1f} us "
                  f"(mlp_prep lays W1 out for the kernel's lanes)",
              f"algorithmic bytes per call: {w.token_heads * bb / 1e6:.2f} MB ({bb} B per token-head: "
              f"no weight tensor); at 8 TB/s: {w.token_heads * bb / 8e12 * 1e6:.1f} us",
              f"kernel source hash (operator sources): {kernel_source_hash(KERNEL_SOURCES_BY_NAME['resident_kernel'])}"]
    with open(os.path.join(ROOT, "profiles", f"lisa_forward_mlp_{w.name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--forward-only", action="store_true",
                    help="skip the reduce/apply reference timing (profiling runs: every "
                         "launch of the kernel is then a forward)")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only lisa_backward (for a profiler run) and print its line")
    ap.add_argument("--layer-only", action="store_true",
                    help="time only lisa_attention_forward (for a profiler run) and print its line")
    ap.add_argument("--summarize-layer", metavar="DIR",
                    help="write the profiles/ summary of a layer kernel trace under DIR and exit")
    ap.add_argument("--mlp-only", action="store_true",
                    help="time only lisa_forward_mlp (predicted walk weights) and print its line")
    ap.add_argument("--phases", action="store_true",
                    help="print the stage timeline of lisa_forward_phases over --steps cold calls and exit")
    ap.add_argument("--phases-profile", action="store_true",
                    help="with --phases: also write profiles/lisa_forward_phases_<workload>.md")
    ap.add_argument("--schedule", default="auto", choices=["auto", "streaming", "resident"],
                    help="forward kernel (lisa_schedule); auto is the library's choice")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="instead of LiSA, run 20 plain device copies of this many MiB "
                         "(the known-size kernel that scales the FETCH_SIZE/WRITE_SIZE counters)")
    ap.add_argument("--summarize-mlp", metavar="DIR",
                    help="write the profiles/ summary of a lisa_forward_mlp kernel trace under DIR and exit")
    ap.add_argument("--summarize-backward", metavar="DIR",
                    help="write the profiles/ summary of a backward kernel trace under DIR and exit")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write profiles/ summaries from rocprofv3 output under DIR and exit")
    args = ap.parse_args()

    if args.summarize_profiles:
        fixed = ("python3 bench.py --steps {s} --warmup {w} --no-cpu-baseline --forward-only --workload "
                 + args.workload + ("" if args.schedule == "auto" else " --schedule " + args.schedule))
        summarize_profiles(args.summarize_profiles, args.workload, {
            "name": args.workload + ("" if args.schedule == "auto" else "_" + args.schedule),
            "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_trace "
                     "-o trace -- " + fixed.format(s=200, w=20),
            "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o fetch -- "
                     + fixed.format(s=10, w=2),
            "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o write -- "
                     + fixed.format(s=10, w=2),
            "copy": "rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE --output-format csv -d gpurun_out/pmc_copy_{fetch|write} "
                    "-o c{fetch|write} -- python3 bench.py --calibrate-copy-mib 256",
            "copy_mib": 256,
            "util": "rocprofv3 --pmc MfmaUtil VALUBusy SQ_INSTS_VALU_MFMA_MOPS_BF16 --output-format csv "
                    "-d gpurun_out/pmc_util -o util -- " + fixed.format(s=10, w=2),
            "insts": "rocprofv3 --pmc SQ_WAVES SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_INSTS_MFMA "
                     "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE --output-format csv -d gpurun_out/pmc_insts -o insts -- "
                     + fixed.format(s=10, w=2),
        })
        return

    if args.summarize_layer:
        summarize_layer(args.summarize_layer, args.workload,
                        "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_layer -o layer -- "
                        "python3 bench.py --layer-only --steps 100 --warmup 10 --no-cpu-baseline --workload "
                        + args.workload)
        return

    if args.summarize_mlp:
        summarize_mlp(args.summarize_mlp, args.workload,
                      "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_mlp -o mlp -- "
                      "python3 bench.py --mlp-only --steps 100 --warmup 10 --no-cpu-baseline --workload "
                      + args.workload)
        return

    if args.summarize_backward:
        summarize_backward(args.summarize_backward, args.workload,
                           "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_bwd -o bwd -- "
                           "python3 bench.py --backward-only --steps 100 --warmup 10 --no-cpu-baseline --workload "
                           + args.workload)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the LiSA path "
              "shards by (batch, head) or by grid-row bands without collectives in this build.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from vision_transformer_token_amd import lisa, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.calibrate_copy_mib:
        nbytes = args.calibrate_copy_mib << 20
        src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(20):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": 20}))
        return
    w = workloads.get(args.workload)
    x = workloads.make_inputs(w)
    stream = torch.cuda.Stream(dev)

    # Q, K, V, Y and the adaptive weights of one input set.
    per_set = sum(t.numel() * t.element_size() for t in (x["q"], x["k"], x["v"], x["v"])
                  ) + (0 if x["weights"] is None else x["weights"].numel() * 4)
    nsets = max(2, -(-ROTATE_BYTES // per_set))
    sets = []
    with torch.cuda.stream(stream):
        for _ in range(nsets):
            d = {key: (x[key].to(dev) if x[key] is not None else None)
                 for key in ("q", "k", "v", "weights", "alpha")}
            d["y"] = torch.empty_like(d["v"])
            sets.append(d)
        prob = lisa.make_problem(sets[0]["q"], sets[0]["v"], grid=(w.H, w.W), T=w.T, eps=w.eps,
                                 schedule=args.schedule)
        ws = lisa.new_workspace(prob, dev)
    torch.cuda.synchronize()
    kernel_name = KERNELS[lisa.lisa_forward_schedule(prob)]

    def forward(d):
        lisa.lisa_forward(d["q"], d["k"], d["v"], grid=(w.H, w.W), T=w.T, alpha=d["alpha"],
                          weights=d["weights"], beta=x["beta"], eps=w.eps, out=d["y"], workspace=ws,
                          stream=stream, schedule=args.schedule)

    def reduce(d):
        lisa.lisa_reduce(d["q"], d["k"], d["v"], grid=(w.H, w.W), eps=w.eps, T=w.T, workspace=ws,
                         outputs=False, stream=stream, schedule=args.schedule)

    def apply(d):
        lisa.lisa_apply(d["q"], d["k"], d["v"], grid=(w.H, w.W), T=w.T, alpha=d["alpha"],
                        weights=d["weights"], beta=x["beta"], eps=w.eps, out=d["y"], workspace=ws,
                        stream=stream, schedule=args.schedule)

    def backward_timing(steps, warmup, pairs=True):
        """lisa_backward over the same input sets (dY drawn once per set); with
        ``pairs``, also forward + backward pairs (the profiler run leaves them out,
        so that its trace holds lisa_backward's launches only)."""
        bws = torch.zeros(lisa.lisa_backward_workspace_size(prob), dtype=torch.uint8, device=dev)
        with torch.cuda.stream(stream):
            dys = [torch.randn(d["v"].shape, device=dev, dtype=torch.float32).to(d["v"].dtype) for d in sets]
            outs = [{"dq": torch.empty_like(d["q"]), "dk": torch.empty_like(d["k"]), "dv": torch.empty_like(d["v"]),
                     "dweights": None if d["weights"] is None else torch.empty_like(d["weights"]),
                     "dalpha": torch.empty_like(d["alpha"])} for d in sets]
        torch.cuda.synchronize()

        def bwd(j):
            d = sets[j]
            lisa.lisa_backward(d["q"], d["k"], d["v"], dys[j], grid=(w.H, w.W), T=w.T, alpha=d["alpha"],
                               weights=d["weights"], beta=x["beta"], eps=w.eps, workspace=bws, out=outs[j],
                               stream=stream)

        for i in range(warmup):
            bwd(i % nsets)
        ba, bz = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ba.record(stream)
        for i in range(steps):
            bwd(i % nsets)
        bz.record(stream)
        torch.cuda.synchronize()
        ms = ba.elapsed_time(bz) / steps
        bb = compulsory_bytes_backward(w)

        # A training step's pair: the forward, then the backward on its
        # workspace, either recomputing the statistics (lisa_backward) or
        # taking the forward's (lisa_backward_after_forward).
        def pair(j, after):
            d = sets[j]
            lisa.lisa_forward(d["q"], d["k"], d["v"], grid=(w.H, w.W), T=w.T, alpha=d["alpha"],
                              weights=d["weights"], beta=x["beta"], eps=w.eps, out=d["y"], workspace=bws,
                              stream=stream)
            fn = lisa.lisa_backward_after_forward if after else lisa.lisa_backward
            fn(d["q"], d["k"], d["v"], dys[j], grid=(w.H, w.W), T=w.T, alpha=d["alpha"], weights=d["weights"],
               beta=x["beta"], eps=w.eps, workspace=bws, out=outs[j], stream=stream)

        pair_ms = {False: None, True: None}
        for after in ((False, True) if pairs else ()):
            for i in range(min(warmup, 20)):
                pair(i % nsets, after)
            torch.cuda.synchronize()
            ba.record(stream)
            for i in range(steps):
                pair(i % nsets, after)
            bz.record(stream)
            torch.cuda.synchronize()
            pair_ms[after] = ba.elapsed_time(bz) / steps
        return {"ms_per_step": ms, "value": w.token_heads / (ms * 1e-3), "unit": "token-heads/s",
                "steps": steps, "algorithmic_bytes_per_call": w.token_heads * bb,
                "roofline_frac": w.token_heads * bb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "forward_backward_ms": pair_ms[False], "forward_backward_after_forward_ms": pair_ms[True]}

    def mlp_timing(steps, warmup, hidden=64):
        """lisa_forward_mlp over the same input sets: the walk weights predicted
        inside the output pass (two-layer MLP of width ``hidden``) instead of read."""
        prm = {k: t.to(dev) for k, t in workloads.mlp_params(w.heads, hidden, w.T, d_h=w.d_h, seed=5).items()}
        mws = torch.zeros(lisa.lisa_forward_mlp_workspace_size(prob, hidden), dtype=torch.uint8, device=dev)
        with torch.cuda.stream(stream):
            ys = [torch.empty_like(d["v"]) for d in sets]
        torch.cuda.synchronize()

        def fwd(j):
            d = sets[j]
            lisa.lisa_forward_mlp(d["q"], d["k"], d["v"], grid=(w.H, w.W), T=w.T, alpha=d["alpha"], eps=w.eps,
                                  workspace=mws, out=ys[j], stream=stream, **prm)

        for i in range(warmup):
            fwd(i % nsets)
        ma, mz = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ma.record(stream)
        for i in range(steps):
            fwd(i % nsets)
        mz.record(stream)
        torch.cuda.synchronize()
        ms = ma.elapsed_time(mz) / steps
        # Compulsory bytes without the weight tensor: Q, K, V read, Y written.
        bb = compulsory_bytes_per_token_head(w) - (4 * w.T if w.mode == "adaptive" else 0)
        return {"ms_per_step": ms, "value": w.token_heads / (ms * 1e-3), "unit": "token-heads/s", "steps": steps,
                "hidden": hidden, "algorithmic_bytes_per_call": w.token_heads * bb,
                "roofline_frac": w.token_heads * bb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}

    def layer_timing(steps, warmup):
        """lisa_attention_forward (QKV projection, LiSA, output projection) at the
        workload's shape, C = 64 heads channels, over rotating layer inputs."""
        prm = workloads.layer_params(w)
        dp = {k: t.to(dev) for k, t in prm.items() if k != "x"}
        lws = torch.zeros(lisa.lisa_attention_workspace_size(prob), dtype=torch.uint8, device=dev)
        with torch.cuda.stream(stream):
            xs = [prm["x"].to(dev) for _ in range(nsets)]
            ys = [torch.empty_like(xx) for xx in xs]
        torch.cuda.synchronize()

        def layer(j):
            d = sets[j]
            lisa.lisa_attention_forward(xs[j], dp["w_qkv"], dp["b_qkv"], dp["w_o"], dp["b_o"], heads=w.heads,
                                        grid=(w.H, w.W), T=w.T, alpha=d["alpha"], weights=d["weights"],
                                        beta=x["beta"], eps=w.eps, out=ys[j], workspace=lws, stream=stream)

        for i in range(warmup):
            layer(i % nsets)
        la, lz = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        la.record(stream)
        for i in range(steps):
            layer(i % nsets)
        lz.record(stream)
        torch.cuda.synchronize()
        ms = la.elapsed_time(lz) / steps
        bb = compulsory_bytes_layer(w)
        tok = w.B * w.n
        return {"ms_per_step": ms, "value": w.token_heads / (ms * 1e-3), "unit": "token-heads/s", "steps": steps,
                "channels": 64 * w.heads, "algorithmic_bytes_per_call": tok * bb,
                "roofline_frac": tok * bb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}

    def workloads_timing(steps, warmup):
        """lisa_forward on every other workload preset, each over its own
        rotating input sets (more than twice the Infinity Cache, so calls start
        cold), timed like the headline: events around `steps` back-to-back
        calls on the bench stream.  The long-range and square-grid presets are
        where the spec bar (n >= 3136) applies besides the headline one."""
        rec = {}
        for name in ("long_range_200x320", "square_64x64", "square_128x128", "square_256x256",
                     "deit_t_224", "deit_t_384", "deit_t_384_t5"):
            ow = workloads.get(name)
            ox = workloads.make_inputs(ow)
            oper = sum(t.numel() * t.element_size() for t in (ox["q"], ox["k"], ox["v"], ox["v"])) + (
                0 if ox["weights"] is None else ox["weights"].numel() * 4)
            on = max(2, -(-ROTATE_BYTES // oper))
            with torch.cuda.stream(stream):
                osets = []
                for _ in range(on):
                    d = {key: (ox[key].to(dev) if ox[key] is not None else None)
                         for key in ("q", "k", "v", "weights", "alpha")}
                    d["y"] = torch.empty_like(d["v"])
                    osets.append(d)
                oprob = lisa.make_problem(osets[0]["q"], osets[0]["v"], grid=(ow.H, ow.W), T=ow.T, eps=ow.eps)
                ows = lisa.new_workspace(oprob, dev)
            torch.cuda.synchronize()

            def timed(schedule):
                def ofwd(d):
                    lisa.lisa_forward(d["q"], d["k"], d["v"], grid=(ow.H, ow.W), T=ow.T, alpha=d["alpha"],
                                      weights=d["weights"], beta=ox["beta"], eps=ow.eps, out=d["y"],
                                      workspace=ows, stream=stream, schedule=schedule)

                for i in range(warmup):
                    ofwd(osets[i % on])
                oa, oz = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                oa.record(stream)
                for i in range(steps):
                    ofwd(osets[i % on])
                oz.record(stream)
                torch.cuda.synchronize()
                return oa.elapsed_time(oz) / steps

            ms = timed(args.schedule)
            # Each kernel alone, where it takes the problem: the evidence for
            # the library's default.
            by = {}
            for sched in ("streaming", "resident"):
                try:
                    lisa.lisa_forward_schedule(lisa.make_problem(osets[0]["q"], osets[0]["v"], grid=(ow.H, ow.W),
                                                                 T=ow.T, eps=ow.eps, schedule=sched))
                    by[sched] = timed(sched)
                except lisa.LisaError:
                    by[sched] = None
            bb = compulsory_bytes_per_token_head(ow)
            rec[name] = {"ms_per_step": ms, "value": ow.token_heads / (ms * 1e-3), "unit": "token-heads/s",
                         "steps": steps, "token_heads": ow.token_heads, "n": ow.n, "T": ow.T,
                         "kernel": KERNELS[lisa.lisa_forward_schedule(lisa.make_problem(
                             osets[0]["q"], osets[0]["v"], grid=(ow.H, ow.W), T=ow.T, eps=ow.eps,
                             schedule=args.schedule))],
                         "ms_per_step_by_schedule": by,
                         "algorithmic_bytes_per_call": ow.token_heads * bb,
                         "roofline_frac": ow.token_heads * bb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
            del osets, ows
            torch.cuda.synchronize()
        return rec

    def phases_timing(calls, warmup):
        """The stage timeline of lisa_forward_phases over `calls` cold calls
        (rotating input sets): per stage, the median, 90th percentile and
        maximum over the active workgroups of the time since the first workgroup started,
        averaged over the calls, in microseconds."""
        import numpy as np

        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        stamps = torch.zeros(cus * lisa.LISA_PHASES, dtype=torch.int64, device=dev)

        def call(d):
            lisa.lisa_forward_phases(d["q"], d["k"], d["v"], grid=(w.H, w.W), T=w.T, alpha=d["alpha"],
                                     weights=d["weights"], beta=x["beta"], eps=w.eps, out=d["y"], workspace=ws,
                                     stream=stream, stamps=stamps)

        for i in range(warmup):
            forward(sets[i % nsets])
        med, p90, mx, rows = [], [], [], None
        for i in range(calls):
            stamps.fill_(0)
            torch.cuda.synchronize()
            call(sets[i % nsets])
            torch.cuda.synchronize()
            st = stamps.view(cus, lisa.LISA_PHASES).cpu().numpy()
            active = st[:, 0] > 0
            rank = st[:, lisa.LISA_PHASES - 1]
            active &= (rank >> 32) != 0xFFFFFFFF  # idle workgroups carry group -1
            a_st = st[active][:, :len(lisa.STAGES)].astype(np.float64)
            t0 = a_st[:, 0].min()
            rel = (a_st - t0) / 100.0  # 100 MHz clock -> microseconds
            rel[a_st == 0] = np.nan  # stages the problem does not have
            med.append(np.nanmedian(rel, axis=0))
            p90.append(np.nanpercentile(rel, 90, axis=0))
            mx.append(np.nanmax(rel, axis=0))
            rows = int(active.sum())
            ranks = int((rank[active] & 0xFFFFFFFF).max()) + 1
        med, p90, mx = (np.nanmean(np.array(v), axis=0) for v in (med, p90, mx))

        def us(v):
            return None if np.isnan(v) else round(float(v), 3)

        return {"workgroups": rows, "calls": calls, "ranks_per_slice": ranks,
                "stages": {name: {"median_us": us(m), "p90_us": us(q), "max_us": us(z)}
                           for name, m, q, z in zip(lisa.STAGES, med, p90, mx)}}

    if args.phases:
        rec = phases_timing(args.steps, args.warmup)
        print(json.dumps({"workload": w.name, "phases": rec}), flush=True)
        if args.phases_profile:
            write_phases_profile(w, rec, "python3 bench.py --phases --phases-profile --steps "
                                 f"{args.steps} --warmup {args.warmup} --workload {w.name}")
        return

    if args.backward_only:
        print(json.dumps({"workload": w.name, "backward": backward_timing(args.steps, args.warmup, pairs=False)}),
              flush=True)
        return
    if args.mlp_only:
        print(json.dumps({"workload": w.name, "forward_mlp": mlp_timing(args.steps, args.warmup)}), flush=True)
        return
    if args.layer_only:
        print(json.dumps({"workload": w.name, "layer": layer_timing(args.steps, args.warmup)}), flush=True)
        return

    for i in range(args.warmup):
        forward(sets[i % nsets])
    torch.cuda.synchronize()

    # Timed region: K whole forward passes, with events at the boundaries of
    # five equal segments (median of the five reported beside the total).
    seg = [i * args.steps // 5 for i in range(6)]
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    torch.cuda.synchronize()
    marks[0].record(stream)
    for i in range(args.steps):
        forward(sets[i % nsets])
        if i + 1 in seg[1:]:
            marks[seg.index(i + 1)].record(stream)
    torch.cuda.synchronize()
    step_ms = marks[0].elapsed_time(marks[5]) / args.steps
    seg_ms = sorted(marks[j].elapsed_time(marks[j + 1]) / max(1, seg[j + 1] - seg[j]) for j in range(5))

    # The same calls captured once into a HIP graph (one forward per input
    # set) and replayed: launch overhead off the host's critical path.
    graph_ms = None
    if not args.forward_only:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for d in sets:
                forward(d)
        reps = max(1, args.steps // nsets)
        g.replay()
        torch.cuda.synchronize()
        ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cur = torch.cuda.current_stream(dev)
        ga.record(cur)
        for _ in range(reps):
            g.replay()
        gb.record(cur)
        torch.cuda.synchronize()
        graph_ms = ga.elapsed_time(gb) / (reps * nsets)
        del g

    # A plain device copy on the same box: the bandwidth a streaming kernel
    # actually gets, for the path's fraction of it.
    copy_gbs = None
    if not args.forward_only:
        cb = 256 << 20
        src = torch.ones(cb // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        ca, cz = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ca.record()
        for _ in range(20):
            dst.copy_(src)
        cz.record()
        torch.cuda.synchronize()
        copy_gbs = 2 * cb * 20 / (ca.elapsed_time(cz) * 1e-3) / 1e9
        del src, dst

    # The same K forwards with events around each launch on the stream it runs
    # on: each launch in isolation (an event between launches adds a gap), for
    # comparison with the two halves below.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        ev[i][0].record(stream)
        forward(sets[i % nsets])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    kernel_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps

    # The two halves the C ABI also offers (statistics only; output from
    # stored statistics), timed the same way, for reference.
    stats_ms = apply_ms = None
    if w.T >= 2 and not args.forward_only:
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            d = sets[i % nsets]
            ev[i][0].record(stream)
            reduce(d)
            ev[i][1].record(stream)
            apply(d)
            ev[i][2].record(stream)
        torch.cuda.synchronize()
        stats_ms = sum(a.elapsed_time(b) for a, b, _ in ev) / args.steps
        apply_ms = sum(b.elapsed_time(c) for _, b, c in ev) / args.steps

    th = w.token_heads
    bpt = compulsory_bytes_per_token_head(w)
    value = th / (step_ms * 1e-3)
    path_gbs = th * bpt / (step_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "token-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "B": w.B,
            "heads": w.heads,
            "grid": f"{w.H}x{w.W}",
            "n": w.n,
            "d_h": w.d_h,
            "d_v": w.d_v,
            "T": w.T,
            "weights": w.mode,
            "token_heads": th,
            "rotating_input_sets": nsets,
        },
        "path_roofline_frac": path_gbs / HBM_PEAK_GBS,
        "ms_per_step_median5": seg_ms[2],
    }
    if graph_ms is not None:
        out["graph"] = {"ms_per_step": graph_ms, "value": th / (graph_ms * 1e-3)}
    if copy_gbs is not None:
        out["copy_gbs"] = copy_gbs
        out["path_copy_frac"] = path_gbs / copy_gbs
    if kernel_ms is not None:
        # One launch of the kernel per step, back to back on `stream`: its
        # average launch duration is the timed region's elapsed time (events
        # on that stream) over the K launches.
        achieved = th * bpt / (step_ms * 1e-3) / 1e9
        traffic = load_counters(w, kernel_name)
        out["roofline"] = {
            "bound": "hbm",
            "kernel": kernel_name,
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "kernel_ms": step_ms,
            "isolated_launch_ms": kernel_ms,
            "algorithmic_bytes_per_launch": th * bpt,
        }
        out["stages_ms"] = {"forward_kernel": kernel_ms, "reduce_only": stats_ms, "apply_only": apply_ms}
    if not args.forward_only:
        out["backward"] = backward_timing(min(args.steps, 500), min(args.warmup, 50))
        out["forward_mlp"] = mlp_timing(min(args.steps, 1000), min(args.warmup, 50))
        out["layer"] = layer_timing(min(args.steps, 500), min(args.warmup, 50))
        out["workloads"] = workloads_timing(min(max(args.steps, 200), 1000), max(args.warmup, 20))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
