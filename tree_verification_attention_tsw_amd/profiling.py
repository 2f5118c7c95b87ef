"""Text summaries of rocprofv3 output for this library's kernels.

Two kinds of summary, both short text files meant to be kept beside the
numbers they support:

* kernel timing: ``rocprofv3 --kernel-trace --stats`` output reduced to the
  calls, average, minimum and maximum duration of every ``tsw::`` kernel;
* HBM traffic: two ``rocprofv3 --pmc`` runs (``FETCH_SIZE``, then
  ``WRITE_SIZE``, KiB per dispatch) reduced to bytes per launch of one
  kernel, each counter scaled by what it reads for a plain float32
  elementwise copy of known size run in the same process (bench.py
  ``--copy-calibration-mib``).

The summaries record a digest of the split kernel's sources so that a
reader (bench.py) can tell whether the counters still describe the current
code.

    python -m tree_verification_attention_tsw_amd.profiling stats DIR OUT --command "..." \\
        [--window split_mfma FIRST COUNT] [--bench-log LOG]
    python -m tree_verification_attention_tsw_amd.profiling traffic FETCH_DIR WRITE_DIR OUT \\
        --kernel split_mfma --copy-mib 1024 --alg-bytes N --command "..." --command "..."
    python -m tree_verification_attention_tsw_amd.profiling counters OUT DIR... --kernel NAME \\
        --units-per-simd N --unit-name tile --command "..."
    python -m tree_verification_attention_tsw_amd.profiling power OUT --workload gqa8b_100k \\
        [--seconds 8] [--half-grid] --command "..."

A third kind of record, socket power under a sustained load: a call runs
back to back for some seconds while ``amd-smi metric`` reports the socket
power and the graphics clocks.  MI355X holds its socket power at a limit by
lowering the graphics clock, so at that limit a call's time follows its
energy rather than its cycle or byte count; the record gives the power, the
clocks and the energy per call (power x time) of the verify call and, for
comparison, of the read-stream kernel (the same K/V bytes through the same
LDS-DMA ring, no arithmetic).
"""
import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re
import shutil
import subprocess
import threading
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
COPY_KERNEL_MARK = "MulFunctor<float>"


# The split kernel's sources: its template, instantiation and dispatch
# units, the device helpers and the argument structures it is launched with.
SPLIT_KERNEL_SOURCES = ("tsw_mfma_impl.h", "tsw_mfma_inst.hip", "tsw_mfma.hip", "tsw_device.h", "tsw_internal.h")


def source_digest():
    """sha256 over the split kernel's sources (name + bytes, sorted)."""
    h = hashlib.sha256()
    files = sorted(os.path.join(PKG, "csrc", n) for n in SPLIT_KERNEL_SOURCES)
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _find(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError("no *%s under %s" % (suffix, d))
    return hits[-1]


def _is_ours(name):
    return "tsw::" in name or name.startswith("_ZN3tsw")


def _short(name):
    """'void tsw::mfma::split_mfma<8, 4, 3, false>(tsw::SplitArgs)' -> 'split_mfma<8, 4, 3, false>'."""
    if name.startswith("_ZN3tsw"):
        # mangled (a template in an anonymous namespace): the last of the
        # length-prefixed names of the nested-name, template arguments dropped
        i, last = 3, name
        while i < len(name) and name[i].isdigit():
            j = i
            while name[j].isdigit():
                j += 1
            n = int(name[i:j])
            last = name[j:j + n]
            i = j + n
        return last + "<...>"
    n = name.replace("(anonymous namespace)::", "").split("(")[0]
    if n.startswith("void "):
        n = n[5:]
    return n.split("::")[-1] if "tsw::" in n else n[:60]


def kernel_stats(d):
    rows = list(csv.DictReader(open(_find(d, "_kernel_stats.csv"))))
    out = []
    for r in rows:
        if not _is_ours(r["Name"]):
            continue
        out.append((_short(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                    float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    return out


def counter_rows(d):
    return list(csv.DictReader(open(_find(d, "_counter_collection.csv"))))


def per_dispatch(rows, counter, kernel_substr):
    """Counter values of every dispatch whose name contains kernel_substr."""
    vals = collections.OrderedDict()
    for r in rows:
        if r["Counter_Name"] != counter or kernel_substr not in r["Kernel_Name"]:
            continue
        key = int(r["Dispatch_Id"])
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return list(vals.values())


def copy_factor(rows, counter, copy_bytes):
    """Bytes per counted KiB, from the calibration copy (largest such dispatch)."""
    v = per_dispatch(rows, counter, COPY_KERNEL_MARK)
    if not v:
        raise ValueError("no calibration copy dispatch (%s) in the %s run" % (COPY_KERNEL_MARK, counter))
    kib = max(v)
    return copy_bytes / (kib * 1024.0), kib


def trace_durations(d, kernel_substr):
    """Durations (us) of the matching dispatches of a kernel trace, in start order."""
    rows = [r for r in csv.DictReader(open(_find(d, "_kernel_trace.csv")))
            if kernel_substr in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    return [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]


def bench_line(path):
    """The last JSON line a bench.py run printed."""
    last = None
    for line in open(path, errors="replace"):
        if line.startswith("{"):
            last = json.loads(line)
    if last is None:
        raise ValueError("no JSON line in %s" % path)
    return last


def write_stats(d, out, commands, window=None, bench_log=None):
    """Whole-run kernel statistics; `window` = (kernel, first, count) adds the
    mean over those dispatches of that kernel (the bench's timed steps), and
    `bench_log` the bench line's own split time for comparison."""
    lines = ["# rocprofv3 kernel durations of the tsw kernels", "commands:"]
    lines += ["  " + c for c in commands]
    lines.append("source_digest: %s" % source_digest())
    lines.append("%-44s %6s %10s %10s %10s" % ("kernel", "calls", "avg_us", "min_us", "max_us"))
    for name, calls, avg, mn, mx in kernel_stats(d):
        lines.append("%-44s %6d %10.2f %10.2f %10.2f" % (name, calls, avg, mn, mx))
    if window:
        kernel, first, count = window
        durs = trace_durations(d, kernel)[first:first + count]
        if len(durs) != count:
            raise ValueError("trace holds %d %s dispatches from %d, expected %d" % (len(durs), kernel, first, count))
        srt = sorted(durs)
        lines.append("timed steps (dispatches %d..%d of %s in start order): avg_us %.2f  median_us %.2f  "
                     "min_us %.2f  max_us %.2f" % (first, first + count - 1, kernel, sum(durs) / count,
                                                   srt[count // 2], srt[0], srt[-1]))
    if bench_log:
        b = bench_line(bench_log)
        keys = ("ms_per_step", "us_per_layer_call", "us_split", "us_split_median5")
        lines.append("bench line of the same run: " + ", ".join(
            "%s %s" % (k, b[k]) for k in keys if b.get(k) is not None)
            + (", roofline.us_per_launch %s" % b["roofline"]["us_per_launch"] if "roofline" in b else ""))
    _write(out, lines)


def write_traffic(fetch_dir, write_dir, out, kernel, copy_mib, alg_bytes, commands):
    copy_bytes = copy_mib * 2 ** 20
    fr, wr = counter_rows(fetch_dir), counter_rows(write_dir)
    ff, fkib = copy_factor(fr, "FETCH_SIZE", copy_bytes)
    wf, wkib = copy_factor(wr, "WRITE_SIZE", copy_bytes)
    fv = per_dispatch(fr, "FETCH_SIZE", kernel)
    wv = per_dispatch(wr, "WRITE_SIZE", kernel)
    if not fv or not wv:
        raise ValueError("no %s dispatches in the counter runs" % kernel)
    fb = sum(fv) / len(fv) * 1024.0 * ff
    wb = sum(wv) / len(wv) * 1024.0 * wf
    lines = ["# HBM traffic per launch of %s (rocprofv3 --pmc, copy-calibrated)" % kernel, "commands:"]
    lines += ["  " + c for c in commands]
    lines.append("source_digest: %s" % source_digest())
    lines.append("copy_calibration: %d bytes read and written; FETCH_SIZE %.1f KiB -> %.4f bytes/KiB-unit; "
                 "WRITE_SIZE %.1f KiB -> %.4f" % (copy_bytes, fkib, ff * 1024, wkib, wf * 1024))
    lines.append("dispatches: fetch run %d, write run %d" % (len(fv), len(wv)))
    lines.append("fetch_bytes_per_launch: %.0f" % fb)
    lines.append("write_bytes_per_launch: %.0f" % wb)
    lines.append("traffic_bytes_per_launch: %.0f" % (fb + wb))
    if alg_bytes:
        lines.append("alg_bytes_per_launch: %d" % alg_bytes)
        lines.append("traffic_over_alg: %.4f" % ((fb + wb) / alg_bytes))
    _write(out, lines)


def dispatch_durations(rows, kernel_substr):
    """Per-dispatch duration (us) of the matching dispatches of a counter run."""
    d = collections.OrderedDict()
    for r in rows:
        if kernel_substr in r["Kernel_Name"]:
            d[int(r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    return list(d.values())


def write_counters(dirs, out, kernel, simds, xcds, units_per_simd, unit_name, commands):
    """Average per-dispatch SQ/GRBM counters of `kernel` over several
    rocprofv3 --pmc runs, with the derived per-SIMD quantities."""
    vals = collections.OrderedDict()
    durs = []
    for d in dirs:
        rows = counter_rows(d)
        durs += dispatch_durations(rows, kernel)
        names = sorted(set(r["Counter_Name"] for r in rows))
        for c in names:
            v = per_dispatch(rows, c, kernel)
            if v:
                vals[c] = sum(v) / len(v)
    if not vals:
        raise ValueError("no %s dispatches in the counter runs" % kernel)
    dur = sum(durs) / len(durs)
    lines = ["# SQ / GRBM counters per dispatch of %s (rocprofv3 --pmc, kernels serialised)" % kernel, "commands:"]
    lines += ["  " + c for c in commands]
    lines.append("source_digest: %s" % source_digest())
    lines.append("dispatches: %d, mean duration under counter collection: %.2f us" % (len(durs), dur))
    lines.append("raw counters (mean per dispatch, summed over the device as rocprofv3 reports them):")
    for c, v in vals.items():
        lines.append("  %-32s %18.1f" % (c, v))
    lines.append("derived (%d SIMDs, %d XCDs, %g %s per SIMD):" % (simds, xcds, units_per_simd, unit_name))
    if "GRBM_GUI_ACTIVE" in vals:
        # GRBM_GUI_ACTIVE spans the whole collection window of a dispatch, so
        # this rate is not taken as the shader clock
        cyc = vals["GRBM_GUI_ACTIVE"] / xcds
        lines.append("  GRBM_GUI_ACTIVE / XCDs / duration = %.0f / %.2f us = %.2f per ns (collection window, "
                     "not the shader clock)" % (cyc, dur, cyc / (dur * 1e3)))
    if "SQ_VALU_MFMA_BUSY_CYCLES" in vals:
        busy = vals["SQ_VALU_MFMA_BUSY_CYCLES"] / simds
        lines.append("  MFMA busy cycles per SIMD: %.0f = %.1f%% of the kernel's cycles at 2.4 GHz, %.1f%% at 2.0 GHz"
                     % (busy, 100.0 * busy / (2.4 * dur * 1e3), 100.0 * busy / (2.0 * dur * 1e3)))
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in vals:
        lines.append("  cycles with an MFMA busy and a VALU instruction issued, per SIMD: %.0f"
                     % (vals["SQ_VALU_MFMA_COEXEC_CYCLES"] / simds))
    for c, label in (("SQ_INSTS_MFMA", "MFMA instructions"), ("SQ_INSTS_VALU", "VALU instructions (MFMA included)"),
                     ("SQ_INSTS_VALU_TRANS_F32", "transcendental (exp) instructions"),
                     ("SQ_INSTS_LDS", "LDS instructions"), ("SQ_INSTS_SALU", "SALU instructions")):
        if c in vals:
            lines.append("  %s per SIMD per %s: %.1f" % (label, unit_name, vals[c] / simds / units_per_simd))
    if "SQ_ACTIVE_INST_VALU" in vals:
        lines.append("  VALU-active cycles per SIMD (SQ_ACTIVE_INST_VALU x 4 / SIMDs): %.0f"
                     % (vals["SQ_ACTIVE_INST_VALU"] * 4 / simds))
    if "SQ_WAIT_INST_ANY" in vals and "SQ_WAVES" in vals:
        lines.append("  wave-cycles waiting to issue, per wave (SQ_WAIT_INST_ANY x 4 / waves): %.0f"
                     % (vals["SQ_WAIT_INST_ANY"] * 4 / vals["SQ_WAVES"]))
    if "SQ_LDS_BANK_CONFLICT" in vals:
        lines.append("  LDS bank-conflict cycles per CU: %.0f" % (vals["SQ_LDS_BANK_CONFLICT"] / (simds / 4)))
    _write(out, lines)


def read_traffic(path):
    """(traffic bytes per launch, digest) from a traffic summary, or None."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if "traffic_bytes_per_launch" not in kv or "source_digest" not in kv:
        return None
    return float(kv["traffic_bytes_per_launch"]), kv["source_digest"]


def _amd_smi():
    exe = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    return exe if os.path.exists(exe) else None


def smi_metric(timeout=30.0):
    """(socket power W, mean graphics clock MHz, per-XCD clocks) from one
    `amd-smi metric -p -c` of GPU 0, or None where the tool or a field is
    missing."""
    exe = _amd_smi()
    if exe is None:
        return None
    try:
        r = subprocess.run([exe, "metric", "-g", "0", "-p", "-c"], capture_output=True, text=True, timeout=timeout)
    except (OSError, subprocess.TimeoutExpired):
        return None
    return parse_smi_metric(r.stdout)


def parse_smi_metric(text):
    """(socket power W, mean graphics clock MHz, per-XCD clocks) from the
    text of `amd-smi metric -p -c`, or None."""
    m = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", text)
    clocks = [float(x) for x in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*([0-9.]+)\s*MHz", text)]
    if m is None or not clocks:
        return None
    return float(m.group(1)), sum(clocks) / len(clocks), clocks


def smi_power_limit(timeout=30.0):
    """The socket power cap in W from `rocm-smi --showmaxpower`, or None."""
    exe = shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi"
    if not os.path.exists(exe):
        return None
    try:
        r = subprocess.run([exe, "--showmaxpower"], capture_output=True, text=True, timeout=timeout)
    except (OSError, subprocess.TimeoutExpired):
        return None
    return parse_power_cap(r.stdout)


def parse_power_cap(text):
    m = re.search(r"Max Graphics Package Power \(W\):\s*([0-9.]+)", text)
    return float(m.group(1)) if m else None


def sustained(batch, seconds, samples=2, settle=None):
    """Run `batch()` (launches some calls, synchronises, returns the GPU
    microseconds per call it measured) back to back for `seconds`, and take
    `samples` amd-smi readings from a second thread once `settle` seconds
    (default: half the run) have passed, so the clocks and the power have
    reached their loaded state.  Returns a dict, or None without amd-smi."""
    if _amd_smi() is None:
        return None
    settle = seconds / 2 if settle is None else settle
    readings = []

    def sampler():
        time.sleep(settle)
        for _ in range(samples):
            got = smi_metric()
            if got is not None:
                readings.append(got)

    th = threading.Thread(target=sampler, daemon=True)
    per_call = []
    t0 = time.perf_counter()
    th.start()
    while time.perf_counter() - t0 < seconds or th.is_alive():
        us = batch()
        if time.perf_counter() - t0 >= settle:
            per_call.append(us)
        if time.perf_counter() - t0 > seconds + 120:
            break
    th.join(timeout=1.0)
    if not readings or not per_call:
        return None
    watts = sum(r[0] for r in readings) / len(readings)
    mhz = sum(r[1] for r in readings) / len(readings)
    per_call.sort()
    us = per_call[len(per_call) // 2]
    return {"us_per_call": round(us, 2), "socket_W": round(watts, 1), "gfx_MHz": round(mhz),
            "gfx_MHz_per_xcd": [round(c) for c in readings[-1][2]], "mJ_per_call": round(watts * us * 1e-3, 2),
            "samples": len(readings), "seconds": round(time.perf_counter() - t0, 1)}


def power_record(w, seconds=6.0, dev="cuda"):
    """Sustained-load power of one attention workload: the product verify
    call, then the read-stream kernel over the same caches."""
    import torch
    import tree_verification_attention_tsw_amd as tsw
    from tree_verification_attention_tsw_amd import workloads as wl
    n_sets = max(2, -(-int(1.5 * 2 ** 30) // w.kv_bytes()))
    sets = [wl.make_qkv(w, layer=i, device=dev) for i in range(n_sets)]
    parent = w.parent()
    q0, k0 = sets[0][0], sets[0][1]
    o = torch.empty((w.n_nodes, w.Hq, w.d), dtype=torch.float32, device=dev)
    lse = torch.empty((w.n_nodes, w.Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(tsw.workspace_size(q0, k0, w.n_prefix), dtype=torch.uint8, device=dev)
    sink = torch.zeros(64, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    kinds = {
        "verify": [tsw.prepare_verify(q, k, v, parent, w.n_prefix, o, lse, ws, stream=stream) for (q, k, v) in sets],
        "read_stream": [tsw.prepare_read_stream(q, k, v, w.n_prefix, sink, stream=stream) for (q, k, v) in sets],
    }
    out = {"workload": w.name, "limit_W": smi_power_limit()}
    for name, calls in kinds.items():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 200

        def batch():
            e0.record(stream)
            for i in range(n):
                calls[i % len(calls)]()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / n

        out[name] = sustained(batch, seconds)
    return out


def half_grid_record(w, seconds=6.0, dev="cuda", n_splits=32, repeat=False):
    """The split kernel alone, sustained, on the workload's grid (n_splits x
    Hkv work-groups) and on half of it: half the kv heads and query heads,
    so every work-group keeps its rows and keys but half the CUs idle
    (repeat: both once more, alternating)."""
    import torch
    import tree_verification_attention_tsw_amd as tsw
    from tree_verification_attention_tsw_amd import workloads as wl
    out = {}
    runs = [("full_grid", w.Hkv), ("half_grid", w.Hkv // 2)]
    if repeat:
        runs += [("full_grid_again", w.Hkv), ("half_grid_again", w.Hkv // 2)]
    for name, hkv in runs:
        ww = wl.Workload(w.name + "_hkv%d" % hkv, Hq=w.G * hkv, Hkv=hkv, d=w.d, n_prefix=w.n_prefix,
                         n_nodes=w.n_nodes, dtype=w.dtype, seed=w.seed, outliers=w.outliers)
        n_sets = max(2, -(-int(1.5 * 2 ** 30) // ww.kv_bytes()))
        sets = [wl.make_qkv(ww, layer=i, device=dev) for i in range(n_sets)]
        po = torch.empty((n_splits, ww.n_nodes, ww.Hq, ww.d), dtype=torch.float32, device=dev)
        pl = torch.empty((n_splits, ww.n_nodes, ww.Hq), dtype=torch.float32, device=dev)
        stream = torch.cuda.current_stream()
        calls = [tsw.prepare_split(q, k, v, ww.parent(), ww.n_prefix, n_splits, po, pl, stream=stream)
                 for (q, k, v) in sets]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

        def batch():
            e0.record(stream)
            for i in range(200):
                calls[i % len(calls)]()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / 200

        r = sustained(batch, seconds)
        if r is not None:
            r["work_groups"] = n_splits * hkv
        out[name] = r
        del sets, calls, po, pl
        torch.cuda.empty_cache()
    return out


def write_half_grid(out, workload, seconds, commands):
    from tree_verification_attention_tsw_amd import workloads as wl
    rec = half_grid_record(wl.WORKLOADS[workload], seconds, repeat=True)
    lines = ["# split kernel alone, sustained: the workload's grid and half of it (half the kv and query",
             "# heads: the same rows and keys per work-group, half the CUs idle); amd-smi metric -p -c, GPU 0"]
    lines += ["command: " + c for c in commands]
    lines += ["source_digest: %s" % source_digest(), "workload: %s" % workload]
    for name, r in rec.items():
        if r is None:
            lines.append("%s: amd-smi not available" % name)
            continue
        lines.append("%s: %d work-groups, %.2f us per launch, socket %.1f W, graphics clock %d MHz, %.2f mJ per launch"
                     % (name, r["work_groups"], r["us_per_call"], r["socket_W"], r["gfx_MHz"], r["mJ_per_call"]))
    _write(out, lines)


def write_power(out, workload, seconds, commands):
    from tree_verification_attention_tsw_amd import workloads as wl
    rec = power_record(wl.WORKLOADS[workload], seconds)
    lines = ["# socket power under a sustained load (amd-smi metric -p -c, GPU 0)"]
    lines += ["command: " + c for c in commands]
    lines += ["source_digest: %s" % source_digest(), "workload: %s" % workload,
              "power_limit_W: %s" % rec["limit_W"]]
    for name in ("verify", "read_stream"):
        r = rec[name]
        if r is None:
            lines.append("%s: amd-smi not available" % name)
            continue
        lines.append("%s: %.2f us per call, socket %.1f W, graphics clock %d MHz (per XCD %s), %.2f mJ per call"
                     % (name, r["us_per_call"], r["socket_W"], r["gfx_MHz"], r["gfx_MHz_per_xcd"], r["mJ_per_call"]))
    _write(out, lines)


def _write(out, lines):
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("out")
    s.add_argument("--command", action="append", default=[])
    s.add_argument("--window", nargs=3, metavar=("KERNEL", "FIRST", "COUNT"),
                   help="also report the mean over dispatches FIRST..FIRST+COUNT-1 of KERNEL")
    s.add_argument("--bench-log", help="bench.py output of the profiled run")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("out")
    t.add_argument("--kernel", default="split_mfma")
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--alg-bytes", type=int, default=0)
    t.add_argument("--command", action="append", default=[])
    c = sub.add_parser("counters")
    c.add_argument("out")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--kernel", default="split_mfma")
    c.add_argument("--simds", type=int, default=1024)
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--units-per-simd", type=float, default=1.0)
    c.add_argument("--unit-name", default="launch")
    c.add_argument("--command", action="append", default=[])
    pw = sub.add_parser("power")
    pw.add_argument("out")
    pw.add_argument("--workload", default="gqa8b_100k")
    pw.add_argument("--seconds", type=float, default=8.0)
    pw.add_argument("--command", action="append", default=[])
    pw.add_argument("--half-grid", action="store_true",
                    help="the split kernel alone on the workload's grid and on half of it")
    a = ap.parse_args()
    if a.cmd == "stats":
        win = (a.window[0], int(a.window[1]), int(a.window[2])) if a.window else None
        write_stats(a.dir, a.out, a.command, win, a.bench_log)
    elif a.cmd == "power":
        if a.half_grid:
            write_half_grid(a.out, a.workload, a.seconds, a.command)
        else:
            write_power(a.out, a.workload, a.seconds, a.command)
    elif a.cmd == "counters":
        write_counters(a.dirs, a.out, a.kernel, a.simds, a.xcds, a.units_per_simd, a.unit_name, a.command)
    else:
        write_traffic(a.fetch_dir, a.write_dir, a.out, a.kernel, a.copy_mib, a.alg_bytes, a.command)


if __name__ == "__main__":
    main()
