"""Per-call hardware counter figures from rocprofv3 --pmc passes (a profiling
aid, not part of the compute path).

A workload is profiled by running ``bench.py --only <workload>`` under
several ``rocprofv3 --pmc`` passes (the hardware collects a limited set of
counters per pass), plus the same FETCH_SIZE / WRITE_SIZE passes over
``bench.py --only copy_calibration``, a device-to-device copy of known size.
This module reads the counter-collection CSVs of those passes and writes

  * ``profiles/<workload>_counters.json``: per-call HBM bytes read and
    written (FETCH_SIZE / WRITE_SIZE in KiB, scaled by what the same counters
    read for the copy), VALU and transcendental instruction counts, tagged
    with a hash of the kernel sources the workload runs, so that bench.py
    ignores figures taken on other code;
  * ``profiles/<workload>_counters.txt``: the same per kernel, readable.

"Per call" is one call of the library entry point the workload times: the
library's kernels (namespace ``ssm::``) summed, each counter averaged over
the dispatches of its own pass (passes are separate runs and may make
different numbers of calls) times the kernel's launches per call (its
dispatch count over that of the least-launched kernel in one pass).

It also turns a ``rocprofv3 --kernel-trace`` run into
``profiles/<workload>_kernel_stats.txt`` (per-kernel launch durations of the
library's kernels).

usage:
  python -m selective_state_space_31_amd.counters pmc WORKLOAD --passes DIR [DIR...]
         --calib DIR [DIR...] [--out profiles] [--command TEXT]
  python -m selective_state_space_31_amd.counters trace WORKLOAD --dir DIR
         [--out profiles] [--command TEXT]
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# Sources each workload family's kernels are built from (host launch code
# included: it picks the launch shapes).
_FWD = ["kernels.hpp", "ssm_scan.hip", "host_util.hpp"]
SOURCES = {
    "fwd": _FWD,
    "bwd": _FWD + ["bwd.hip"],
    "ssd": ["ssd.hip", "host_util.hpp"],
    "conv": ["conv1d.hip", "host_util.hpp"],
    "decode": ["ssm_scan.hip", "host_util.hpp"],
}


def family(workload):
    if workload.endswith("_bwd"):
        return "bwd"
    if workload.startswith("ssd_"):
        return "ssd"
    if workload.startswith("conv1d_"):
        return "conv"
    if workload.startswith("decode_"):
        return "decode"
    return "fwd"


def source_hash(workload):
    """First 16 hex digits of the SHA-256 of the workload family's sources
    (the forward also hashes its per-type instantiation files)."""
    fam = family(workload)
    names = list(SOURCES[fam])
    if fam in ("fwd", "bwd"):
        names += sorted(n for n in os.listdir(CSRC) if n.startswith("fwd_") and n.endswith(".hip"))
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(n.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _waves(r):
    """Waves a dispatch launched (Grid_Size and Workgroup_Size count work-items),
    or None when the CSV does not give the sizes."""
    try:
        grid, wg = int(r["Grid_Size"]), int(r["Workgroup_Size"])
    except (KeyError, ValueError):
        return None
    if wg <= 0:
        return None
    return (grid // wg) * ((wg + 63) // 64)


def _rows(dirs):
    """(file, dispatch id, kernel name, counter, value, launched waves) of
    every counter-collection CSV under the given rocprofv3 output directories."""
    out = []
    for d in dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit("no counter_collection.csv under %s" % d)
        for fn in files:
            with open(fn, newline="") as f:
                for r in csv.DictReader(f):
                    out.append((fn, int(r["Dispatch_Id"]), r["Kernel_Name"], r["Counter_Name"],
                                float(r["Counter_Value"]), _waves(r)))
    return out


def _short(name):
    s = name.replace("ssm::", "").replace("(anonymous namespace)::", "")
    return s.split("(")[0] if "(" in s else s


def per_kernel(dirs):
    """Per-dispatch means over the library's kernels:
    {kernel: {counter: mean value per dispatch}} and, per kernel, its launches
    per call and the waves one of its dispatches launches.  Each counter is
    averaged over the dispatches of its own pass (passes are separate runs
    and need not make the same number of calls)."""
    vals, waves, per_file = {}, {}, {}
    for fn, did, kname, cname, val, wv in _rows(dirs):
        if "ssm::" not in kname:
            continue
        k = _short(kname)
        vals.setdefault(k, {}).setdefault(cname, {})[(fn, did)] = val
        if wv is not None:
            waves.setdefault(k, {})[(fn, did)] = wv
        per_file.setdefault(fn, {}).setdefault(k, set()).add(did)
    mean = {k: {c: sum(v.values()) / len(v) for c, v in cs.items()} for k, cs in vals.items()}
    # launches per call from a pass that saw every kernel: dispatches of the
    # kernel over those of the least-launched one
    lpc = {k: 1.0 for k in mean}
    for fn in sorted(per_file):
        cnt = per_file[fn]
        if set(cnt) == set(mean):
            lo = min(len(v) for v in cnt.values())
            lpc = {k: len(v) / lo for k, v in cnt.items()}
            break
    wmean = {k: sum(w.values()) / len(w) for k, w in waves.items() if w}
    npass = {fn: min(len(v) for v in cnt.values()) for fn, cnt in per_file.items()}
    return mean, lpc, wmean, npass


def calibration(dirs):
    """Bytes per KiB-unit of FETCH_SIZE and WRITE_SIZE: a 1 GiB copy's
    counters (median over its dispatches) against the bytes it moves."""
    copy_bytes = float(1 << 30)
    fetch, write = [], []
    for _, _, kname, cname, val, _ in _rows(dirs):
        if "copy" not in kname.lower() or val <= 0:
            continue
        if cname == "FETCH_SIZE":
            fetch.append(val)
        elif cname == "WRITE_SIZE":
            write.append(val)
    if not fetch or not write:
        raise SystemExit("calibration passes hold no copy kernel FETCH_SIZE / WRITE_SIZE")
    fk, wk = statistics.median(fetch), statistics.median(write)
    return dict(fetch_kib=fk, write_kib=wk, fetch_scale=copy_bytes / (fk * 1024.0),
                write_scale=copy_bytes / (wk * 1024.0))


def summarize(workload, pass_dirs, calib_dirs, command=""):
    mean, lpc, wmean, npass = per_kernel(pass_dirs)
    if not mean:
        raise SystemExit("no library kernels in the counter passes")
    cal = calibration(calib_dirs)
    kernels = {}
    tot = {}
    valu = trans = 0.0
    for k in sorted(mean):
        pc = {c: v * lpc[k] for c, v in mean[k].items()}
        pc["launches_per_call"] = lpc[k]
        # A check that the SQ counters saw every launched wave (they do on
        # this part: coverage 1); instruction counts are scaled by it.
        cov = 1.0
        if k in wmean and mean[k].get("SQ_WAVES"):
            pc["waves_launched"] = wmean[k] * lpc[k]
            cov = mean[k]["SQ_WAVES"] / wmean[k]
            pc["sq_wave_coverage"] = cov
        kernels[k] = pc
        for c, v in pc.items():
            if c not in ("launches_per_call", "waves_launched", "sq_wave_coverage"):
                tot[c] = tot.get(c, 0.0) + v
        if "SQ_INSTS_VALU" in pc and cov > 0:
            valu += pc["SQ_INSTS_VALU"] / cov
        if "SQ_INSTS_VALU_TRANS_F32" in pc and cov > 0:
            trans += pc["SQ_INSTS_VALU_TRANS_F32"] / cov
    res = dict(workload=workload, kernel_source_sha256_16=source_hash(workload),
               calls_profiled=sorted(npass.values()), calibration=cal, command=command,
               kernels=kernels, per_call=tot)
    if "FETCH_SIZE" in tot:
        res["hbm_read_bytes_per_call"] = tot["FETCH_SIZE"] * 1024.0 * cal["fetch_scale"]
    if "WRITE_SIZE" in tot:
        res["hbm_write_bytes_per_call"] = tot["WRITE_SIZE"] * 1024.0 * cal["write_scale"]
    if "FETCH_SIZE" in tot and "WRITE_SIZE" in tot:
        res["hbm_bytes_per_call"] = res["hbm_read_bytes_per_call"] + res["hbm_write_bytes_per_call"]
    if "SQ_INSTS_VALU" in tot:
        res["valu_insts_per_call"] = valu  # scaled to every launched wave
    if "SQ_INSTS_VALU_TRANS_F32" in tot:
        res["valu_trans_insts_per_call"] = trans
    return res


def text(res):
    lines = ["# rocprofv3 --pmc counters per call, workload %s" % res["workload"],
             "# command (one pass per counter set): %s" % res["command"],
             "# calibration: 1 GiB copy reads FETCH_SIZE %.0f KiB, WRITE_SIZE %.0f KiB"
             " -> bytes = FETCH_SIZE x 1024 x %.3f, WRITE_SIZE x 1024 x %.3f"
             % (res["calibration"]["fetch_kib"], res["calibration"]["write_kib"],
                res["calibration"]["fetch_scale"], res["calibration"]["write_scale"]),
             "# kernel sources hash %s; calls profiled per pass: %s" % (
                 res["kernel_source_sha256_16"], res["calls_profiled"]), ""]
    for k, pc in res["kernels"].items():
        lines.append("== %s  (%.0f launch(es) per call)" % (k, pc["launches_per_call"]))
        for c in sorted(pc):
            if c not in ("launches_per_call", "waves_launched", "sq_wave_coverage"):
                lines.append("   %-26s %14.6g" % (c, pc[c]))
        if "sq_wave_coverage" in pc:
            lines.append("   -> waves launched %.0f; the SQ counters cover %.1f%% of them"
                         % (pc["waves_launched"], 100.0 * pc["sq_wave_coverage"]))
        w = pc.get("SQ_WAVES")
        if w and "SQ_INSTS_VALU" in pc:
            tr = pc.get("SQ_INSTS_VALU_TRANS_F32")
            lines.append("   -> VALU instructions per wave %.0f%s" % (
                pc["SQ_INSTS_VALU"] / w,
                "" if tr is None else "; transcendental share %.1f%%" % (100.0 * tr / pc["SQ_INSTS_VALU"])))
        lines.append("")
    lines.append("== per call (all kernels)")
    for key in ("hbm_read_bytes_per_call", "hbm_write_bytes_per_call", "hbm_bytes_per_call",
                "valu_insts_per_call", "valu_trans_insts_per_call"):
        # (the VALU figures scaled to every launched wave)
        if key in res:
            lines.append("   %-26s %14.6g" % (key, res[key]))
    return "\n".join(lines) + "\n"


def trace_text(workload, d, command=""):
    """Per-kernel launch durations of the library's kernels from a
    rocprofv3 --kernel-trace run."""
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit("no kernel_trace.csv under %s" % d)
    dur = {}
    for fn in files:
        with open(fn, newline="") as f:
            for r in csv.DictReader(f):
                if "ssm::" not in r["Kernel_Name"]:
                    continue
                k = _short(r["Kernel_Name"])
                dur.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if not dur:
        raise SystemExit("no library kernels in the trace")
    calls = min(len(v) for v in dur.values())
    total = sum(sum(v) for v in dur.values())
    lines = ["# rocprofv3 kernel trace, workload %s (library kernels only)" % workload,
             "# command: %s" % command,
             "# kernel sources hash %s; durations in microseconds" % source_hash(workload),
             "%-64s %6s %10s %10s %10s %10s %7s" % ("kernel", "calls", "avg_us", "median_us", "min_us",
                                                  "max_us", "share")]
    per_call = 0.0
    for k, v in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
        per_call += sum(v) / calls
        lines.append("%-64s %6d %10.2f %10.2f %10.2f %10.2f %6.1f%%" % (
            k[:64], len(v), statistics.mean(v), statistics.median(v), min(v), max(v),
            100.0 * sum(v) / total))
    lines.append("# kernel time per call (each kernel's total over %d calls): %.2f us" % (calls, per_call))
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("mode", choices=["pmc", "trace"])
    ap.add_argument("workload")
    ap.add_argument("--passes", nargs="+")
    ap.add_argument("--calib", nargs="+")
    ap.add_argument("--dir")
    ap.add_argument("--out", default=os.path.join(os.path.dirname(HERE), "profiles"))
    ap.add_argument("--command", default="")
    a = ap.parse_args(argv)
    os.makedirs(a.out, exist_ok=True)
    if a.mode == "trace":
        t = trace_text(a.workload, a.dir, a.command)
        with open(os.path.join(a.out, a.workload + "_kernel_stats.txt"), "w") as f:
            f.write(t)
        print(t)
        return 0
    if not a.passes or not a.calib:
        ap.error("pmc needs --passes and --calib")
    res = summarize(a.workload, a.passes, a.calib, a.command)
    with open(os.path.join(a.out, a.workload + "_counters.json"), "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
    with open(os.path.join(a.out, a.workload + "_counters.txt"), "w") as f:
        f.write(text(res))
    print(text(res))


if __name__ == "__main__":
    sys.exit(main())
