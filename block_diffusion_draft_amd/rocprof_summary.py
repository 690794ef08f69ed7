"""Summaries of rocprofv3 CSV output (``-f csv``) for the committed profiles.

    python -m block_diffusion_draft_amd.rocprof_summary stats DIR
        per-kernel statistics (``*kernel_stats.csv``).
    python -m block_diffusion_draft_amd.rocprof_summary trace DIR [PATTERN]
        per (kernel, grid) average durations from ``*kernel_trace.csv``.
    python -m block_diffusion_draft_amd.rocprof_summary traffic --fetch DIR --write DIR
            --kernel PATTERN --copy-bytes N [--out FILE]
        HBM bytes per launch of the kernels matching PATTERN from a FETCH_SIZE run and
        a WRITE_SIZE run, each counter scaled by what it reads for a plain device copy
        of N bytes in the same run (N bytes fetched, N written): the mean over the
        --copies largest copy-kernel dispatches.
    python -m block_diffusion_draft_amd.rocprof_summary launches --fetch DIR --write DIR
            --sq DIR --trace DIR --kernel PATTERN --copy-bytes N
        per launch shape (grid) of the kernels matching PATTERN: average duration (kernel
        trace), HBM bytes per launch (FETCH_SIZE and WRITE_SIZE scaled by the copy as
        in ``traffic``) and the achieved GB/s, and from a run with SQ counters the VALU
        and MFMA instructions per wave, the VALU busy fraction SQ_ACTIVE_INST_VALU x 4 /
        (SIMDs x cycles), the MFMA busy fraction SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x
        cycles), cycles = GRBM_GUI_ACTIVE / 8 XCDs, and the launch's waves per SIMD
        (SQ_WAVES / SIMDs).
    python -m block_diffusion_draft_amd.rocprof_summary mfma DIR [PATTERN]
        per (kernel, grid) matrix-core use from a run with the counters
        SQ_VALU_MFMA_BUSY_CYCLES (MFMA busy cycles summed over the SIMDs; 32 per
        32x32x16 bf16 MFMA) and GRBM_GUI_ACTIVE (the launch's GPU cycles, summed over
        the 8 XCDs): busy / (SIMDs x cycles), SIMDs = 4 per CU.
"""
import argparse
import csv
import glob
import hashlib
import os
import re
import statistics
import sys


def _find(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits


def _rows(d, suffix):
    out = []
    for p in _find(d, suffix):
        with open(p, newline="") as f:
            out.extend(csv.DictReader(f))
    return out


def short(name, n=64):
    name = name.replace("(anonymous namespace)::", "")
    name = re.sub(r"^void ", "", name)
    name = re.sub(r"\(.*$", "", name)
    return name if len(name) <= n else name[:n - 3] + "..."


def stats(d, out=sys.stdout):
    rows = _rows(d, "kernel_stats.csv")
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out.write(f"{'kernel':64s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} "
              f"{'total_us':>10s} {'pct':>6s}\n")
    for r in rows:
        out.write(f"{short(r['Name']):64s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.1f} "
                  f"{float(r['MinNs']) / 1e3:9.1f} {float(r['MaxNs']) / 1e3:9.1f} "
                  f"{float(r['TotalDurationNs']) / 1e3:10.1f} {float(r['Percentage']):6.1f}\n")


def trace(d, pattern="", out=sys.stdout):
    rows = _rows(d, "kernel_trace.csv")
    agg = {}
    for r in rows:
        name = r["Kernel_Name"]
        if pattern and not re.search(pattern, name):
            continue
        grid = (r.get("Grid_Size_X") or r.get("Grid_Size", ""), r.get("Grid_Size_Y", ""),
                r.get("Grid_Size_Z", ""))
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        agg.setdefault((short(name, 56), grid), []).append(dur)
    out.write(f"{'kernel':56s} {'grid (threads)':>24s} {'calls':>6s} {'avg_us':>9s} {'median_us':>9s}\n")
    for (n, g), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        gs = "x".join(x for x in g if x)
        out.write(f"{n:56s} {gs:>24s} {len(v):6d} {sum(v) / len(v):9.1f} "
                  f"{statistics.median(v):9.1f}\n")


def _counter(d, name, kernel_pat):
    """{kernel dispatch -> counter value} for kernels matching kernel_pat."""
    vals = {}
    grids = {}
    for r in _rows(d, "counter_collection.csv"):
        if r["Counter_Name"] != name or not re.search(kernel_pat, r["Kernel_Name"]):
            continue
        key = r["Dispatch_Id"]
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        grids[key] = int(r.get("Grid_Size") or 0)
    return vals, grids


def mfma(d, pattern="", cus=256, xcds=8, out=sys.stdout):
    per = {}
    for r in _rows(d, "counter_collection.csv"):
        if pattern and not re.search(pattern, r["Kernel_Name"]):
            continue
        e = per.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"],
                                              "grid": int(r.get("Grid_Size") or 0)})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    agg = {}
    for e in per.values():
        if "SQ_VALU_MFMA_BUSY_CYCLES" not in e or not e.get("GRBM_GUI_ACTIVE"):
            continue
        cyc = e["GRBM_GUI_ACTIVE"] / xcds
        agg.setdefault((short(e["name"], 48), e["grid"]), []).append(
            (e["SQ_VALU_MFMA_BUSY_CYCLES"] / (4 * cus * cyc), e["SQ_VALU_MFMA_BUSY_CYCLES"], cyc))
    out.write(f"{'kernel':48s} {'grid':>10s} {'launches':>8s} {'mfma_busy':>9s} "
              f"{'mfma_cycles':>13s} {'gpu_cycles':>11s}\n")
    for (n, g), v in sorted(agg.items(), key=lambda kv: -sum(x[2] for x in kv[1])):
        k = len(v)
        out.write(f"{n:48s} {g:10d} {k:8d} {sum(x[0] for x in v) / k:9.3f} "
                  f"{sum(x[1] for x in v) / k:13.0f} {sum(x[2] for x in v) / k:11.0f}\n")


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic(fetch_dir, write_dir, kernel, copy_bytes, copies=3, copy_pat="copyBuffer"):
    res = {}
    for cname, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        k, _ = _counter(d, cname, kernel)
        c, _ = _counter(d, cname, copy_pat)
        if not k or len(c) < copies:
            raise SystemExit(f"{cname}: no dispatches of {kernel!r} or too few copy dispatches")
        cv = sorted(c.values())[-copies:]
        kib_per_copy = sum(cv) / len(cv)
        scale = copy_bytes / (kib_per_copy * 1024.0)
        kv = list(k.values())
        res[cname] = dict(kib_per_launch=sum(kv) / len(kv), launches=len(kv),
                          copy_kib=kib_per_copy, copies=len(cv), scale=scale,
                          bytes_per_launch=sum(kv) / len(kv) * 1024.0 * scale)
    res["hbm_bytes_per_launch"] = res["FETCH_SIZE"]["bytes_per_launch"] + \
        res["WRITE_SIZE"]["bytes_per_launch"]
    return res


def _per_dispatch(d, pattern):
    """{dispatch id: {"name", "grid", counter: value summed over dimensions}}."""
    per = {}
    for r in _rows(d, "counter_collection.csv"):
        if not re.search(pattern, r["Kernel_Name"]):
            continue
        e = per.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"],
                                              "grid": int(r.get("Grid_Size") or 0)})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return per


def launches(fetch_dir, write_dir, sq_dir, trace_dir, kernel, copy_bytes, copies=3,
             copy_pat="copyBuffer", cus=256, xcds=8, out=sys.stdout):
    """Per launch shape of the kernels matching `kernel`: duration, scaled HBM bytes and
    SQ counters.  The counter runs and the kernel-trace run are runs of the same command,
    so a dispatch id names the same launch in each; the trace supplies each dispatch's
    grid shape (x by y: launches of equal total size but different shape stay apart)."""
    shape = {}
    for r in _rows(trace_dir, "kernel_trace.csv"):
        shape[r["Dispatch_Id"]] = f"{r.get('Grid_Size_X') or r.get('Grid_Size')}x{r.get('Grid_Size_Y') or 1}"
    scales = {}
    for cname, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        c, _ = _counter(d, cname, copy_pat)
        cv = sorted(c.values())[-copies:]
        scales[cname] = copy_bytes / (sum(cv) / len(cv) * 1024.0)
    agg = {}
    for cname, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        for di, e in _per_dispatch(d, kernel).items():
            if cname in e:
                key = (short(e["name"], 40), shape.get(di, str(e["grid"])))
                agg.setdefault(key, {}).setdefault(cname, []).append(e[cname] * 1024.0 * scales[cname])
    for di, e in _per_dispatch(sq_dir, kernel).items():
        a = agg.setdefault((short(e["name"], 40), shape.get(di, str(e["grid"]))), {})
        for k, v in e.items():
            if k not in ("name", "grid"):
                a.setdefault(k, []).append(v)
    for r in _rows(trace_dir, "kernel_trace.csv"):
        if not re.search(kernel, r["Kernel_Name"]):
            continue
        key = (short(r["Kernel_Name"], 40), shape[r["Dispatch_Id"]])
        if key in agg:
            agg[key].setdefault("us", []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    mean = lambda v: sum(v) / len(v) if v else float("nan")
    out.write(f"{'kernel':40s} {'grid':>10s} {'us':>7s} {'hbm_MB':>8s} {'GB/s':>7s} "
              f"{'valu/wave':>9s} {'mfma/wave':>9s} {'valu_busy':>9s} {'mfma_busy':>9s} "
              f"{'waves/simd':>10s}\n")
    for (n, g), a in sorted(agg.items(), key=lambda kv: -mean(kv[1].get("us", [0]))):
        us = mean(a.get("us", []))
        hbm = mean(a.get("FETCH_SIZE", [])) + mean(a.get("WRITE_SIZE", []))
        cyc = mean(a.get("GRBM_GUI_ACTIVE", [])) / xcds
        waves = mean(a.get("SQ_WAVES", []))
        simds = 4 * cus
        out.write(f"{n:40s} {g:>10s} {us:7.1f} {hbm / 1e6:8.2f} {hbm / us / 1e3:7.0f} "
                  f"{mean(a.get('SQ_INSTS_VALU', [])) / waves:9.0f} "
                  f"{mean(a.get('SQ_INSTS_MFMA', [])) / waves:9.0f} "
                  f"{mean(a.get('SQ_ACTIVE_INST_VALU', [])) * 4 / (simds * cyc):9.3f} "
                  f"{mean(a.get('SQ_VALU_MFMA_BUSY_CYCLES', [])) / (simds * cyc):9.3f} "
                  f"{waves / simds:10.2f}\n")


def hbm(fetch_dir, write_dir, trace_dir, kernel="", copy_bytes=1 << 31, copies=3,
        copy_pat="copyBuffer", out=sys.stdout):
    """Every kernel of a step, per launch shape: launches, mean duration (trace run) and
    FETCH_SIZE / WRITE_SIZE per launch in MB (each scaled by what it reads for the plain
    device copy of copy_bytes in the same run), and their sum over the duration.  The
    three runs are runs of the same command; dispatch ids join them."""
    shape, dur = {}, {}
    for r in _rows(trace_dir, "kernel_trace.csv"):
        sh = f"{r.get('Grid_Size_X') or r.get('Grid_Size')}x{r.get('Grid_Size_Y') or 1}x{r.get('Grid_Size_Z') or 1}"
        shape[r["Dispatch_Id"]] = sh
        if re.search(kernel, r["Kernel_Name"]):
            dur.setdefault((short(r["Kernel_Name"], 40), sh), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    agg = {}
    for cname, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        c, _ = _counter(d, cname, copy_pat)
        cv = sorted(c.values())[-copies:]
        scale = copy_bytes / (sum(cv) / len(cv) * 1024.0)
        names = {}
        per = {}
        for r in _rows(d, "counter_collection.csv"):
            if r["Counter_Name"] != cname or not re.search(kernel, r["Kernel_Name"]):
                continue
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = r["Kernel_Name"]
        for di, v in per.items():
            key = (short(names[di], 40), shape.get(di, "?"))
            agg.setdefault(key, {}).setdefault(cname, []).append(v * 1024.0 * scale)
    mean = lambda v: sum(v) / len(v) if v else 0.0
    out.write(f"{'kernel':40s} {'grid':>20s} {'launches':>8s} {'us':>8s} {'fetch_MB':>9s} "
              f"{'write_MB':>9s} {'GB/s':>7s}\n")
    keys = sorted(set(dur) | set(agg), key=lambda k: -mean(dur.get(k, [])) * len(dur.get(k, [])))
    for k in keys:
        a = agg.get(k, {})
        us = mean(dur.get(k, []))
        f, w = mean(a.get("FETCH_SIZE", [])), mean(a.get("WRITE_SIZE", []))
        out.write(f"{k[0]:40s} {k[1]:>20s} {len(dur.get(k, [])):8d} {us:8.1f} {f / 1e6:9.2f} "
                  f"{w / 1e6:9.2f} {(f + w) / us / 1e3 if us else 0.0:7.0f}\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats"); a.add_argument("dir")
    a = sub.add_parser("trace"); a.add_argument("dir"); a.add_argument("pattern", nargs="?", default="")
    a = sub.add_parser("mfma"); a.add_argument("dir"); a.add_argument("pattern", nargs="?", default="")
    a = sub.add_parser("launches")
    for o in ("--fetch", "--write", "--sq", "--trace", "--kernel"):
        a.add_argument(o, required=True)
    a.add_argument("--copy-bytes", type=int, required=True)
    a = sub.add_parser("hbm")
    for o in ("--fetch", "--write", "--trace"):
        a.add_argument(o, required=True)
    a.add_argument("--kernel", default="")
    a.add_argument("--copy-bytes", type=int, required=True)
    a = sub.add_parser("traffic")
    a.add_argument("--fetch", required=True); a.add_argument("--write", required=True)
    a.add_argument("--kernel", required=True); a.add_argument("--copy-bytes", type=int, required=True)
    a.add_argument("--copies", type=int, default=3)
    a.add_argument("--source", nargs="*", default=[], help="kernel sources to fingerprint")
    a.add_argument("--out")
    args = ap.parse_args()
    if args.cmd == "stats":
        stats(args.dir)
    elif args.cmd == "trace":
        trace(args.dir, args.pattern)
    elif args.cmd == "mfma":
        mfma(args.dir, args.pattern)
    elif args.cmd == "launches":
        launches(args.fetch, args.write, args.sq, args.trace, args.kernel, args.copy_bytes)
    elif args.cmd == "hbm":
        hbm(args.fetch, args.write, args.trace, args.kernel, args.copy_bytes)
    else:
        r = traffic(args.fetch, args.write, args.kernel, args.copy_bytes, args.copies)
        lines = [f"kernel_pattern {args.kernel}",
                 f"hbm_bytes_per_launch {r['hbm_bytes_per_launch']:.0f}"]
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            x = r[c]
            lines.append(f"{c.lower()}_kib_per_launch {x['kib_per_launch']:.1f} launches {x['launches']}")
            lines.append(f"{c.lower()}_copy_kib {x['copy_kib']:.1f} copies {x['copies']} "
                         f"copy_bytes {args.copy_bytes} scale {x['scale']:.4f}")
        if args.source:
            lines.append(f"kernel_source_sha256_16 {source_hash(args.source)}")
        text = "\n".join(lines) + "\n"
        if args.out:
            with open(args.out, "w") as f:
                f.write(text)
        sys.stdout.write(text)


if __name__ == "__main__":
    main()
