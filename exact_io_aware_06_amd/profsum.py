"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

    python -m exact_io_aware_06_amd.profsum stats  <kernel_stats.csv> <out.txt> <command...>
    python -m exact_io_aware_06_amd.profsum counters [--kernel SUBSTR] [--last N] <workload> <out.txt> <pmc_dir>... -- <command...>
    python -m exact_io_aware_06_amd.profsum traffic [--kernel SUBSTR] <workload> <fetch_dir> <write_dir> \
        <copy_fetch_dir> <copy_write_dir> <copy_mib> <kernel_src[,src...]> <out.txt> <command...>

`stats` copies the per-kernel duration table and, from the kernel trace
beside it, adds the busiest kernel's mean over its last 150 dispatches
(bench.py's timed calls, after the clock-settling ones). `counters` averages the SQ/GRBM
counters of one kernel (the kernels whose name contains SUBSTR, default
"fwd_bf16") over its dispatches and derives MFMA busy
fraction (per SIMD, from SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs and the
per-XCD GRBM_GUI_ACTIVE), instruction mix per 256x64 wave tile and the LDS bank
conflict rate. `traffic` turns FETCH_SIZE and
WRITE_SIZE (KiB per dispatch, from two separate --pmc runs) into HBM bytes per
launch, each scaled by what the same counter reads for a device-to-device copy
of known size (bench.py --copy-calibration), and records the sha256 of the
kernel source so that bench.py reports the figure only while the kernel is
unchanged.
"""

import csv
import hashlib
import os
import re
import sys


def _counter(d, name, kernel_substr):
    path = os.path.join(d, "pmc_counter_collection.csv")
    per = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != name or kernel_substr not in r["Kernel_Name"]:
            continue
        key = int(r["Dispatch_Id"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {name} rows for {kernel_substr!r} in {path}")
    vals = [per[k] for k in sorted(per)]
    return sum(vals) / len(vals), len(vals)


def stats(src, out, cmd, last=150):
    rows = list(csv.DictReader(open(src)))
    with open(out, "w") as f:
        f.write(f"# rocprofv3 --kernel-trace --stats summary\n# command: {cmd}\n")
        f.write("kernel | calls | avg_us | min_us | max_us | pct\n")
        for r in rows:
            f.write(f"{r['Name']} | {r['Calls']} | {float(r['AverageNs'])/1e3:.1f} | "
                    f"{float(r['MinNs'])/1e3:.1f} | {float(r['MaxNs'])/1e3:.1f} | "
                    f"{float(r['Percentage']):.2f}\n")
        # the kernel trace beside the stats: the busiest kernel over its last
        # `last` dispatches (bench.py's 100 timed and 50 single-timed calls,
        # after the clock-settling and warm-up calls, whose clocks still ramp)
        trace = os.path.join(os.path.dirname(src), os.path.basename(src).replace(
            "kernel_stats.csv", "kernel_trace.csv"))
        if rows and os.path.exists(trace):
            name = rows[0]["Name"]
            d = [(int(t["End_Timestamp"]) - int(t["Start_Timestamp"])) / 1e3
                 for t in csv.DictReader(open(trace)) if t["Kernel_Name"] == name]
            if len(d) > last:
                tail = sorted(d[-last:])
                f.write(f"# {name}: mean of the last {last} dispatches {sum(tail) / last:.1f} us, "
                        f"median {tail[last // 2]:.1f} us ({len(d) - last} earlier dispatches "
                        f"excluded; all {len(d)}: mean {sum(d) / len(d):.1f} us)\n")


def _durations_ns(d, kernel):
    """Per-dispatch kernel durations (ns) from the kernel trace written next
    to the counters (rocprofv3 --pmc ... --kernel-trace), keyed by dispatch."""
    path = next((os.path.join(d, n) for n in ("kernel_trace.csv", "pmc_kernel_trace.csv")
                 if os.path.exists(os.path.join(d, n))), None)
    if path is None:
        return {}
    out = {}
    for r in csv.DictReader(open(path)):
        if kernel in r["Kernel_Name"]:
            out[int(r["Dispatch_Id"])] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return out


def counters(workload, out, dirs, cmd, kernel="fwd_bf16", last=0):
    """Mean of each counter over the dispatches of `kernel` (the last `last`
    of them when last > 0: the calls after the clocks have settled)."""
    acc = {}
    durs = []
    full_name = ""
    for d in dirs:
        path = os.path.join(d, "pmc_counter_collection.csv")
        per = {}
        for r in csv.DictReader(open(path)):
            if kernel not in r["Kernel_Name"]:
                continue
            full_name = r["Kernel_Name"]
            key = (r["Counter_Name"], int(r["Dispatch_Id"]))
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        disp = sorted({k[1] for k in per})
        if last > 0:
            disp = disp[-last:]
        keep = set(disp)
        names = {}
        for (n, di), v in per.items():
            if di in keep:
                names.setdefault(n, []).append(v)
        for n, vs in names.items():
            acc.setdefault(n, []).append(sum(vs) / len(vs))
        dd = _durations_ns(d, kernel)
        durs += [dd[x] for x in disp if x in dd]
    c = {n: sum(v) / len(v) for n, v in acc.items()}
    if not acc:
        raise SystemExit(f"no counter rows for kernels matching {kernel!r}")
    which = f"the last {last} dispatches of each run" if last > 0 else "every dispatch"
    lines = [f"# rocprofv3 --pmc counters of the kernels matching {kernel!r}, workload {workload}",
             f"# averaged over {which}",
             f"# command (one run per counter group): {cmd}",
             "counter | mean per dispatch"]
    lines += [f"{n} | {c[n]:.1f}" for n in sorted(c)]
    if durs:
        dur = sum(durs) / len(durs)
        lines.append(f"kernel_duration_us_under_pmc | {dur / 1e3:.1f}")
        if "GRBM_GUI_ACTIVE" in c:
            lines.append(f"gui_active_cycles_per_xcd_over_duration_GHz | {c['GRBM_GUI_ACTIVE'] / 8.0 / dur:.3f}")
    lines.append("# derived")
    gui = c.get("GRBM_GUI_ACTIVE", 0.0) / 8.0   # GUI-active cycles of one XCD
    if gui > 0:
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            lines.append(f"mfma_busy_fraction_per_simd | {c['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024 / gui:.3f}")
        for n in ("SQ_LDS_DATA_FIFO_FULL", "SQ_LDS_CMD_FIFO_FULL", "SQ_LDS_IDX_ACTIVE",
                  "SQ_LDS_BANK_CONFLICT"):
            if n in c:
                lines.append(f"{n.lower()}_per_cu_over_gui | {c[n] / 256 / gui:.3f}")
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in c and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
        lines.append(f"mfma_coexec_over_busy | {c['SQ_VALU_MFMA_COEXEC_CYCLES'] / c['SQ_VALU_MFMA_BUSY_CYCLES']:.3f}")
    if "SQ_LDS_BANK_CONFLICT" in c and "SQ_LDS_IDX_ACTIVE" in c:
        lines.append(f"lds_bank_conflict_over_idx_active | {c['SQ_LDS_BANK_CONFLICT'] / max(c['SQ_LDS_IDX_ACTIVE'], 1):.4f}")
    mf = c.get("SQ_INSTS_MFMA", 0.0)
    if mf > 0 and kernel.startswith("fwd_"):
        # MFMAs per wave per 64-key tile: 32 at head dimension 128, 16 at 64
        dm = re.search(r"kernel<(\d+)[,>]", full_name)
        per_tile = {128: 32, 64: 16}.get(int(dm.group(1))) if dm else None
        if per_tile:
            wt = mf / per_tile   # MFMA instructions per wave per 64-key tile
            if "SQ_INSTS_VALU" in c:
                lines.append(f"valu_non_mfma_per_wave_tile | {(c['SQ_INSTS_VALU'] - mf) / wt:.1f}")
            if "SQ_INSTS_LDS" in c:
                lines.append(f"lds_insts_per_wave_tile | {c['SQ_INSTS_LDS'] / wt:.1f}")
            if "SQ_INSTS_VALU_TRANS_F32" in c:
                lines.append(f"transcendental_per_wave_tile | {c['SQ_INSTS_VALU_TRANS_F32'] / wt:.1f}")
    open(out, "w").write("\n".join(lines) + "\n")


def source_sha256(paths):
    """sha256 over the concatenated bytes of the kernel's source files."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic(workload, fdir, wdir, cfdir, cwdir, copy_mib, src, out, cmd, kernel="fwd_"):
    # the forward kernel only (a split launch also runs the merge kernel)
    fetch, nf = _counter(fdir, "FETCH_SIZE", kernel)
    write, nw = _counter(wdir, "WRITE_SIZE", kernel)
    cfetch, _ = _counter(cfdir, "FETCH_SIZE", "copyBuffer")
    cwrite, _ = _counter(cwdir, "WRITE_SIZE", "copyBuffer")
    copy_kib = float(copy_mib) * 1024.0
    kf, kw = copy_kib / cfetch, copy_kib / cwrite
    hbm = fetch * kf * 1024 + write * kw * 1024
    sha = source_sha256(src.split(","))
    with open(out, "w") as f:
        f.write(f"# HBM traffic of the attention forward kernel, workload {workload}\n")
        f.write(f"# command: {cmd}\n")
        f.write(f"# counters: FETCH_SIZE and WRITE_SIZE in separate rocprofv3 --pmc runs "
                f"({nf} and {nw} dispatches averaged)\n")
        f.write(f"# calibration: a {copy_mib} MiB device-to-device copy reads FETCH_SIZE "
                f"{cfetch:.0f} KiB and WRITE_SIZE {cwrite:.0f} KiB\n")
        f.write(f"fetch_kib_per_dispatch: {fetch:.1f}\n")
        f.write(f"write_kib_per_dispatch: {write:.1f}\n")
        f.write(f"fetch_scale: {kf:.4f}\n")
        f.write(f"write_scale: {kw:.4f}\n")
        f.write(f"hbm_bytes_per_launch: {hbm:.0f}\n")
        f.write(f"kernel_source: {','.join(os.path.relpath(x) for x in src.split(','))}\n")
        f.write(f"source_sha256: {sha}\n")


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "stats":
        stats(sys.argv[2], sys.argv[3], " ".join(sys.argv[4:]))
    elif mode == "counters":
        args = sys.argv[2:]
        kernel = "fwd_bf16"
        last = 0
        while args[0] in ("--kernel", "--last"):
            if args[0] == "--kernel":
                kernel = args[1]
            else:
                last = int(args[1])
            args = args[2:]
        cut = args.index("--")
        counters(args[0], args[1], args[2:cut], " ".join(args[cut + 1:]), kernel, last)
    elif mode == "traffic":
        args = sys.argv[2:]
        kernel = "fwd_"
        if args[0] == "--kernel":
            kernel, args = args[1], args[2:]
        traffic(*args[:8], " ".join(args[8:]), kernel=kernel)
    else:
        raise SystemExit(__doc__)
