"""Turn rocprofv3 outputs into the short summaries kept under profiles/.

Three summaries:
  * kernel_summary(): per-kernel call counts and durations from a
    ``--kernel-trace --stats -f csv`` run (the ``*_kernel_stats.csv`` file);
  * traffic_summary(): HBM bytes per dispatch from two ``--pmc`` runs
    (FETCH_SIZE, then WRITE_SIZE, both in KiB per dispatch), each scaled by
    what the same counter reads for a plain device copy of known size that
    ``bench.py --pmc-run`` launches first;
  * counter_summary(): the median per dispatch of the dominant kernel for
    every counter of one or more ``--pmc`` runs (shader sequencer counters:
    wave cycles, waits, VALU and matrix-core activity), with the ratios that
    follow from them.

Usage (from the repository root, after the rocprofv3 runs):
  python -m ancestral_draft_token_amd.profiling [opts] kernels <stats.csv> <out.md> <command...>
  python -m ancestral_draft_token_amd.profiling [opts] traffic <fetch.csv> <write.csv> <workload> <mall> <out.json> <command...>
  python -m ancestral_draft_token_amd.profiling [opts] counters <out.md> <workload> <pmc.csv>[,<pmc.csv>...] <command...>
opts: --kernel <name part> (the kernel summarised; default the sampler's
markov_bias_gumbel_argmax) and --source <file under csrc/> (whose hash the
summary records; default dspark.hip).
"""

from __future__ import annotations

import csv
import hashlib
import json
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 512 << 20       # the calibration copy in bench.py --pmc-run: reads and writes this much
DOMINANT = "markov_bias_gumbel_argmax"


def source_hash(source: str = "dspark.hip") -> str:
    with open(os.path.join(PKG, "csrc", source), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def kernel_summary(stats_csv: str, out_md: str, command: str, source: str = "dspark.hip") -> None:
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# rocprofv3 kernel summary", "", f"command: `{command}`", "",
             f"source sha256[:16] of csrc/{source}: {source_hash(source)}", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("|", "/")
        if len(name) > 90:
            name = name[:87] + "..."
        lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _per_dispatch(path: str, counter: str):
    """[(dispatch id, kernel name, value)] for one counter, summed over its dimensions."""
    acc = {}
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") != counter:
            continue
        key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    return sorted((d, n, v) for (d, n), v in acc.items())


def traffic_summary(fetch_csv: str, write_csv: str, workload: str, mall: str, out_json: str,
                    command: str = "", kernel: str = DOMINANT, source: str = "dspark.hip") -> dict:
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    kib = COPY_BYTES / 1024.0
    # the calibration copies: the device-to-device copies that write COPY_BYTES
    calib = [d for d, n, v in write if "copy" in n.lower() and abs(v - kib) < 0.05 * kib][:3]
    if not calib:
        raise SystemExit("no calibration copy dispatch found")
    fmap = {d: v for d, _, v in fetch}
    wmap = {d: v for d, _, v in write}
    copy_f = statistics.median(fmap[d] for d in calib)
    copy_w = statistics.median(wmap[d] for d in calib)
    f_scale, w_scale = kib / copy_f, kib / copy_w
    dom = [d for d, n, _ in write if kernel in n]
    rec = {
        "workload": workload, "mall": mall, "kernel": kernel, "source": source, "source_sha": source_hash(source),
        "command": command,
        "copy_bytes": COPY_BYTES, "copy_dispatches": calib,
        "copy_fetch_kib": copy_f, "copy_write_kib": copy_w,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "dispatches": len(dom),
        "fetch_bytes_per_launch": statistics.median(fmap[d] for d in dom) * f_scale * 1024.0,
        "write_bytes_per_launch": statistics.median(wmap[d] for d in dom) * w_scale * 1024.0,
    }
    rec["bytes_per_launch"] = rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    others = {}
    for d, n, v in write:
        if d in calib or kernel in n or d not in fmap:
            continue
        name = n.split("(")[0][:70]
        others.setdefault(name, []).append((fmap[d] * f_scale * 1024.0, v * w_scale * 1024.0))
    rec["other_kernels"] = {n: {"fetch_bytes": statistics.median(x[0] for x in v),
                                "write_bytes": statistics.median(x[1] for x in v), "dispatches": len(v)}
                            for n, v in others.items()}
    with open(out_json, "w") as fh:
        json.dump(rec, fh, indent=1)
    return rec


RATIOS = [
    # (name, numerator, denominator, what it says)
    ("VALU active / wave cycles", "SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES",
     "share of a wave's cycles spent issuing VALU instructions"),
    ("waiting / wave cycles", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES",
     "share of a wave's cycles spent waiting (s_waitcnt, barriers, dependencies)"),
    ("waiting on s_waitcnt / wave cycles", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES",
     "share spent waiting for a memory or LDS result"),
    ("LDS bank conflicts / LDS busy", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE",
     "share of the LDS's busy cycles lost to bank conflicts"),
]
SIMDS = 256 * 4   # MI355X: 256 compute units of 4 SIMDs
XCDS = 8          # GRBM_GUI_ACTIVE comes summed over the 8 XCDs (each counts the shader clock)


def counter_summary(out_md: str, workload: str, csvs, command: str = "", kernel: str = DOMINANT,
                    source: str = "dspark.hip") -> dict:
    """Median per dispatch of every counter of the kernel, over the runs given."""
    med = {}
    disp = 0
    for path in csvs:
        names = sorted({r["Counter_Name"] for r in csv.DictReader(open(path))})
        for c in names:
            vals = [v for _, n, v in _per_dispatch(path, c) if kernel in n]
            if vals:
                med[c] = statistics.median(vals)
                disp = max(disp, len(vals))
    lines = ["# rocprofv3 counter summary", "", f"command: `{command}`", "",
             f"source sha256[:16] of csrc/{source}: {source_hash(source)}", "",
             f"workload: {workload}; kernel: {kernel}; dispatches: {disp}; "
             "values are the median per dispatch, summed over the device", "",
             "| counter | per dispatch |", "|---|---|"]
    for c, v in sorted(med.items()):
        lines.append(f"| {c} | {v:.6g} |")
    lines += ["", "| ratio | value | meaning |", "|---|---|---|"]
    ratios = {}
    for name, num, den, what in RATIOS:
        if num in med and den in med and med[den] > 0:
            ratios[name] = med[num] / med[den]
            lines.append(f"| {name} | {ratios[name]:.3f} | {what} |")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in med and med.get("GRBM_GUI_ACTIVE", 0) > 0:
        ratios["matrix cores busy"] = med["SQ_VALU_MFMA_BUSY_CYCLES"] / (med["GRBM_GUI_ACTIVE"] / XCDS * SIMDS)
        lines.append(f"| matrix cores busy | {ratios['matrix cores busy']:.3f} | SQ_VALU_MFMA_BUSY_CYCLES / "
                     f"(GRBM_GUI_ACTIVE / {XCDS} XCDs x {SIMDS} SIMDs) |")
    if "SQ_INSTS_MFMA" in med:
        lines.append(f"| matrix instructions per dispatch | {med['SQ_INSTS_MFMA']:.4g} | v_mfma issued |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return {"counters": med, "ratios": ratios}


if __name__ == "__main__":
    argv = sys.argv[1:]
    opts = {"kernel": DOMINANT, "source": "dspark.hip"}
    while argv and argv[0] in ("--kernel", "--source"):
        opts[argv[0][2:]] = argv[1]
        argv = argv[2:]
    if not argv:
        raise SystemExit(__doc__)
    if argv[0] == "kernels":
        kernel_summary(argv[1], argv[2], " ".join(argv[3:]), source=opts["source"])
    elif argv[0] == "traffic":
        print(json.dumps(traffic_summary(*argv[1:6], command=" ".join(argv[6:]), **opts), indent=1))
    elif argv[0] == "counters":
        print(json.dumps(counter_summary(argv[1], argv[2], argv[3].split(","), command=" ".join(argv[4:]), **opts),
                         indent=1))
    else:
        raise SystemExit(__doc__)
