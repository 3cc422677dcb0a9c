"""Summarise rocprofv3 output of ``bench.py`` into the kernel-duration and HBM-traffic records.

Inputs are the CSV files of three runs of the same bench command:

* ``--trace``: ``rocprofv3 --kernel-trace --stats --output-format csv`` (``*_kernel_stats.csv``);
* ``--fetch`` / ``--write``: ``rocprofv3 --pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` with
  ``--kernel-trace`` (``*_counter_collection.csv``), run with ``bench.py --calibrate-copy`` so
  that a 64 MiB device copy (the runtime's copyBuffer kernel) gives the counters' scale.

Writes a markdown table (average duration and HBM bytes per read, per T and weight format) and
the JSON traffic record that ``bench.py`` reads, keyed to the library's source hash.

    python -m bf16_hyper_connection_amd.rocprof_summary --trace DIR --fetch DIR --write DIR \\
        --md profiles/x.md --json profiles/x.json --command "..." --command "..."
"""

import argparse
import collections
import csv
import glob
import json
import os
import re
import statistics

from bf16_hyper_connection_amd import build

S, D, R = 4, 2560, 320
FORMATS = {0: "bf16", 1: "q8_0"}
COPY_BYTES = 64 << 20


def algorithmic_bytes(fmt, T):
    w = 2 * R * S * D * 2 if fmt == 0 else 2 * (R * S * D + R * S * D // 32 * 2)
    return w + S * D * 4 + T * (S * D * 4 + S * D * 4 + D * 4)


def kernel_key(name):
    """('down'|'up', T, fmt, inj, pend) of a read kernel's demangled name, ('quantize',) or None."""
    m = re.search(r"hcr::hc_down<(\d+), (\d+)>", name)
    if m:
        return ("down", int(m.group(1)), int(m.group(2)), False, False)
    m = re.search(r"hcr::hc_up<(\d+), (true|false), (true|false), (\d+)>", name)
    if m:
        return ("up", int(m.group(1)), int(m.group(4)), m.group(2) == "true", m.group(3) == "true")
    m = re.search(r"hcr::hc_up_mfma<(\d+), (true|false), (true|false), (\d+)>", name)  # matrix cores
    if m:
        return ("up", int(m.group(1)), int(m.group(4)), m.group(2) == "true", m.group(3) == "true")
    if "hcr::q8_quantize" in name:
        return ("quantize",)
    m = re.search(r"hcr::mv_bf16<(\d+), (\d+)>", name)
    if m:
        return ("matvec", int(m.group(1)), int(m.group(2)))
    # the calibration library (include/hcr_calib.h)
    if "cal_empty" in name:
        return ("cal_empty",)
    m = re.search(r"cal_down_loads<(\d+), (true|false)>", name)  # (T, one store per work-group)
    if m:
        return ("cal_down_loads", int(m.group(1))) if m.group(2) == "false" else ("cal_down_loads_store", int(m.group(1)))
    m = re.search(r"cal_up_mfma_loads<(\d+)>", name)
    if m:
        return ("cal_up_loads", int(m.group(1)))
    m = re.search(r"cal_up_(valu|mfma)<(\d+)>", name)
    if m:
        return ("cal_up_" + m.group(1), int(m.group(2)))
    m = re.search(r"cal_slab_read_down<(\d+), (true|false)>", name)
    if m:
        return ("cal_slab_read_down", int(m.group(1)), m.group(2) == "true")
    m = re.search(r"cal_slab_read_up<(\d+), (true|false)>", name)
    if m:
        return ("cal_slab_read_up", int(m.group(1)), m.group(2) == "true")
    m = re.search(r"cal_slab_down<(\d+), (\d+)>", name)
    if m:
        return ("cal_slab_down", int(m.group(1)), int(m.group(2)))
    m = re.search(r"cal_slab_up<(\d+)>", name)
    if m:
        return ("cal_slab_up", int(m.group(1)))
    return None


MV_ROWS, MV_COLS = 12288, 2560


def matvec_bytes(T):
    return MV_ROWS * MV_COLS * 2 + T * MV_COLS * 4 + T * MV_ROWS * 4


def _one(pattern, d):
    files = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one {pattern} under {d}, found {files}")
    return files[0]


def durations(trace_dir):
    out = {}
    with open(_one("*kernel_stats.csv", trace_dir)) as fh:
        for r in csv.DictReader(fh):
            k = kernel_key(r["Name"])
            if k:
                out[k] = (float(r["AverageNs"]) / 1000.0, int(r["Calls"]))
    return out


def timed_region(trace_dir):
    """The read dispatches between the last two marker kernels (bench.py runs a torch neg_ kernel just
    before and just after its timed region): (reads, mean µs per read from first start to last end,
    mean down µs, mean up µs)."""
    with open(_one("*kernel_trace.csv", trace_dir)) as fh:
        rows = sorted(csv.DictReader(fh), key=lambda r: int(r["Dispatch_Id"]))
    marks = [i for i, r in enumerate(rows) if "neg_kernel" in r["Kernel_Name"]]
    if len(marks) < 2:
        return None
    region = [r for r in rows[marks[-2] + 1:marks[-1]] if kernel_key(r["Kernel_Name"])]
    if not region:
        return None
    dur = collections.defaultdict(list)
    for r in region:
        dur[kernel_key(r["Kernel_Name"])[0]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    reads = len(dur["down"])
    span = (max(int(r["End_Timestamp"]) for r in region) - min(int(r["Start_Timestamp"]) for r in region)) / 1000.0
    per_read = sorted(d + u for d, u in zip(dur["down"], dur["up"]))
    pct = {p: per_read[min(len(per_read) - 1, int(p / 100.0 * len(per_read)))] for p in (10, 50, 90)}
    # per T: each down dispatch with the up dispatch that follows it (the read's two kernels, in order)
    per_T = collections.defaultdict(list)
    pending_down = None
    for r in region:
        k = kernel_key(r["Kernel_Name"])
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        if k[0] == "down":
            pending_down = (k[1], d)
        elif k[0] == "up" and pending_down and pending_down[0] == k[1]:
            per_T[k[1]].append(pending_down[1] + d)
            pending_down = None
    return reads, span / reads, statistics.mean(dur["down"]), statistics.mean(dur["up"]), pct, per_T


def percentiles(v):
    v = sorted(v)
    return [v[min(len(v) - 1, int(p / 100.0 * len(v)))] for p in (10, 50, 90)]


def counters(d, counter):
    vals, copy = collections.defaultdict(list), []
    with open(_one("*counter_collection.csv", d)) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            k = kernel_key(r["Kernel_Name"])
            if k:
                vals[k].append(v)
            elif "copyBuffer" in r["Kernel_Name"] and v > 8192:
                copy.append(v)
    if not copy:
        raise SystemExit(f"no calibration copy in {d}: run bench.py with --calibrate-copy")
    return {k: statistics.median(v) for k, v in vals.items()}, statistics.median(copy)


SQ_COUNTERS = ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
               "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_VMEM"]


def sq_table(d, commands):
    """Markdown: per read kernel (BF16, no pending write or injection) and T, the median per dispatch of one
    rocprofv3 --pmc pass over SQ_COUNTERS, and those counts per wave."""
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    with open(_one("*counter_collection.csv", d)) as fh:
        for r in csv.DictReader(fh):
            k = kernel_key(r["Kernel_Name"])
            if k and k[0] in ("down", "up") and k[2] == 0 and not k[3] and not k[4]:
                vals[(k[0], k[1])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    from bf16_hyper_connection_amd.build import source_hash
    md = ["# SQ counters of the read kernels (MI355X)", "", "Commands (run from the repository root, on one MI355X):",
          "", "```"] + commands + ["```", "", f"Library sources sha256 {source_hash()[:16]}…", "",
          "Medians per dispatch (BF16 weights, no pending write or injection; down = `hc_down`, up = "
          "`hc_up_mfma`), then per wave: WAIT_ANY (waiting on anything, mostly memory), "
          "ACTIVE_INST_VALU (the wave's VALU issue) and WAIT_INST_ANY (an instruction ready but not issued: "
          "dependencies, or the other wave of the SIMD issuing). Counts are the counters' own units.", "",
          "| kernel | T | waves | wave cycles | WAIT_ANY | WAIT_INST_ANY | ACTIVE_INST_ANY | ACTIVE_INST_VALU | "
          "per wave: cycles | WAIT_ANY | VALU | WAIT_INST |",
          "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for key in sorted(vals):
        v = {n: statistics.median(vals[key][n]) for n in SQ_COUNTERS if vals[key][n]}
        if len(v) < len(SQ_COUNTERS):
            continue
        w = v["SQ_WAVES"]
        md.append(f"| {key[0]} | {key[1]} | {w:.0f} | {v['SQ_WAVE_CYCLES']:,.0f} | {v['SQ_WAIT_ANY']:,.0f} | "
                  f"{v['SQ_WAIT_INST_ANY']:,.0f} | {v['SQ_ACTIVE_INST_ANY']:,.0f} | {v['SQ_ACTIVE_INST_VALU']:,.0f} | "
                  f"{v['SQ_WAVE_CYCLES'] / w:.0f} | {v['SQ_WAIT_ANY'] / w:.0f} | {v['SQ_ACTIVE_INST_VALU'] / w:.0f} | "
                  f"{v['SQ_WAIT_INST_ANY'] / w:.0f} |")
    return "\n".join(md) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--sq", help="a rocprofv3 --pmc run over SQ_COUNTERS: write only its table to --md")
    ap.add_argument("--trace")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--md", required=True)
    ap.add_argument("--json")
    ap.add_argument("--command", action="append", default=[])
    ap.add_argument("--bench-log", help="stdout of the traced bench run (its JSON line: the traced event figure)")
    ap.add_argument("--bench-json", help="the JSON line of an untraced bench.py run of the same session")
    a = ap.parse_args()
    if a.sq:
        with open(a.md, "w") as fh:
            fh.write(sq_table(a.sq, a.command))
        return
    if not (a.trace and a.fetch and a.write and a.json):
        ap.error("--trace, --fetch, --write and --json are required (or --sq)")

    dur = durations(a.trace)
    fetch, fetch_copy = counters(a.fetch, "FETCH_SIZE")
    write, write_copy = counters(a.write, "WRITE_SIZE")
    fs, ws = COPY_BYTES / 1024.0 / fetch_copy, COPY_BYTES / 1024.0 / write_copy

    rec = {"about": "HBM bytes per read (down + up kernels, no pending write or injection) on MI355X from two "
                    "rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE), each scaled by the same counter for a "
                    f"64 MiB device copy: FETCH_SIZE x {fs:.4f}, WRITE_SIZE x {ws:.4f}",
           "commands": a.command, "fetch_scale": fs, "write_scale": ws,
           "calibration_copy_KiB": {"bytes": COPY_BYTES, "FETCH_SIZE": fetch_copy, "WRITE_SIZE": write_copy},
           "source_sha256": build.source_hash()}
    lines = ["| format | T | down avg µs | up avg µs | sum µs | down FETCH KiB | up FETCH KiB | down WRITE KiB | "
             "up WRITE KiB | HBM bytes/read (scaled) | algorithmic bytes/read |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for fmt, fname in FORMATS.items():
        per_T, tot = {}, []
        for T in range(1, 17):
            kd, ku = ("down", T, fmt, False, False), ("up", T, fmt, False, False)
            if kd not in dur or ku not in dur:
                continue
            f_d, f_u = fetch.get(kd), fetch.get(ku)
            w_d, w_u = write.get(kd), write.get(ku)
            row = {"down_us": round(dur[kd][0], 3), "up_us": round(dur[ku][0], 3),
                   "calls": dur[kd][1], "algorithmic_bytes": algorithmic_bytes(fmt, T)}
            if None not in (f_d, f_u, w_d, w_u):
                fb, wb = (f_d + f_u) * 1024 * fs, (w_d + w_u) * 1024 * ws
                row.update(fetch_bytes=int(round(fb)), write_bytes=int(round(wb)), total_bytes=int(round(fb + wb)))
                if T <= 8:
                    tot.append(fb + wb)
            per_T[str(T)] = row
            lines.append(f"| {fname} | {T} | {row['down_us']:.3f} | {row['up_us']:.3f} | "
                         f"{row['down_us'] + row['up_us']:.3f} | "
                         + " | ".join("—" if v is None else f"{v:.1f}" for v in (f_d, f_u, w_d, w_u))
                         + " | " + (f"{row['total_bytes']:,}" if "total_bytes" in row else "—")
                         + f" | {row['algorithmic_bytes']:,} |")
        if per_T:
            rec[fname] = {"per_T": per_T,
                          "bytes_per_read_mean_T1_8": int(round(sum(tot) / len(tot))) if len(tot) == 8 else None}
    tr = timed_region(a.trace)
    if tr:
        rec["timed_region"] = {"reads": tr[0], "us_per_read": round(tr[1], 3), "down_avg_us": round(tr[2], 3),
                               "up_avg_us": round(tr[3], 3),
                               "down_plus_up_us_p10_p50_p90": [round(tr[4][p], 3) for p in (10, 50, 90)],
                               "per_T_down_plus_up_us_p10_p50_p90": {str(T): [round(x, 3) for x in percentiles(v)]
                                                                     for T, v in sorted(tr[5].items())}}
    q = ("quantize",)
    if q in dur:
        rec["q8_0_quantize"] = {"avg_us": round(dur[q][0], 3), "calls": dur[q][1],
                                "fetch_KiB": fetch.get(q), "write_KiB": write.get(q)}

    mv_lines = []
    for T in range(1, 5):
        k = ("matvec", T, (MV_COLS // 8 + 63) // 64)
        if k in dur:
            row = {"avg_us": round(dur[k][0], 3), "calls": dur[k][1], "algorithmic_bytes": matvec_bytes(T),
                   "algorithmic_GBps": round(matvec_bytes(T) / dur[k][0] / 1e3, 1)}
            if k in fetch and k in write:
                row["hbm_bytes"] = int(round(fetch[k] * 1024 * fs + write[k] * 1024 * ws))
            rec.setdefault("matvec_bf16", {})[str(T)] = row
            mv_lines.append(f"| {T} | {row['avg_us']:.3f} | {row['algorithmic_GBps']:.0f} | "
                            + (f"{row['hbm_bytes']:,}" if "hbm_bytes" in row else "—")
                            + f" | {row['algorithmic_bytes']:,} |")

    with open(a.json, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    md = ["# Kernel durations and HBM traffic per read (MI355X)", "",
          "Commands (run from the repository root, on one MI355X):", "", "```"] + a.command + ["```", "",
          f"Counter scale from a 64 MiB device copy in the same runs: FETCH_SIZE x {fs:.4f}, WRITE_SIZE x {ws:.4f}.",
          f"Library sources sha256 {rec['source_sha256'][:16]}…", ""] + lines
    for fname in FORMATS.values():
        if fname in rec and rec[fname]["bytes_per_read_mean_T1_8"]:
            alg = sum(algorithmic_bytes(0 if fname == "bf16" else 1, T) for T in range(1, 9)) / 8
            b = rec[fname]["bytes_per_read_mean_T1_8"]
            md.append("")
            md.append(f"{fname}: mean over T = 1..8, {b:,} HBM bytes per read vs {int(alg):,} algorithmic "
                      f"({100.0 * (b / alg - 1):+.1f} %).")
    if tr:
        def last_json(path):
            if not path:
                return None
            with open(path) as fh:
                js = [ln for ln in fh if ln.startswith("{")]
            return json.loads(js[-1])["value"] if js else None
        traced, untraced = last_json(a.bench_log), last_json(a.bench_json)
        rec["timed_region"].update(bench_event_us_per_read_untraced=untraced, bench_event_us_per_read_traced=traced)
        tot = tr[2] + tr[3]
        md += ["", f"Timed region of the traced bench run (its timed steps, found between two marker kernels): "
                   f"{tr[0]} reads; average dispatch duration hc_down {tr[2]:.3f} µs + hc_up_mfma {tr[3]:.3f} µs = "
                   f"{tot:.3f} µs per read (p10 / p50 / p90 of down + up per read: "
                   f"{tr[4][10]:.3f} / {tr[4][50]:.3f} / {tr[4][90]:.3f} µs)."
                   + (f" An untraced `python bench.py` of the same session measured {untraced:.3f} µs per read "
                      f"event-timed (its `value`; {100 * tot / untraced - 100:+.1f} %)." if untraced else "")
                   + (f" Under the tracer the dispatches are spaced out: the traced run's own event figure is "
                      f"{traced:.3f} µs per read." if traced else "")]
        if tr[5]:
            md += ["", "Per T in the timed region, down + up per read (µs):", "",
                   "| T | reads | p10 | p50 | p90 |", "|---|---|---|---|---|"]
            for T, v in sorted(tr[5].items()):
                p10, p50, p90 = percentiles(v)
                md.append(f"| {T} | {len(v)} | {p10:.3f} | {p50:.3f} | {p90:.3f} |")
    cal_lines, ab_lines = [], []
    for T in range(1, 17):
        kd, ku, kld, klu = ("down", T, 0, False, False), ("up", T, 0, False, False), ("cal_down_loads", T), \
            ("cal_up_loads", T)
        if kld in dur and klu in dur and kd in dur and ku in dur:
            cal_lines.append(f"| {T} | {dur[kd][0]:.3f} | {dur[kld][0]:.3f} | {dur[kd][0] - dur[kld][0]:+.3f} | "
                             f"{dur[ku][0]:.3f} | {dur[klu][0]:.3f} | {dur[ku][0] - dur[klu][0]:+.3f} |")
        kv, km = ("cal_up_valu", T), ("cal_up_mfma", T)
        if kv in dur and km in dur:
            rec.setdefault("up_kernels_alone", {})[str(T)] = {"valu_us": round(dur[kv][0], 3),
                                                             "mfma_us": round(dur[km][0], 3)}
            ab_lines.append(f"| {T} | {dur[kv][0]:.3f} | {dur[km][0]:.3f} | {dur[km][0] - dur[kv][0]:+.3f} | "
                            "matrix cores |")
    slab_lines = []
    for T in range(1, 9):
        ks = [("cal_slab_down", T, k) for k in range(3)]
        if all(k in dur for k in ks) and ("cal_slab_up", T) in dur:
            rec.setdefault("slab_probe", {})[str(T)] = {"down_loads_us": round(dur[ks[0]][0], 3),
                                                        "down_stores_us": round(dur[ks[1]][0], 3),
                                                        "down_finish_us": round(dur[ks[2]][0], 3),
                                                        "up_lo_loads_us": round(dur[("cal_slab_up", T)][0], 3)}
            slab_lines.append(f"| {T} | {dur[ks[0]][0]:.3f} | {dur[ks[1]][0]:.3f} | {dur[ks[2]][0]:.3f} | "
                              f"{dur[ks[2]][0] - dur[ks[1]][0]:+.3f} | {dur[('cal_slab_up', T)][0]:.3f} |")
    sread_lines = []
    for T in range(1, 9):
        kd, ku = ("cal_slab_read_down", T, False), ("cal_slab_read_up", T, False)
        rd, ru = ("down", T, 0, False, False), ("up", T, 0, False, False)
        if kd in dur and ku in dur and rd in dur and ru in dur:
            rec.setdefault("slab_read", {})[str(T)] = {"down_us": round(dur[kd][0], 3), "up_us": round(dur[ku][0], 3)}
            sread_lines.append(f"| {T} | {dur[kd][0]:.3f} | {dur[ku][0]:.3f} | {dur[kd][0] + dur[ku][0]:.3f} | "
                               f"{dur[rd][0]:.3f} | {dur[ru][0]:.3f} | {dur[rd][0] + dur[ru][0]:.3f} |")
    if ("cal_empty",) in dur:
        rec["cal_empty_avg_us"] = round(dur[("cal_empty",)][0], 3)
    if cal_lines:
        md += ["", "Calibration kernels (`libhcr_calib.so`, the read's grids with only its global loads) against the "
                   "read's own kernels, BF16, average µs per dispatch"
                   + (f"; an empty kernel on the same grids averages {dur[('cal_empty',)][0]:.3f} µs"
                      if ("cal_empty",) in dur else "") + ":", "",
               "| T | hc_down | its loads alone | excess | up kernel | its loads alone | excess |",
               "|---|---|---|---|---|---|---|"] + cal_lines
    if ab_lines:
        md += ["", "The two up kernels alone (the calibration library's `cal_up_valu<T>` = hc_up's body, "
                   "`cal_up_mfma<T>` = hc_up_mfma's body; BF16, no pending write or injection), average µs per "
                   "dispatch:", "", "| T | vector ALUs (v_dot2) | matrix cores | difference | the read dispatches |",
               "|---|---|---|---|---|"] + ab_lines
    if slab_lines:
        md += ["", "The pages' down shape as probes (`hcrc_slab_pair`: 10 rows x a 1,280-column slab, 256 work-groups; "
                   "the up grid loading lo only), average µs per dispatch of the down kernel: its loads, + its "
                   "partial stores, + the last-arriver finish (agent-scope acquire-release counter, the 8th "
                   "work-group of a row group sums the 8 slabs):", "",
               "| T | loads | + stores | + finish | the finish's cost | up kernel loading lo |", "|---|---|---|---|---|---|"]
        md += slab_lines
    if sread_lines:
        md += ["", "The whole read in the pages' shape with its arithmetic (`hcrc_slab_read`: the slab down kernel "
                   "with its partials, sums of squares and last-arriver finish applying rs and writing lo, then the "
                   "read's up kernel on lo alone; no pending write or injection) against the read, average µs per "
                   "dispatch:", "",
               "| T | slab down + finish | up on lo | sum | hc_down | hc_up_mfma | sum |",
               "|---|---|---|---|---|---|---|"] + sread_lines
    if q in dur:
        md += ["", f"q8_quantize (one 320 x 10240 or 10240 x 320 matrix): {dur[q][0]:.3f} µs average over "
                   f"{dur[q][1]} calls."]
    if mv_lines:
        md += ["", f"Skinny BF16 matvec ({MV_ROWS} x {MV_COLS}, 8 rotated copies), `mv_bf16<T, 5>`:", "",
               "| T | avg µs | algorithmic GB/s | HBM bytes/call (scaled) | algorithmic bytes/call |",
               "|---|---|---|---|---|"] + mv_lines
    with open(a.md, "w") as fh:
        fh.write("\n".join(md) + "\n")


if __name__ == "__main__":
    main()
