"""Summaries of rocprofv3 output for profiles/ (kernel statistics, counter-derived HBM traffic).

    python -m chunked_prefill_paged_ca_amd.profiling stats <kernel_stats.csv> <title> <command>
        -> markdown table of per-kernel dispatch durations on stdout
    python -m chunked_prefill_paged_ca_amd.profiling trace <kernel_trace.csv> <title> <command>
           [<kernel substring>:<N>]
        -> markdown table of dispatch durations per (kernel, grid size) on stdout, and the
           statistics of the first N dispatches of one kernel
    python -m chunked_prefill_paged_ca_amd.profiling traffic <fetch counter_collection.csv>
           <write counter_collection.csv> <copy MiB> <command> <workload>
        -> JSON: FETCH_SIZE / WRITE_SIZE per attention launch, scaled by what the same counters
           read for a device-to-device copy of known size, on stdout; <workload> is the name of
           the workload the counters were taken on (a reading holds for that workload only)
    python -m chunked_prefill_paged_ca_amd.profiling parts <SQ counter_collection.csv>
           <fetch counter_collection.csv> <write counter_collection.csv> <parts_run output> <command>
           [<stall counter_collection.csv>]
        -> markdown: MFMA utilisation, executed bf16 MFMA flops and HBM bytes of the decode-only
           and chunk-only attention launches of parts_run.py, on stdout

None touches the GPU; they read the CSV files rocprofv3 wrote.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# The attention kernel's sources and the host code that shapes its launch (decode shares, chunk
# key splits and hence how many fp32 partials are written and merged).
ATTENTION_SOURCES = ("attn_mixed.hip", "attn_decode.h", "attn_chunk.h", "mfma.h", "internal.h",
                     "api.hip", "merge.hip")


def kernel_sources_sha256() -> str:
    """Hash of the sources behind the attention launch: a stored counter reading is valid only
    for them."""
    h = hashlib.sha256()
    for name in ATTENTION_SOURCES:
        with open(os.path.join(HERE, "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def short_name(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0]


def stats_md(path: str, title: str, cmd: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = [f"# {title}", "", "Command (run from the repository root on one MI355X; TMPDIR=/tmp):", "",
           f"    {cmd}", "", "rocprofv3 kernel statistics (per-dispatch durations):", "",
           "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {short_name(r['Name'])[:80]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.2f} |")
    return "\n".join(out) + "\n"


def trace_md(path: str, title: str, cmd: str, first: str = "") -> str:
    """Per-dispatch durations from a rocprofv3 kernel_trace.csv, grouped by kernel AND grid size:
    one bench run launches the same kernel for several workloads (different grids), and each
    workload's launches are averaged on their own.  first = "<kernel substring>:<N>" adds the
    statistics of the first N dispatches of that kernel (e.g. the launches the bench's roofline
    line timed, which come first in its run)."""
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    gcols = [c for c in ("Grid_Size_X", "Grid_Size") if rows and c in rows[0]]
    groups = defaultdict(list)
    first_at = {}
    for i, r in enumerate(rows):
        grid = int(r[gcols[0]]) if gcols else 0
        key = (short_name(r["Kernel_Name"]), grid)
        groups[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        first_at.setdefault(key, i)
    out = [f"# {title}", "", "Command (run from the repository root on one MI355X; TMPDIR=/tmp):", "",
           f"    {cmd}", "", "rocprofv3 kernel trace, grouped by kernel and grid size (work-items), "
           "in order of first dispatch:", "",
           "| kernel | grid | calls | avg us | p10 us | p50 us | p90 us |", "|---|---|---|---|---|---|---|"]
    for key in sorted(groups, key=lambda k: first_at[k]):
        v = np.asarray(groups[key])
        out.append(f"| {key[0][:70]} | {key[1]} | {v.size} | {v.mean():.2f} | "
                   f"{np.percentile(v, 10):.2f} | {np.percentile(v, 50):.2f} | {np.percentile(v, 90):.2f} |")
    if first:
        sub, n = first.rsplit(":", 1)
        v = np.asarray([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows
                        if sub in r["Kernel_Name"]][:int(n)])
        out += ["", f"The first {v.size} dispatches of `{sub}` (in this run, the launches the bench's "
                f"roofline line timed): avg {v.mean():.2f} us, p10 {np.percentile(v, 10):.2f}, "
                f"p50 {np.percentile(v, 50):.2f}, p90 {np.percentile(v, 90):.2f} us."]
    return "\n".join(out) + "\n"


def _per_dispatch(path: str, counter: str):
    """{dispatch id: (kernel name, value summed over the counter's instances)}."""
    acc = defaultdict(float)
    names = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d = r["Dispatch_Id"]
        acc[d] += float(r["Counter_Value"])
        names[d] = r["Kernel_Name"]
    return {d: (names[d], v) for d, v in acc.items()}


def traffic(fetch_csv: str, write_csv: str, copy_mib: int, cmd: str, workload: str) -> dict:
    copy_bytes = copy_mib * (1 << 20)
    res = {"command": cmd, "workload": workload, "copy_reference_bytes": copy_bytes}
    for key, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        per = _per_dispatch(path, counter)  # KiB per dispatch
        attn = [v for n, v in per.values() if "mixed_kernel" in n]
        copies = [v for n, v in per.values() if "copy" in n.lower()]
        if not attn or not copies:
            raise SystemExit(f"{path}: no attention or copy dispatch with {counter}")
        copy_kib = max(copies)
        factor = copy_kib * 1024.0 / copy_bytes  # counter bytes per real byte
        attn_kib = sum(attn) / len(attn)
        res[key] = {"counter": counter, "attention_kib_per_launch": round(attn_kib, 1),
                    "launches": len(attn), "copy_kib": round(copy_kib, 1),
                    "factor": round(factor, 4), "bytes_per_launch": int(attn_kib * 1024.0 / factor)}
    res["hbm_bytes_per_launch"] = res["fetch"]["bytes_per_launch"] + res["write"]["bytes_per_launch"]
    res["sources_sha256"] = kernel_sources_sha256()
    return res


def _instances(path: str):
    """{dispatch id: (kernel name, {counter: [values of its instances]})}."""
    out = {}
    for r in csv.DictReader(open(path)):
        d = int(r["Dispatch_Id"])
        name, vals = out.setdefault(d, (r["Kernel_Name"], defaultdict(list)))
        vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
    return out


SIMDS = 256 * 4  # MI355X: 256 CUs x 4 SIMDs
XCDS = 8


STALL_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
                  "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS")


def parts(sq_csv: str, fetch_csv: str, write_csv: str, timing: dict, cmd: str,
          stall_csv: str = "") -> str:
    """Counters of the decode-only and chunk-only attention launches of parts_run.py.

    The attention dispatches alternate in launch order (timing["attention_launch_order"]).
    rocprofv3 writes each counter summed over its instances (SIMDs, shader engines, XCDs), so
    GRBM_GUI_ACTIVE / 8 is one XCD's active cycles and MFMA utilisation -- rocprofv3's MfmaUtil --
    is SQ_VALU_MFMA_BUSY_CYCLES / SIMDs over that; executed bf16 MFMA flops are SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; HBM bytes are
    FETCH_SIZE and WRITE_SIZE scaled by what the same counters read for the reference copy
    (timing["copy_mib"] MiB read and written)."""
    order = timing["attention_launch_order"]
    copy_bytes = timing["copy_mib"] * (1 << 20)

    def attention(per):
        ids = sorted(d for d, (n, _) in per.items() if "mixed_kernel" in n)
        return {kind: [per[d][1] for i, d in enumerate(ids) if order[i % len(order)] == kind] for kind in order}

    def scaled(path, counter):
        per = _instances(path)
        copies = [sum(v[counter]) for n, v in per.values() if "copy" in n.lower() and counter in v]
        if not copies:
            raise SystemExit(f"{path}: no reference copy with {counter}")
        factor = max(copies) * 1024.0 / copy_bytes
        return {k: float(np.mean([sum(v[counter]) for v in vs])) * 1024.0 / factor
                for k, vs in attention(per).items()}, factor

    sq = attention(_instances(sq_csv))
    fetch, ff = scaled(fetch_csv, "FETCH_SIZE")
    write, wf = scaled(write_csv, "WRITE_SIZE")
    ms = timing["kernel_ms"]
    rows = []
    for kind in order:
        vs = sq[kind]
        util = float(np.mean([sum(v["SQ_VALU_MFMA_BUSY_CYCLES"]) / SIMDS / (sum(v["GRBM_GUI_ACTIVE"]) / XCDS)
                              for v in vs]))
        mops = float(np.mean([sum(v["SQ_INSTS_VALU_MFMA_MOPS_BF16"]) for v in vs])) * 512
        t = ms[kind] * 1e-3
        rows.append((kind, ms[kind] * 1e3, util, mops, mops / t / 1e12, fetch[kind], write[kind],
                     (fetch[kind] + write[kind]) / t / 1e9, len(vs)))
    out = [f"# Decode-only and chunk-only attention launches: {timing['workload']}", "",
           "Command (run from the repository root on one MI355X; TMPDIR=/tmp):", "", f"    {cmd}", "",
           f"Event time per launch from parts_run ({timing['steps']} timed steps); counters averaged "
           f"over every launch of each kind ({rows[0][-1]} each).  FETCH_SIZE reads {ff:.3g} and "
           f"WRITE_SIZE {wf:.3g} counter KiB per real KiB on the reference copy; bytes below are "
           "scaled by those factors.", "",
           "| launch | event us | MFMA busy (MfmaUtil) | executed bf16 MFMA flops | executed TF/s | HBM read MB | "
           "HBM written MB | HBM GB/s |", "|---|---|---|---|---|---|---|---|"]
    for kind, us, util, mops, tf, rd, wr, gbs, _ in rows:
        out.append(f"| {kind} | {us:.1f} | {100 * util:.1f} % | {mops / 1e9:.1f} G | {tf:.0f} | "
                   f"{rd / 1e6:.1f} | {wr / 1e6:.1f} | {gbs:.0f} |")
    if stall_csv:
        st = attention(_instances(stall_csv))
        out += ["", "Where the waves' time goes (a fourth counter pass; each SQ counter summed over its "
                "instances and averaged over the launches of each kind; shares are of SQ_WAVE_CYCLES, the "
                "summed residency of every wave, in the same units as the per-wave ACTIVE_INST and "
                "WAIT_INST counters):", "",
                "| launch | issuing VALU | issuing LDS | waiting on any dependency | waiting on LDS | "
                "LDS instructions | LDS bank-conflict cycles |", "|---|---|---|---|---|---|---|"]
        for kind in order:
            vs = st[kind]

            def mean(c):
                return float(np.mean([sum(v[c]) for v in vs if c in v])) if vs and c in vs[0] else float("nan")
            wave = mean("SQ_WAVE_CYCLES")
            out.append(f"| {kind} | {100 * mean('SQ_ACTIVE_INST_VALU') / wave:.1f} % | "
                       f"{100 * mean('SQ_ACTIVE_INST_LDS') / wave:.1f} % | "
                       f"{100 * mean('SQ_WAIT_INST_ANY') / wave:.1f} % | "
                       f"{100 * mean('SQ_WAIT_INST_LDS') / wave:.1f} % | {mean('SQ_INSTS_LDS') / 1e6:.2f} M | "
                       f"{mean('SQ_LDS_BANK_CONFLICT') / 1e6:.3f} M |")
    ca = timing["chunk_alg_flops"]
    out += ["", f"Algorithmic work: decode rows {timing['decode_alg_bytes'] / 1e6:.1f} MB "
            f"({timing['decode_alg_bytes'] / (ms['decode'] * 1e-3) / 1e9:.0f} GB/s over the decode launch, "
            f"{timing['decode_alg_bytes'] / (ms['decode'] * 1e-3) / 8e12 * 100:.1f} % of 8 TB/s); chunk rows "
            f"{ca / 1e9:.1f} GFLOP ({ca / (ms['chunk'] * 1e-3) / 1e12:.0f} TF/s over the chunk launch, "
            f"{ca / (ms['chunk'] * 1e-3) / 2.5e15 * 100:.1f} % of 2.5 PFLOP/s) and "
            f"{timing['chunk_alg_bytes'] / 1e6:.1f} MB of unique K/V and q."]
    return "\n".join(out) + "\n"


def main(argv):
    if len(argv) >= 6 and argv[0] == "parts":
        timing = json.loads(open(argv[4]).read().strip().splitlines()[-1])
        sys.stdout.write(parts(argv[1], argv[2], argv[3], timing, argv[5],
                               argv[6] if len(argv) > 6 else ""))
    elif len(argv) >= 4 and argv[0] == "trace":
        sys.stdout.write(trace_md(argv[1], argv[2], argv[3], argv[4] if len(argv) > 4 else ""))
    elif len(argv) >= 4 and argv[0] == "stats":
        sys.stdout.write(stats_md(argv[1], argv[2], argv[3]))
    elif len(argv) >= 6 and argv[0] == "traffic":
        print(json.dumps(traffic(argv[1], argv[2], int(argv[3]), argv[4], argv[5]), indent=1))
    else:
        print(__doc__, file=sys.stderr)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
