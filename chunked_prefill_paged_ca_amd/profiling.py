"""Summaries of rocprofv3 output for profiles/ (kernel statistics, counter-derived HBM traffic).

    python -m chunked_prefill_paged_ca_amd.profiling stats <kernel_stats.csv> <title> <command>
        -> markdown table of per-kernel dispatch durations on stdout
    python -m chunked_prefill_paged_ca_amd.profiling traffic <fetch counter_collection.csv>
           <write counter_collection.csv> <copy MiB> <command> <workload>
        -> JSON: FETCH_SIZE / WRITE_SIZE per attention launch, scaled by what the same counters
           read for a device-to-device copy of known size, on stdout; <workload> is the name of
           the workload the counters were taken on (a reading holds for that workload only)

Neither touches the GPU; they read the CSV files rocprofv3 wrote.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
ATTENTION_SOURCES = ("attn_mixed.hip", "attn_decode.h", "attn_chunk.h", "mfma.h", "internal.h")


def kernel_sources_sha256() -> str:
    """Hash of the attention kernel's sources: a stored counter reading is valid only for them."""
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


def main(argv):
    if len(argv) >= 4 and argv[0] == "stats":
        sys.stdout.write(stats_md(argv[1], argv[2], argv[3]))
    elif len(argv) >= 6 and argv[0] == "traffic":
        print(json.dumps(traffic(argv[1], argv[2], int(argv[3]), argv[4], argv[5]), indent=1))
    else:
        print(__doc__, file=sys.stderr)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
