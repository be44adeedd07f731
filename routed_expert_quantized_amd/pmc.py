"""Reduce rocprofv3 counter-collection CSVs to per-kernel means per dispatch.

    python -m routed_expert_quantized_amd.pmc reduce <counter_collection.csv> [...]
        prints one JSON object: {kernel: {counter: mean value per dispatch, "dispatches": n}}

    python -m routed_expert_quantized_amd.pmc stats <kernel_stats.csv>
        prints a markdown table of per-kernel calls and average/min/max durations

    python -m routed_expert_quantized_amd.pmc traffic --fetch F.json --write W.json
        --kernel NAME_SUBSTRING --calib NAME_SUBSTRING --calib-bytes B [--sha S]
        converts the kernel's FETCH_SIZE / WRITE_SIZE (KiB per dispatch) into bytes
        per launch, scaled by the factor a plain copy of B bytes read and wrote
        under the same counters (bytes moved / counter reading).

Counter runs use one counter per pass (FETCH_SIZE, then WRITE_SIZE), launched as
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o run -- python3 bench.py ...
"""
from __future__ import annotations

import csv
import json
import sys
from collections import defaultdict


def _short(name: str) -> str:
    name = name.strip().replace("(anonymous namespace)", "{anon}")
    if name.startswith("void "):
        name = name[5:]
    # drop the argument list, keep template arguments
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def reduce(paths):
    per = defaultdict(lambda: defaultdict(dict))  # kernel -> counter -> dispatch -> value
    for p in paths:
        with open(p, newline="") as f:
            for r in csv.DictReader(f):
                k = _short(r.get("Kernel_Name", ""))
                c = r.get("Counter_Name", "")
                d = (p, r.get("Dispatch_Id", ""))
                per[k][c][d] = per[k][c].get(d, 0.0) + float(r.get("Counter_Value", 0.0))
    out = {}
    for k, cs in per.items():
        o = {}
        for c, ds in cs.items():
            o[c] = sum(ds.values()) / len(ds)
            o["dispatches"] = len(ds)
        out[k] = o
    return out


def _find(d, sub):
    hits = [k for k in d if sub in k]
    if not hits:
        raise SystemExit(f"no kernel matching {sub!r}; kernels: {sorted(d)}")
    if len(hits) > 1:
        hits.sort(key=lambda k: -d[k].get("dispatches", 0))
    return hits[0]


def traffic(fetch, write, kernel, calib, calib_bytes, sha=None):
    kf, kw = _find(fetch, kernel), _find(write, kernel)
    cf, cw = _find(fetch, calib), _find(write, calib)
    f_kib, w_kib = fetch[kf]["FETCH_SIZE"], write[kw]["WRITE_SIZE"]
    cal_f, cal_w = fetch[cf]["FETCH_SIZE"], write[cw]["WRITE_SIZE"]
    sf = calib_bytes / cal_f  # bytes per counter unit, reads
    sw = calib_bytes / cal_w  # bytes per counter unit, writes
    res = {"kernel": kf, "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib,
           "dispatches": fetch[kf]["dispatches"], "calib_kernel": cf, "calib_bytes": calib_bytes,
           "calib_fetch_kib": cal_f, "calib_write_kib": cal_w, "fetch_scale": sf, "write_scale": sw,
           "fetch_bytes_per_launch": f_kib * sf, "write_bytes_per_launch": w_kib * sw,
           "bytes_per_launch": f_kib * sf + w_kib * sw}
    if sha:
        res["kernel_source_sha"] = sha
    return res


def stats_table(path, top=12):
    """Markdown table of a rocprofv3 kernel_stats.csv: calls and per-launch
    average / min / max in microseconds, longest total time first."""
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            rows.append((_short(r["Name"]), int(r["Calls"]), float(r["TotalDurationNs"]),
                         float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"])))
    rows.sort(key=lambda r: -r[2])
    out = ["| kernel | calls | avg (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
    for name, calls, _, avg, mn, mx in rows[:top]:
        if not name.startswith("moe::") and "<" in name:
            name = name[:name.index("<")] + "<…>"  # library kernels other than this one: base name only
        out.append(f"| `{name}` | {calls} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} |")
    return "\n".join(out)


def main(argv):
    if len(argv) >= 2 and argv[0] == "stats":
        print(stats_table(argv[1]))
        return 0
    if len(argv) >= 2 and argv[0] == "reduce":
        print(json.dumps(reduce(argv[1:]), indent=1))
        return 0
    if argv and argv[0] == "traffic":
        import argparse
        ap = argparse.ArgumentParser()
        ap.add_argument("--fetch", required=True)
        ap.add_argument("--write", required=True)
        ap.add_argument("--kernel", required=True)
        ap.add_argument("--calib", required=True)
        ap.add_argument("--calib-bytes", type=float, required=True)
        ap.add_argument("--sha", default=None)
        a = ap.parse_args(argv[1:])
        with open(a.fetch) as f:
            fj = json.load(f)
        with open(a.write) as f:
            wj = json.load(f)
        print(json.dumps(traffic(fj, wj, a.kernel, a.calib, a.calib_bytes, a.sha), indent=1))
        return 0
    print(__doc__, file=sys.stderr)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
