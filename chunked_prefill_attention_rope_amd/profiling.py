"""Summaries of rocprofv3 CSV output (kernel-trace stats and PMC counters).

    python -m chunked_prefill_attention_rope_amd.profiling stats <kernel_stats.csv>
    python -m chunked_prefill_attention_rope_amd.profiling pmc <counter_collection.csv> [regex]

    python -m chunked_prefill_attention_rope_amd.profiling traffic <key> <layer text> \
        <profile_attn args> <fetch.csv> <write.csv> <copy_fetch.csv> <copy_write.csv> \
        <copy_bytes> [regex]

`stats` prints a markdown table of per-kernel calls and durations; `pmc`
prints, per kernel, the counters summed over the dispatch's instances and
averaged over its dispatches; `digest` prints the hash of the attention
sources that a traffic measurement is tied to; `traffic` turns a FETCH_SIZE run
and a WRITE_SIZE run of one workload's attention call (and the same two counters
on a plain copy of copy_bytes, which fixes their scale) into HBM bytes per call,
recorded in profiles/traffic.json with the source digest.
"""
import collections
import csv
import hashlib
import json
import os
import re
import sys

_CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
# sources whose change invalidates counters measured on the attention call
ATTN_SOURCES = ("attn_mfma.hip", "attn_mfma_ops.h", "attn_valu.hip", "attn_common.h", "cp_common.h",
                "cp_api.hip")


def source_digest(names=ATTN_SOURCES):
    """sha1 over the given csrc files (identifies the kernel build a measurement used)."""
    h = hashlib.sha1()
    for n in names:
        with open(os.path.join(_CSRC, n), "rb") as f:
            h.update(n.encode() + b"\0" + f.read())
    return h.hexdigest()


def kernel_stats(path):
    rows = list(csv.DictReader(open(path)))
    out = []
    for r in rows:
        out.append(dict(name=r["Name"], calls=int(r["Calls"]),
                        avg_us=float(r["AverageNs"]) / 1e3, total_us=float(r["TotalDurationNs"]) / 1e3,
                        min_us=float(r["MinNs"]) / 1e3, max_us=float(r["MaxNs"]) / 1e3,
                        pct=float(r["Percentage"])))
    return out


def pmc_per_kernel(path, pattern=None):
    """{kernel: {counter: mean over dispatches of the per-dispatch sum}}."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for r in csv.DictReader(open(path)):
        if pattern and not re.search(pattern, r["Kernel_Name"]):
            continue
        d = int(r["Dispatch_Id"])
        per[d][r["Counter_Name"]] += float(r["Counter_Value"])
        names[d] = r["Kernel_Name"]
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for d, cs in per.items():
        for c, v in cs.items():
            agg[names[d]][c].append(v)
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in agg.items()}


def counter_kib_per_call(path, counter, pattern):
    """KiB of one counter per call: per-dispatch sums averaged over the dispatches of
    each kernel matching pattern, then added over those kernels (one call launches each
    once)."""
    res = pmc_per_kernel(path, pattern)
    return sum(cs.get(counter, 0.0) for cs in res.values()), sorted(res)


PMC_CMD = ("rocprofv3 --pmc {FETCH_SIZE|WRITE_SIZE} --output-format csv -d <dir> -o p -- "
           "python3 -m chunked_prefill_attention_rope_amd.profile_attn ")


def record_traffic(workload, layer, args, fetch_csv, write_csv, cal_fetch_csv, cal_write_csv,
                   copy_bytes, pattern=r"k_attn_"):
    # the copy itself only (the run also fills its source buffer)
    cal_f, _ = counter_kib_per_call(cal_fetch_csv, "FETCH_SIZE", r"copyBuffer")
    cal_w, _ = counter_kib_per_call(cal_write_csv, "WRITE_SIZE", r"copyBuffer")
    ff, fw = copy_bytes / (cal_f * 1024), copy_bytes / (cal_w * 1024)
    f_kib, names = counter_kib_per_call(fetch_csv, "FETCH_SIZE", pattern)
    w_kib, _ = counter_kib_per_call(write_csv, "WRITE_SIZE", pattern)
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "profiles", "traffic.json")
    rec = json.load(open(path)) if os.path.exists(path) else {}
    rec["_calibration"] = {
        "copy_bytes": copy_bytes, "fetch_kib": round(cal_f, 2), "write_kib": round(cal_w, 2),
        "fetch_factor": round(ff, 4), "write_factor": round(fw, 4),
        "command": PMC_CMD + f"--copy-bytes {copy_bytes} --reps 3"}
    fb, wb = int(round(f_kib * 1024 * ff)), int(round(w_kib * 1024 * fw))
    rec[workload] = {
        "bytes_per_call": fb + wb, "fetch_bytes": fb, "write_bytes": wb,
        "fetch_kib_raw": round(f_kib, 2), "write_kib_raw": round(w_kib, 2),
        "kernels": " + ".join(short(n, 40) for n in names), "layer": layer,
        "source_sha1": source_digest(), "command": PMC_CMD + args}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    return rec[workload]


def short(name, n=90):
    name = re.sub(r"\(anonymous namespace\)::", "", name)
    return name if len(name) <= n else name[:n - 3] + "..."


def main(argv):
    if len(argv) >= 2 and argv[0] == "stats":
        print("| kernel | calls | avg us | min us | max us | total us | % |")
        print("|---|---:|---:|---:|---:|---:|---:|")
        for k in kernel_stats(argv[1]):
            print(f"| `{short(k['name'])}` | {k['calls']} | {k['avg_us']:.2f} | {k['min_us']:.2f} "
                  f"| {k['max_us']:.2f} | {k['total_us']:.1f} | {k['pct']:.1f} |")
        return 0
    if len(argv) >= 2 and argv[0] == "pmc":
        res = pmc_per_kernel(argv[1], argv[2] if len(argv) > 2 else None)
        for k, cs in res.items():
            print(f"- `{short(k)}`")
            for c, v in sorted(cs.items()):
                print(f"  - {c}: {v:.6g}")
        return 0
    if len(argv) >= 9 and argv[0] == "traffic":
        r = record_traffic(argv[1], argv[2], argv[3], argv[4], argv[5], argv[6], argv[7],
                           int(argv[8]), *(argv[9:10]))
        print(json.dumps(r))
        return 0
    if argv and argv[0] == "digest":
        print(source_digest())
        return 0
    print(__doc__)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
