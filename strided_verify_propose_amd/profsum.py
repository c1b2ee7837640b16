"""Summaries of rocprofv3 CSV output for profiles/.

  python -m strided_verify_propose_amd.profsum trace <kernel_stats.csv> <out.txt> "<command>"
  python -m strided_verify_propose_amd.profsum hbm <fetch counter_collection.csv>
      <write counter_collection.csv> <out.txt> "<fetch command>" "<write command>"

The HBM summary scales each kernel's FETCH_SIZE and WRITE_SIZE (KiB per dispatch) by
what the same counters read for a 1 GiB device-to-device copy in the same run, and
records the SHA-256 of the attention sources it was taken on (attention.hip, device.h and
the attention section of launch.h), so that a reader can tell when the counters no longer
describe the kernel.
"""
from __future__ import annotations

import csv
import hashlib
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
ATTN_SOURCES = ["csrc/attention.hip", "csrc/device.h", "csrc/launch.h"]
# in launch.h only the attention section (up to the next section rule) feeds the kernel
SECTION_OF = {"csrc/launch.h": "// ---------------------------------------------------------------- attention"}
SECTION_RULE = "// ----------------------------------------------------------------"
COPY_BYTES = 1 << 30


def attention_source_hash() -> str:
    """SHA-256 of the attention sources with comments and blank lines removed, so that a
    change of wording does not invalidate the counters but any change of code does."""
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            lines = fh.read().splitlines()
        if f in SECTION_OF:
            start = lines.index(SECTION_OF[f])
            end = next((i for i in range(start + 1, len(lines)) if lines[i].startswith(SECTION_RULE)),
                       len(lines))
            lines = lines[start:end]
        for line in lines:
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()


def short(name: str) -> str:
    name = name.replace("isd::(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    return name if len(name) < 90 else name[:87] + "..."


def trace(stats_csv, out, command):
    rows = list(csv.DictReader(open(stats_csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"# rocprofv3 kernel trace summary", f"command: {command}", "",
             f"{'kernel':90s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]
    for r in rows:
        lines.append(f"{short(r['Name']):90s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                     f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):6.2f}")
    open(out, "w").write("\n".join(lines) + "\n")


def per_kernel(counter_csv, counter):
    """{kernel name: [value per dispatch]} and the largest value of the runtime's
    buffer-copy kernel: the benchmark's 1 GiB calibration copy (a same-dtype device copy),
    far larger than the small copies around it.  Dtype conversions run other kernels."""
    vals = defaultdict(list)
    big_copy = 0.0
    for r in csv.DictReader(open(counter_csv)):
        if r["Counter_Name"] != counter:
            continue
        v = float(r["Counter_Value"])
        vals[r["Kernel_Name"]].append(v)
        if "copybuffer" in r["Kernel_Name"].lower():
            big_copy = max(big_copy, v)
    return vals, big_copy


def hbm(fetch_csv, write_csv, out, cmd_fetch, cmd_write):
    fv, cf = per_kernel(fetch_csv, "FETCH_SIZE")
    wv, cw = per_kernel(write_csv, "WRITE_SIZE")
    f_scale = COPY_BYTES / (cf * 1024.0)
    w_scale = COPY_BYTES / (cw * 1024.0)
    lines = ["# HBM traffic per dispatch from rocprofv3 counters", f"fetch command: {cmd_fetch}",
             f"write command: {cmd_write}", "",
             f"calibration: 1 GiB device copy reads FETCH_SIZE {cf:.0f} KiB -> fetch scale {f_scale:.4f}; "
             f"WRITE_SIZE {cw:.0f} KiB -> write scale {w_scale:.4f}", "",
             f"{'kernel':90s} {'n':>4s} {'FETCH_KiB':>12s} {'WRITE_KiB':>12s} {'traffic_MB':>11s}"]
    traffic = {}
    for k in sorted(set(fv) | set(wv)):
        if "isd::" not in k:
            continue
        f = sum(fv.get(k, [0])) / max(1, len(fv.get(k, [0])))
        w = sum(wv.get(k, [0])) / max(1, len(wv.get(k, [0])))
        t = f * 1024 * f_scale + w * 1024 * w_scale
        traffic[short(k)] = t
        lines.append(f"{short(k):90s} {len(fv.get(k, [])):4d} {f:12.1f} {w:12.1f} {t / 1e6:11.2f}")
    attn = [v for k, v in traffic.items() if k.startswith(("attn_bf16_kernel", "attn_combine_kernel"))]
    lines += ["", "isd_attention_step = attn_bf16_kernel + attn_combine_kernel (one launch each)",
              f"attention_source_sha256: {attention_source_hash()}"]
    if len(attn) == 2:
        lines.append(f"attention_step_traffic_bytes: {int(sum(attn))}")
    open(out, "w").write("\n".join(lines) + "\n")


def read_attention_traffic(path):
    """HBM bytes of one isd_attention_step (both kernels) from a summary, or None if the
    summary is absent or was taken on other attention sources."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("attention_source_sha256") != attention_source_hash():
        return None
    t = kv.get("attention_step_traffic_bytes")
    return int(t) if t else None


if __name__ == "__main__":
    if sys.argv[1] == "trace":
        trace(*sys.argv[2:5])
    elif sys.argv[1] == "hbm":
        hbm(*sys.argv[2:7])
    else:
        raise SystemExit(__doc__)
