"""Summaries of rocprofv3 CSV output for profiles/.

  python -m strided_verify_propose_amd.profsum trace <kernel_stats.csv> <out.txt> "<command>"
  python -m strided_verify_propose_amd.profsum hbm <fetch counter_collection.csv>
      <write counter_collection.csv> <out.txt> "<fetch command>" "<write command>"
  python -m strided_verify_propose_amd.profsum mfma <counter_collection.csv> <out.txt> "<command>"
  python -m strided_verify_propose_amd.profsum sweep <sweep.jsonl> <out.txt> "<command>"
  python -m strided_verify_propose_amd.profsum stalls <out.txt> <counter_collection.csv> "<command>"
      [<counter_collection.csv> "<command>" ...]

The HBM summary scales each kernel's FETCH_SIZE and WRITE_SIZE (KiB per dispatch) by
what the same counters read for a 1 GiB device-to-device copy in the same run, and
records the SHA-256 of the attention sources it was taken on (attention.hip, device.h and
the attention section of launch_types.h), so that a reader can tell when the counters no longer
describe the kernel.
"""
from __future__ import annotations

import csv
import hashlib
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
ATTN_SOURCES = ["csrc/attention.hip", "csrc/device.h", "csrc/launch_types.h"]
# in launch_types.h only the attention section (up to the next section rule) feeds the kernel
SECTION_OF = {"csrc/launch_types.h": "// ---------------------------------------------------------------- attention"}
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


PROJ_SOURCES = ["csrc/gemm.hip", "csrc/gemm_packed.hip", "csrc/gemm_big.hip", "csrc/device.h", "csrc/tiles.h"]


def source_hash(files) -> str:
    """SHA-256 of source files with comments and blank lines removed."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            for line in fh.read().splitlines():
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


SIMDS = 1024       # 256 CUs x 4 SIMDs
CLOCK_GHZ = 2.4


def mfma(counter_csv, out, command):
    """MFMA activity per kernel: bf16 MFMA flops (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) and
    the MFMA pipes' busy cycles (SQ_VALU_MFMA_BUSY_CYCLES, summed over the 1024 SIMDs),
    against the dispatch's own duration in the same run (its start and end timestamps):
    busy share = busy cycles / (1024 x duration x 2.4 GHz), rate = flops / duration
    against the 2.5 PFLOP/s bf16 peak."""
    vals = defaultdict(lambda: defaultdict(list))
    dur = defaultdict(dict)
    for r in csv.DictReader(open(counter_csv)):
        vals[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
        dur[r["Kernel_Name"]][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
    lines = ["# MFMA counters per dispatch (rocprofv3 --pmc), mean over dispatches", f"command: {command}", "",
             f"{'kernel':60s} {'n':>3s} {'GFLOP':>9s} {'dur_us':>8s} {'mfma_busy':>10s} {'PFLOP/s':>8s} {'frac':>6s}"]
    for k, c in vals.items():
        if "isd::" not in k:
            continue
        mean = {n: sum(v) / len(v) for n, v in c.items()}
        flops = mean.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        us = sum(dur[k].values()) / len(dur[k])
        busy = mean.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (SIMDS * us * CLOCK_GHZ * 1e3) if us else 0.0
        rate = flops / (us * 1e-6) / 1e15 if us else 0.0
        lines.append(f"{short(k)[:60]:60s} {len(dur[k]):3d} {flops / 1e9:9.3f} {us:8.2f} {100 * busy:9.1f}% "
                     f"{rate:8.3f} {rate / 2.5:6.3f}")
    lines += ["", "dur_us: the dispatch's end - start timestamps under the profiler (dispatches serialised);",
              "mfma_busy: SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x dur x 2.4 GHz); frac: PFLOP/s / 2.5.",
              f"projection_source_sha256: {source_hash(PROJ_SOURCES)}"]
    open(out, "w").write("\n".join(lines) + "\n")


def read_mfma(path, kernel_prefixes):
    """{kernel: {"gflop", "dur_us", "mfma_busy", "frac"}} for the kernels named, from an
    MFMA summary taken on the current projection sources, else None."""
    if not os.path.exists(path):
        return None
    text = open(path).read().splitlines()
    kv = dict(l.split(":", 1) for l in text if l.startswith("projection_source_sha256:"))
    if kv.get("projection_source_sha256", "").strip() != source_hash(PROJ_SOURCES):
        return None
    res = {}
    for line in text:
        for k in kernel_prefixes:
            if line.startswith(k):
                f = line[60:].split()
                res[k] = {"gflop": float(f[1]), "dur_us": float(f[2]), "mfma_busy": float(f[3].rstrip("%")) / 100,
                          "frac": float(f[5])}
    return res or None


def sweep(jsonl, out, command):
    """The concurrency sweep's JSON lines as a table."""
    import json
    rows = [json.loads(l) for l in open(jsonl) if l.startswith("{")]
    lines = ["# Concurrency sweep: whole ISD step (projection, attention, verification) per C and N",
             f"command: {command}", "",
             f"{'p':>4s} {'N':>2s} {'C':>4s} {'ms/step':>8s} {'steps/s':>8s} {'tokens/s':>9s} {'p_hat':>6s} "
             f"{'TPF':>6s} {'proj_us':>8s} {'attn_us':>8s} {'ver_us':>8s} {'attn%HBM':>8s} {'ver%HBM':>8s} "
             f"{'proj%MFMA':>9s}"]
    for r in rows:
        u = r["us"]
        lines.append(f"{r.get('acceptance_target', 0.9):4.1f} {r['stride_N']:2d} {r['C']:4d} {r['ms_per_step']:8.4f} "
                     f"{r['steps_per_s']:8.1f} {r['tokens_per_s']:9.0f} {r['p_hat']:6.3f} "
                     f"{r['tpf_closed_form_at_p_hat']:6.3f} {u['gated_lora_proj']:8.2f} {u['attention']:8.2f} "
                     f"{u['verify']:8.2f} {100 * r['attention_hbm_frac']:8.1f} {100 * r['verify_hbm_frac']:8.1f} "
                     f"{100 * r['proj_mfma_frac']:9.1f}")
    if rows:
        lines += ["", f"proposal noise sd: " + ", ".join(
            sorted({f"{r.get('acceptance_target')}: {r.get('proposal_noise_sd')}" for r in rows}))]
    open(out, "w").write("\n".join(lines) + "\n")


STALL_SHARES = [  # (label, counter, denominator): wave-cycle shares and per-unit busy shares
    ("waiting (any)", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES"),
    ("waiting to issue", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
    ("issuing", "SQ_ACTIVE_INST_ANY", "SQ_WAVE_CYCLES"),
    ("waiting to issue LDS", "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES"),
]


def stalls(out, *pairs):
    """Per-kernel means of every counter in one or more rocprofv3 --pmc passes (one CSV
    and its command per pass), as a table with one column per kernel, headed by the
    wave-cycle shares above, the MFMA pipes' busy share (as in the MFMA summary) and the
    share of time the CUs' L1 caches wait on data pending from L2
    (TCP_PENDING_STALL_CYCLES over 256 CUs)."""
    vals = defaultdict(lambda: defaultdict(list))
    dur = defaultdict(dict)
    cmds = []
    for path, cmd in zip(pairs[0::2], pairs[1::2]):
        cmds.append(cmd)
        for r in csv.DictReader(open(path)):
            if "isd::" not in r["Kernel_Name"]:
                continue
            vals[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
            dur[r["Kernel_Name"]][(path, r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
    kernels = sorted(vals, key=lambda n: -sum(dur[n].values()) / len(dur[n]))
    mean = {k: {n: sum(v) / len(v) for n, v in vals[k].items()} for k in kernels}
    us = {k: sum(dur[k].values()) / len(dur[k]) for k in kernels}
    names = [short(k).split("(")[0].split("<")[0][:16] for k in kernels]
    lines = ["# Wait and activity counters per dispatch (rocprofv3 --pmc), mean over dispatches"]
    lines += [f"pass {i + 1} command: {c}" for i, c in enumerate(cmds)]
    lines += ["", "kernels: " + "; ".join(f"{n} = {short(k)}" for n, k in zip(names, kernels)), "",
              f"{'':34s}" + "".join(f"{n:>17s}" for n in names),
              f"{'duration under the profiler, us':34s}" + "".join(f"{us[k]:17.2f}" for k in kernels)]

    def row(label, f):
        cells = []
        for k in kernels:
            v = f(mean[k], us[k])
            cells.append(f"{v:17.1f}" if v is not None else f"{'-':>17s}")
        lines.append(f"{label:34s}" + "".join(cells))

    for label, num, den in STALL_SHARES:
        row(f"% wave cycles {label}", lambda m, t, a=num, b=den: 100 * m[a] / m[b] if a in m and m.get(b) else None)
    row("% MFMA pipes busy", lambda m, t: 100 * m["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * t * CLOCK_GHZ * 1e3)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m and t else None)
    row("% L1 stalled on pending L2 data", lambda m, t: 100 * m["TCP_PENDING_STALL_CYCLES"] / (256 * t * CLOCK_GHZ * 1e3)
        if "TCP_PENDING_STALL_CYCLES" in m and t else None)
    lines.append("")
    for n in sorted({c for k in kernels for c in mean[k]}):
        lines.append(f"{n:34s}" + "".join(f"{mean[k][n]:17.6g}" if n in mean[k] else f"{'-':>17s}" for k in kernels))
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
    elif sys.argv[1] == "mfma":
        mfma(*sys.argv[2:5])
    elif sys.argv[1] == "sweep":
        sweep(*sys.argv[2:5])
    elif sys.argv[1] == "stalls":
        stalls(*sys.argv[2:])
    else:
        raise SystemExit(__doc__)
