"""Turn a rocprofv3 kernel-trace pass over `bench.py` and the bench's own JSON line (taken
in the same GPU session, without the profiler) into the kernel-time summary under profiles/.

Usage (repository root, library built in-tree):

    rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o bench -- \\
        python3 bench.py --steps 20 --warmup 10 --no-cpu-baseline
    python3 bench.py > bench.json
    python -m gqa_flash_attention_amd.kernel_stats <dir> bench.json

The summary lists each kernel's dispatch count and average / min / max duration from
`bench_kernel_stats.csv`, the rates those averages give for the prefill, the decode and the
two probes, and beside them the bench's HIP-event figures, which hold each launch's dispatch.

Per-size kernel times (every prefill and decode size of the workload):

    rocprofv3 --kernel-trace --output-format csv -d <dir> -o sizes -- \
        python3 bench.py --kernel-sizes sizes.jsonl
    python -m gqa_flash_attention_amd.kernel_stats --sizes <dir> sizes.jsonl

writes profiles/kernel_time_prefill_decode_sizes.md and profiles/kernel_time.json (with the
digest of the kernel sources, so bench.py reports these kernel times only while they match).
"""

from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def summarize(prof_dir: str, bench_json: str, out: str) -> str:
    sys.path.insert(0, ROOT)
    import bench  # noqa: E402  (same repository; only for the probe sizes)
    paths = glob.glob(os.path.join(prof_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no kernel_stats.csv under {prof_dir}")
    rows = list(csv.DictReader(open(paths[0])))
    b = json.load(open(bench_json))

    def avg(fragment):
        r = next((r for r in rows if fragment in r["Name"]), None)
        if r is None:
            raise SystemExit(f"no kernel matching {fragment!r} in {paths[0]}")
        return float(r["AverageNs"])

    pfa, dca = avg("prefill_kernel"), avg("decode_kernel")
    mfa, hba = avg("probe_mfma"), avg("probe_hbm")
    flops, dbytes = b["prefill"]["flops"], b["decode"]["bytes"]
    mflop = bench.probe_mfma_flops()
    S, L = b["config"]["prefill_S"], b["config"]["decode_L"]
    lines = [f"# Kernel-time summary: bench step (causal prefill S={S} + decode L={L}, B=1, 32q/8kv, d=128, "
             "bf16) and the two roofline probes", "",
             "Commands (repository root, library built in-tree beforehand with "
             "`python -m gqa_flash_attention_amd.build`):", "", "```", "export TMPDIR=/tmp",
             "rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o bench -- python3 bench.py "
             "--steps 20 --warmup 10 --no-cpu-baseline",
             "python3 bench.py > bench.json",
             "python -m gqa_flash_attention_amd.kernel_stats <dir> bench.json", "```", "",
             "30 dispatches per attention kernel = 10 warm-up + 20 timed steps; 4 per probe = 1 warm-up + 3 "
             "timed. Durations per dispatch (ns), from `bench_kernel_stats.csv`:", "",
             "| kernel | calls | average ns | min ns | max ns | share of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in rows[:5]:
        lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} | "
                     f"{float(r['Percentage']):.2f}% |")
    lines += ["",
              "From these averages: prefill %.0f TFLOP/s (%.3f of 2.5 PF); decode %.0f GB/s (%.3f of 8 TB/s); "
              "MFMA probe %.0f TFLOP/s for %.3e flop; HBM probe %.0f GB/s over %d MiB." % (
                  flops / pfa / 1e3, flops / pfa / 1e3 / 2500, dbytes / dca, dbytes / dca / 8000,
                  mflop / mfa / 1e3, mflop, bench.PROBE_HBM_BYTES / hba, bench.PROBE_HBM_BYTES >> 20),
              "",
              "HIP-event figures printed by `python3 bench.py` (default arguments) in the same GPU session, "
              "without the profiler:",
              "- prefill: %.0f us per launch (%.0f TFLOP/s) vs rocprofv3 average %.0f us;" % (
                  b["prefill"]["ms"] * 1e3, b["value"], pfa / 1e3),
              "- decode (one fused launch): %.1f us per launch (%.0f GB/s) vs rocprofv3 average %.1f us. The event "
              "pair around each launch also holds its dispatch (~2-4 us);" % (
                  b["decode"]["ms"] * 1e3, b["decode"]["value"], dca / 1e3)]
    mp = b["roofline"].get("measured_peak")
    hp = b["roofline_decode"].get("measured_peak")
    if mp:
        lines.append("- MFMA probe: %.0f TFLOP/s at a measured %.2f GHz shader clock;" % (mp["value"], mp["clock_ghz"]))
    if hp:
        lines.append("- HBM read probe: %.0f GB/s over %d MiB." % (hp["value"], bench.PROBE_HBM_BYTES >> 20))
    lines += ["",
              "Boards differ by several percent: the shader clock under load is set by the power cap (the MFMA "
              "probe has measured 1.70-1.84 GHz on different boxes)."]
    text = "\n".join(lines) + "\n"
    with open(out, "w") as f:
        f.write(text)
    return text


SIZES_CMD = ("rocprofv3 --kernel-trace --output-format csv -d <dir> -o sizes -- "
             "python3 bench.py --kernel-sizes sizes.jsonl")


def _trace_dispatches(prof_dir: str):
    """[(kind, duration_ns)] of the attention kernels in dispatch order: kind 'prefill' for
    every prefill form, 'decode' for the fused and split decode kernels."""
    paths = glob.glob(os.path.join(prof_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no kernel_trace.csv under {prof_dir}")
    out = []
    for r in csv.DictReader(open(paths[0])):
        name = r["Kernel_Name"]
        if "prefill_kernel" in name or "prefill_split_kernel" in name:
            kind = "prefill"
        elif "decode_kernel" in name:
            kind = "decode"
        else:
            continue
        out.append((int(r["Start_Timestamp"]), kind, int(r["End_Timestamp"]) - int(r["Start_Timestamp"]), name))
    out.sort()
    return [(k, d, n) for _, k, d, n in out]


def _pct(xs, p):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, int(p * (len(xs) - 1)))]


def summarize_sizes(prof_dir: str, sizes_jsonl: str, out_md: str, out_json: str) -> str:
    """Per-size kernel time from a trace of `bench.py --kernel-sizes`: the dispatches of each
    kind are taken in order, each size consuming its settling calls and then its timed calls
    (the counts its JSON line records); statistics over the timed ones."""
    sys.path.insert(0, ROOT)
    import bench  # noqa: E402  (same repository: peaks, digest)
    disp = _trace_dispatches(prof_dir)
    rows = [json.loads(ln) for ln in open(sizes_jsonl) if ln.strip()]
    pos = {"prefill": 0, "decode": 0}
    by_kind = {k: [d for d in disp if d[0] == k] for k in pos}
    res = {}
    for r in rows:
        kind = r["mode"]
        n0, n1 = r["settle_calls"], r["timed_calls"]
        seq = by_kind[kind][pos[kind]: pos[kind] + n0 + n1]
        if len(seq) != n0 + n1:
            raise SystemExit(f"trace holds {len(seq)} {kind} dispatches for {r}, expected {n0 + n1}")
        pos[kind] += n0 + n1
        ns = [d for _, d, _ in seq[n0:]]
        names = sorted({n for _, _, n in seq[n0:]})
        med = statistics.median(ns)
        e = {"kernel": names, "calls": n1, "kernel_us_median": med / 1e3, "kernel_us_mean": sum(ns) / len(ns) / 1e3,
             "kernel_us_p05": _pct(ns, 0.05) / 1e3, "kernel_us_p95": _pct(ns, 0.95) / 1e3,
             "kernel_us_min": min(ns) / 1e3, "event_us_median": r["event_ms_median"] * 1e3,
             "event_us_p05": r["event_ms_p05"] * 1e3, "event_us_p95": r["event_ms_p95"] * 1e3}
        if kind == "prefill":
            key = f"prefill_S{r['S']}"
            e["tflops_kernel"] = r["flops"] / (med * 1e-9) / 1e12
            e["frac_kernel"] = e["tflops_kernel"] / bench.PEAK_BF16_TFLOPS
            e["tflops_event"] = r["flops"] / (r["event_ms_median"] * 1e-3) / 1e12
        else:
            # batch-1 decodes by length; batched and ragged ones also by batch
            key = f"decode_L{r['L']}" if r.get("B", 1) == 1 else (
                f"decode_B{r['B']}_L{r['L']}" + ("_ragged" if r.get("ragged") else ""))
            e["gbs_kernel"] = r["bytes"] / (med * 1e-9) / 1e9
            e["frac_kernel"] = e["gbs_kernel"] / bench.PEAK_HBM_GBS
            e["gbs_event"] = r["bytes"] / (r["event_ms_median"] * 1e-3) / 1e9
        res[key] = e
    for k in pos:
        if pos[k] != len(by_kind[k]):
            raise SystemExit(f"{len(by_kind[k]) - pos[k]} {k} dispatches in the trace are not accounted for")
    doc = {"sources_digest": bench.kernel_sources_digest(), "command": SIZES_CMD, "sizes": res}
    with open(out_json, "w") as f:
        json.dump(doc, f, indent=1)
    lines = ["# Kernel time per workload size: causal prefill and decode, B = 1 (and batched decodes), 32 query / 8 KV "
             "heads, d = 128, bf16",
             "", "Commands (repository root, library built in-tree beforehand with "
             "`python -m gqa_flash_attention_amd.build`):", "", "```", "export TMPDIR=/tmp", SIZES_CMD,
             "python -m gqa_flash_attention_amd.kernel_stats --sizes <dir> sizes.jsonl", "```", "",
             f"Kernel sources digest `{doc['sources_digest']}`. Per size: ~0.2 s of settling calls, then the timed "
             "calls; kernel time is each dispatch's own duration in the trace, the event span is the bench's HIP "
             "events around each call (it also holds the dispatch). Decode caches rotate over >= 1 GB of copies, "
             "so each decode reads from HBM. decode_B<B>_L<L> rows are batched decodes with every sequence at the "
             "full length; the _ragged row has lengths U[1, L] (bytes counted over the actual lengths). Fractions "
             "are of 2.5 PFLOP/s (bf16 dense) and 8 TB/s.", "",
             "| size | kernel | calls | kernel us median (p05-p95) | event us median | rate by kernel time | "
             "fraction of peak |", "|---|---|---|---|---|---|---|"]
    for key, e in res.items():
        rate = (f"{e['tflops_kernel']:.0f} TFLOP/s" if key.startswith("prefill")
                else f"{e['gbs_kernel']:.0f} GB/s")
        kn = ", ".join(f"`{n}`" for n in e["kernel"])
        lines.append(f"| {key} | {kn} | {e['calls']} | {e['kernel_us_median']:.2f} ({e['kernel_us_p05']:.2f}-"
                     f"{e['kernel_us_p95']:.2f}) | {e['event_us_median']:.2f} | {rate} | {e['frac_kernel']:.3f} |")
    text = "\n".join(lines) + "\n"
    with open(out_md, "w") as f:
        f.write(text)
    return text


FLOOR_CMD = ("rocprofv3 --kernel-trace --output-format csv -d <dir> -o floor -- "
             "python3 bench.py --read-floor floor.jsonl")


def summarize_read_floor(prof_dir: str, floor_jsonl: str, out_md: str, decode_json: str | None) -> str:
    """Kernel time of each read-floor point (bench.py --read-floor), matched in dispatch order,
    beside the decode's own kernel time at the same L (profiles/kernel_time.json) when given."""
    paths = glob.glob(os.path.join(prof_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no kernel_trace.csv under {prof_dir}")
    disp = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                  for r in csv.DictReader(open(paths[0])) if "probe_hbm_read" in r["Kernel_Name"])
    rows = [json.loads(ln) for ln in open(floor_jsonl) if ln.strip()]
    dec = {}
    if decode_json and os.path.exists(decode_json):
        dec = json.load(open(decode_json)).get("sizes", {})
    pos = 0
    lines = ["# Cold pure-read floor at the decode sizes (batch 1, K + V of 8 KV heads x 128 bf16)", "",
             "Commands (repository root, library built in-tree beforehand):", "", "```", "export TMPDIR=/tmp",
             FLOOR_CMD, "python -m gqa_flash_attention_amd.kernel_stats --read-floor <dir> floor.jsonl", "```", "",
             "The library's HBM read probe (`gqa_attn_probe_hbm_read`: 16-byte non-temporal loads, the workgroups "
             "of each XCD reading one 256-byte slice of every 2 KB row, as the decode does) reads exactly the "
             "bytes of a batch-1 decode's K and V cache (4096 L), from one of >= 1 GB of buffers in rotation so "
             "the MALL holds none. It does no arithmetic and no merge: a decode of the same cache cannot finish "
             "in less kernel time than the best point. Decode kernel times are from "
             "`profiles/kernel_time.json` (same kernel-trace method, a run on another box).", "",
             "| L | bytes | workgroups | read kernel us (median) | GB/s | fraction of 8 TB/s | decode kernel us | "
             "decode / best read |", "|---|---|---|---|---|---|---|---|"]
    best = {}
    table = []
    for r in rows:
        n0, n1 = r["settle_calls"], r["timed_calls"]
        seq = disp[pos: pos + n0 + n1]
        if len(seq) != n0 + n1:
            raise SystemExit(f"trace holds {len(seq)} probe dispatches for {r}, expected {n0 + n1}")
        pos += n0 + n1
        med = statistics.median(d for _, d in seq[n0:]) / 1e3
        best[r["L"]] = min(best.get(r["L"], 1e30), med)
        table.append((r, med))
    for r, med in table:
        d = dec.get(f"decode_L{r['L']}")
        dk = f"{d['kernel_us_median']:.2f}" if d else "-"
        ratio = f"{d['kernel_us_median'] / best[r['L']]:.2f}" if d else "-"
        lines.append(f"| {r['L']} | {r['bytes']} | {r['workgroups']} | {med:.2f} | {r['bytes'] / med / 1e3:.0f} | "
                     f"{r['bytes'] / med / 1e3 / 8000:.3f} | {dk} | {ratio} |")
    text = "\n".join(lines) + "\n"
    with open(out_md, "w") as f:
        f.write(text)
    return text


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("prof_dir")
    ap.add_argument("bench_json", help="the bench's JSON line, or with --sizes the --kernel-sizes JSONL")
    ap.add_argument("--sizes", action="store_true",
                    help="summarize a trace of `bench.py --kernel-sizes` into per-size kernel times")
    ap.add_argument("--read-floor", action="store_true",
                    help="summarize a trace of `bench.py --read-floor` (the cold pure-read floor)")
    ap.add_argument("--out", default=None)
    ap.add_argument("--out-json", default=os.path.join(ROOT, "profiles", "kernel_time.json"))
    a = ap.parse_args()
    if a.read_floor:
        out = a.out or os.path.join(ROOT, "profiles", "hbm_read_floor_decode_sizes.md")
        print(summarize_read_floor(a.prof_dir, a.bench_json, out, os.path.join(ROOT, "profiles", "kernel_time.json")))
    elif a.sizes:
        out = a.out or os.path.join(ROOT, "profiles", "kernel_time_prefill_decode_sizes.md")
        print(summarize_sizes(a.prof_dir, a.bench_json, out, a.out_json))
    else:
        out = a.out or os.path.join(ROOT, "profiles", "bench_prefill_S32768_decode_L65536_kernel_stats.md")
        print(summarize(a.prof_dir, a.bench_json, out))


if __name__ == "__main__":
    main()
