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
"""

from __future__ import annotations

import argparse
import csv
import glob
import json
import os
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("prof_dir")
    ap.add_argument("bench_json")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles",
                                                  "bench_prefill_S32768_decode_L65536_kernel_stats.md"))
    a = ap.parse_args()
    print(summarize(a.prof_dir, a.bench_json, a.out))


if __name__ == "__main__":
    main()
