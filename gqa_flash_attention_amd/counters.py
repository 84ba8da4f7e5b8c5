"""Turn two rocprofv3 counter passes over `bench.py` into per-launch hardware figures for
the bench's two kernels: shader clock, matrix-core utilisation, MFMA work against the
algorithmic FLOPs, LDS bank conflicts (prefill) and L2 hit rate (decode).

Usage (each pass a separate process; the command lines are also written into the summary):

    rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 \\
        SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_LDS SQ_LDS_BANK_CONFLICT \\
        --output-format csv -d <dir_sq> -o pmc -- \\
        python3 bench.py --steps 5 --warmup 3 --no-cpu-baseline --no-probes
    rocprofv3 --pmc GRBM_GUI_ACTIVE TCC_HIT_sum TCC_MISS_sum \\
        --output-format csv -d <dir_tcc> -o pmc -- \\
        python3 bench.py --steps 5 --warmup 3 --no-cpu-baseline --no-probes
    python -m gqa_flash_attention_amd.counters <dir_sq> <dir_tcc>

Definitions (the SQ counters are summed over every SIMD or shader engine of the device,
GRBM_GUI_ACTIVE over its XCDs, so one XCD's busy cycles are GRBM_GUI_ACTIVE / XCDs):
- clock = GRBM_GUI_ACTIVE / XCDs / dispatch duration;
- MFMA utilisation = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs x SIMDs), the
  fraction of SIMD cycles the matrix core is busy (rocprofv3's MfmaUtil);
- MFMA FLOPs = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (rocprofv3's MfmaFlopsBF16), against the
  causal half's 2*2*S*(S+1)/2*Hq*D: the excess is the diagonal tiles' masked part;
- MFMA/VALU co-execution and LDS bank conflicts as fractions of SIMD cycles and of LDS
  instruction cycles;
- L2 hit rate = TCC_HIT / (TCC_HIT + TCC_MISS).
XCD and SIMD counts come from the agent table the passes write. Dispatches are taken after
the bench's warm-up ones; figures are medians over the rest.
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

PASS_SQ = ("GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 "
           "SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_LDS SQ_LDS_BANK_CONFLICT")
PASS_TCC = "GRBM_GUI_ACTIVE TCC_HIT_sum TCC_MISS_sum"
BENCH_ARGS = "--steps 5 --warmup 3 --no-cpu-baseline --no-probes"


def _agent(d: str):
    paths = glob.glob(os.path.join(d, "**", "*agent_info.csv"), recursive=True)
    for p in paths:
        for r in csv.DictReader(open(p)):
            if r.get("Agent_Type") == "GPU":
                return int(r["Num_Xcc"]), int(r["Simd_Count"])
    raise SystemExit(f"no GPU agent in the agent table under {d}")


def _dispatches(d: str):
    """kernel name -> list (in dispatch order) of {counter: value, 'ns': duration}."""
    paths = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no counter_collection.csv under {d}")
    by = collections.OrderedDict()
    for p in paths:
        for r in csv.DictReader(open(p)):
            key = (r["Kernel_Name"], int(r["Dispatch_Id"]))
            e = by.setdefault(key, {"ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            # rows of one counter over several dimensions are summed
            e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    per = collections.defaultdict(list)
    for (name, _), e in sorted(by.items(), key=lambda kv: kv[0][1]):
        per[name].append(e)
    return per


def _pick(per, fragment: str, skip: int):
    names = [n for n in per if fragment in n]
    if len(names) != 1:
        raise SystemExit(f"expected one kernel matching {fragment!r}, found {names}")
    ds = per[names[0]]
    if len(ds) <= skip:
        raise SystemExit(f"{names[0]}: only {len(ds)} dispatches")
    return names[0], ds[skip:]


def summarize(dir_sq: str, dir_tcc: str, prefill_s: int, decode_l: int, warmup: int):
    sys.path.insert(0, ROOT)
    import bench  # noqa: E402  (same repository; only for the formulas and the source digest)
    xcc, simds = _agent(dir_sq)
    sq = _dispatches(dir_sq)
    tcc = _dispatches(dir_tcc)
    med = lambda ds, k: statistics.median(e[k] for e in ds)  # noqa: E731
    out = {"sources_digest": bench.kernel_sources_digest(), "xcds": xcc, "simds": simds, "kernels": {}}
    for frag, key in (("prefill_kernel", f"prefill_S{prefill_s}"), ("decode_kernel", f"decode_L{decode_l}")):
        name, ds = _pick(sq, frag, warmup)
        _, dt = _pick(tcc, frag, warmup)
        ns = med(ds, "ns")
        xcd_cycles = med(ds, "GRBM_GUI_ACTIVE") / xcc
        simd_cycles = xcd_cycles * simds
        e = {"kernel": name, "dispatches": len(ds), "duration_us": ns / 1e3,
             "clock_ghz": xcd_cycles / ns,
             "mfma_util": med(ds, "SQ_VALU_MFMA_BUSY_CYCLES") / simd_cycles,
             "mfma_valu_coexec": med(ds, "SQ_VALU_MFMA_COEXEC_CYCLES") / simd_cycles,
             "lds_bank_conflict_per_lds_cycle": (med(ds, "SQ_LDS_BANK_CONFLICT") / med(ds, "SQ_ACTIVE_INST_LDS")
                                                 if med(ds, "SQ_ACTIVE_INST_LDS") > 0 else 0.0),
             "mfma_flops": med(ds, "SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512.0,
             "l2_hit_rate": med(dt, "TCC_HIT_sum") / max(1.0, med(dt, "TCC_HIT_sum") + med(dt, "TCC_MISS_sum")),
             "tcc_pass_duration_us": med(dt, "ns") / 1e3}
        if key.startswith("prefill"):
            e["algorithmic_flops"] = bench.prefill_flops(prefill_s)
            e["mfma_flops_over_algorithmic"] = e["mfma_flops"] / e["algorithmic_flops"]
        out["kernels"][key] = e
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("dir_sq")
    ap.add_argument("dir_tcc")
    ap.add_argument("--prefill-s", type=int, default=32768)
    ap.add_argument("--decode-l", type=int, default=65536)
    ap.add_argument("--warmup", type=int, default=3, help="leading dispatches per kernel to skip")
    ap.add_argument("--out", default=None)
    a = ap.parse_args()
    res = summarize(a.dir_sq, a.dir_tcc, a.prefill_s, a.decode_l, a.warmup)
    out = a.out or os.path.join(ROOT, "profiles", f"counters_prefill_S{a.prefill_s}_decode_L{a.decode_l}.md")
    p = res["kernels"][f"prefill_S{a.prefill_s}"]
    d = res["kernels"][f"decode_L{a.decode_l}"]
    lines = [f"# Hardware counters per launch: causal prefill S={a.prefill_s} and decode L={a.decode_l} "
             "(B=1, 32q/8kv, d=128, bf16)", "",
             "Commands (repository root, library built in-tree; each pass its own process):", "", "```",
             "export TMPDIR=/tmp",
             f"rocprofv3 --pmc {PASS_SQ} --output-format csv -d <dir_sq> -o pmc -- python3 bench.py {BENCH_ARGS}",
             f"rocprofv3 --pmc {PASS_TCC} --output-format csv -d <dir_tcc> -o pmc -- python3 bench.py {BENCH_ARGS}",
             "python -m gqa_flash_attention_amd.counters <dir_sq> <dir_tcc>", "```", "",
             f"Device: {res['xcds']} XCDs, {res['simds']} SIMDs. Medians over the {p['dispatches']} prefill and "
             f"{d['dispatches']} decode dispatches after the warm-up ones (durations here are under counter "
             "collection).", "",
             "| kernel | duration | shader clock | MFMA utilisation | MFMA/VALU co-execution | LDS bank conflicts per LDS cycle | L2 hit rate |",
             "|---|---|---|---|---|---|---|"]
    for e in (p, d):
        # GRBM_GUI_ACTIVE also counts the dispatch's set-up and drain outside its timestamps,
        # which is noise for a multi-ms kernel but not for one of ~50 us
        clk = f"{e['clock_ghz']:.2f} GHz" if e["duration_us"] > 1000 else "n/a (short kernel)"
        lines.append(f"| `{e['kernel']}` | {e['duration_us']:.1f} us | {clk} | "
                     f"{100 * e['mfma_util']:.1f}% | {100 * e['mfma_valu_coexec']:.1f}% | "
                     f"{e['lds_bank_conflict_per_lds_cycle']:.3f} | {100 * e['l2_hit_rate']:.1f}% |")
    lines += ["",
              f"Prefill MFMA work: {p['mfma_flops']:.4e} FLOP counted by the matrix cores against "
              f"{p['algorithmic_flops']:.4e} algorithmic (ratio {p['mfma_flops_over_algorithmic']:.4f}; the excess "
              "is the masked part of the diagonal tiles, so no tile above the diagonal is computed).",
              "",
              f"Prefill at the spec peak: {p['mfma_util']:.3f} busy x {p['clock_ghz']:.2f} / 2.4 GHz = "
              f"{p['mfma_util'] * p['clock_ghz'] / 2.4:.3f} of 2.5 PFLOP/s, to compare with the achieved "
              f"{p['algorithmic_flops'] / (p['duration_us'] * 1e-6) / 2.5e15:.3f} from this pass's own duration.",
              "",
              "The shader clock is GRBM_GUI_ACTIVE per XCD over the dispatch's duration. That counter also "
              "runs during a dispatch's set-up and drain, outside its timestamps, so the ratio is only "
              "given for the multi-millisecond prefill.",
              "",
              f"Kernel sources digest: `{res['sources_digest']}`."]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
