"""Turn two rocprofv3 counter passes over `bench.py` into HBM bytes per kernel launch.

Usage (each pass a separate process; see the command lines written into the summary):

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir_fetch> -o pmc -- \\
        python3 bench.py --steps 5 --warmup 3 --no-cpu-baseline --no-probes --calib-copy-mb 1024
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir_write> -o pmc -- \\
        python3 bench.py --steps 5 --warmup 3 --no-cpu-baseline --no-probes --calib-copy-mb 1024
    python -m gqa_flash_attention_amd.traffic <dir_fetch> <dir_write> [--copy-mb 1024]

FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch. Each is scaled by the factor that
makes the same counter agree with the known size of the calibration copy (the largest
`copyBuffer` dispatch: it reads and writes exactly --copy-mb MiB). The result goes to
profiles/traffic.json (read by bench.py, which reports it only while the kernel sources
are unchanged) and to a short Markdown summary next to it.
"""

from __future__ import annotations

import argparse
import collections
import csv
import datetime
import glob
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _read(d: str, counter: str):
    paths = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = collections.defaultdict(list)
    copies = []
    for p in paths:
        for r in csv.DictReader(open(p)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            name = r["Kernel_Name"]
            per[name].append(v)
            if "copyBuffer" in name:
                copies.append((int(r["Grid_Size"]), v))
    if not copies:
        raise SystemExit(f"no calibration copy found in {d}")
    return per, max(copies)[1]


def summarize(dir_fetch: str, dir_write: str, copy_mb: int, prefill_s: int, decode_l: int):
    sys.path.insert(0, ROOT)
    import bench  # noqa: E402  (same repository; only for the source digest and the formulas)
    fetch, copy_fetch_kib = _read(dir_fetch, "FETCH_SIZE")
    write, copy_write_kib = _read(dir_write, "WRITE_SIZE")
    known = copy_mb * 1024 * 1024
    f_fetch = known / (copy_fetch_kib * 1024.0)
    f_write = known / (copy_write_kib * 1024.0)
    out = {"sources_digest": bench.kernel_sources_digest(),
           "taken": datetime.date.today().isoformat(),
           "calibration": {"copy_bytes": known, "fetch_kib": copy_fetch_kib, "write_kib": copy_write_kib,
                           "fetch_scale": f_fetch, "write_scale": f_write},
           "kernels": {}}
    keys = {"prefill_kernel": f"prefill_S{prefill_s}", "decode_kernel": f"decode_L{decode_l}"}
    for name in fetch:
        key = next((k for frag, k in keys.items() if frag in name), None)
        if key is None or name not in write:
            continue
        fb = sum(fetch[name]) / len(fetch[name]) * 1024.0 * f_fetch
        wb = sum(write[name]) / len(write[name]) * 1024.0 * f_write
        algo = bench.prefill_bytes(prefill_s) if key.startswith("prefill") else bench.decode_bytes(decode_l)
        out["kernels"][key] = {"kernel": name, "dispatches": len(fetch[name]),
                               "fetch_bytes": fb, "write_bytes": wb, "hbm_bytes_per_launch": fb + wb,
                               "algorithmic_bytes": algo, "ratio_to_algorithmic": (fb + wb) / algo}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("dir_fetch")
    ap.add_argument("dir_write")
    ap.add_argument("--copy-mb", type=int, default=1024)
    ap.add_argument("--prefill-s", type=int, default=32768)
    ap.add_argument("--decode-l", type=int, default=65536)
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles", "traffic.json"))
    a = ap.parse_args()
    res = summarize(a.dir_fetch, a.dir_write, a.copy_mb, a.prefill_s, a.decode_l)
    with open(a.out, "w") as f:
        json.dump(res, f, indent=1)
    md = os.path.splitext(a.out)[0] + f"_prefill_S{a.prefill_s}_decode_L{a.decode_l}.md"
    cal = res["calibration"]
    lines = [f"# HBM traffic per launch: causal prefill S={a.prefill_s} and decode L={a.decode_l} (B=1, 32q/8kv, d=128)", "",
             "Commands (repository root, library built in-tree):", "", "```",
             "export TMPDIR=/tmp",
             f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir_fetch> -o pmc -- python3 bench.py --steps 5 --warmup 3 --no-cpu-baseline --no-probes --calib-copy-mb {a.copy_mb}",
             f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir_write> -o pmc -- python3 bench.py --steps 5 --warmup 3 --no-cpu-baseline --no-probes --calib-copy-mb {a.copy_mb}",
             "python -m gqa_flash_attention_amd.traffic <dir_fetch> <dir_write>", "```", "",
             f"Calibration: a {a.copy_mb} MiB device copy read FETCH_SIZE = {cal['fetch_kib']:.0f} KiB and "
             f"WRITE_SIZE = {cal['write_kib']:.0f} KiB, so the scale factors are {cal['fetch_scale']:.3f} (fetch) "
             f"and {cal['write_scale']:.3f} (write).", "",
             "| kernel | dispatches | fetched MB | written MB | HBM MB per launch | algorithmic MB | ratio |",
             "|---|---|---|---|---|---|---|"]
    for k, e in res["kernels"].items():
        lines.append(f"| `{e['kernel']}` | {e['dispatches']} | {e['fetch_bytes'] / 1e6:.1f} | {e['write_bytes'] / 1e6:.1f} | "
                     f"{e['hbm_bytes_per_launch'] / 1e6:.1f} | {e['algorithmic_bytes'] / 1e6:.1f} | {e['ratio_to_algorithmic']:.2f} |")
    lines.append("")
    lines.append(f"Kernel sources digest: `{res['sources_digest']}` (bench.py reports the traffic only while it matches).")
    with open(md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(res, indent=1))


if __name__ == "__main__":
    main()
