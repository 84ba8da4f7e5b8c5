#!/usr/bin/env python3
"""Throughput of the GQA attention forward hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
a causal prefill (B=1, S=32768, 32 query heads / 8 KV heads, d=128, bf16),
then a one-token decode against a KV cache of L=65536 (same heads) -- the
largest prefill and decode sizes of the workload (chowfi/kernels README,
"Result" table: prefill 2K..32K, decode 2K..64K).

Printed (rank 0, one JSON line): the contract fields, with
- value      : causal prefill TFLOP/s (FLOPs = 2*2*S*(S+1)/2*Hq*D, the causal half);
- decode     : decode KV-read GB/s (bytes = K+V read once = 2*L*Hkv*D*2, plus q and out);
- roofline   : the prefill kernel against the bf16 dense MFMA peak (it is most of the step);
- roofline_decode : the decode kernel against the HBM peak;
  both also carry measured_peak / frac_of_measured: the same kernel against the rate
  the library's own probes reach on this board (cold 16-byte HBM reads; register-resident
  bf16 MFMA with random operands, with the clock it ran at), taken after the timed steps;
- cpu_baseline: the fp64 CPU oracle on a bounded sample of the same prefill;
  cpu_baseline_decode: the same oracle on the whole decode.
Kernel durations come from HIP events recorded on the stream the kernels run on,
inside the timed region. The prefill streams ~671 MB between decodes, which flushes
the 256 MB MALL, so every decode reads its cache from HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-probes]
    python bench.py --sweep out.jsonl     # every prefill/decode size, one JSON line each
    python bench.py --sweep-chunks out.jsonl   # decode split sizes, paired timing
    python bench.py --sweep-forms out.jsonl    # prefill workgroup forms, paired timing
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HQ, HKV, D = 32, 8, 128
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
METRIC = "causal prefill TFLOP/s + decode KV-read GB/s (GQA 32q/8kv d128 bf16, 1 GPU)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def prefill_flops(S: int, B: int = 1) -> float:
    return 2.0 * 2.0 * S * (S + 1) / 2.0 * HQ * D * B


def prefill_bytes(S: int, B: int = 1) -> float:
    """q, k, v read once and out written once."""
    return float(S * B * (HQ + HKV + HKV + HQ) * D * 2)


def decode_bytes(L_total: int, B: int = 1) -> float:
    """K+V read once per KV head for L_total cached tokens, plus q and out."""
    return 2.0 * L_total * HKV * D * 2 + 2.0 * B * HQ * D * 2


def kernel_sources_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gqa_flash_attention_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key: str):
    """HBM bytes per launch measured with rocprofv3 counters, if taken on the current sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("sources_digest") != kernel_sources_digest():
        return None
    entry = t.get("kernels", {}).get(kernel_key)
    return None if entry is None else entry.get("hbm_bytes_per_launch")


KERNEL_TIME_FILE = os.path.join(ROOT, "profiles", "kernel_time.json")


def load_kernel_time(key: str):
    """Per-size kernel time (rocprofv3 trace of `--kernel-sizes`) if taken on the current sources."""
    try:
        with open(KERNEL_TIME_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("sources_digest") != kernel_sources_digest():
        return None
    return t.get("sizes", {}).get(key)


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def make_inputs(S: int, L: int, dev):
    import torch
    from gqa_inputs import decode_inputs, prefill_inputs, seed_base
    q, k, v = prefill_inputs(1, S, base=seed_base(2, 4))
    qd, kc, vc, lens = decode_inputs(1, L, base=seed_base(1, 5))
    t = [x.to(dev) for x in (q, k, v, qd, kc, vc, lens)]
    torch.cuda.synchronize()
    return t


def cpu_baseline(S: int, budget_s: float = 15.0):
    """Time the fp64 oracle on contiguous 256-row blocks of the S-token causal prefill,
    spread evenly over the sequence, until about budget_s seconds have been spent."""
    import numpy as np
    import oracle
    from gqa_inputs import bf16_bits, prefill_inputs, seed_base
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    q, k, v = prefill_inputs(1, S, base=seed_base(2, 4))
    qb, kb, vb = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    blocks = 256
    order = []
    nblk = S // blocks
    # visit blocks in a stride order that covers early, late and middle positions evenly
    step = max(1, nblk // 16)
    for off in range(step):
        order.extend(range(off, nblk, step))
    flops = 0.0
    rows_done = 0
    spent = 0.0
    for bi in order:
        r0 = bi * blocks
        rows = np.arange(r0, r0 + blocks)
        t0 = time.perf_counter()
        oracle.prefill(qb, kb, vb, causal=True, rows=rows)
        spent += time.perf_counter() - t0
        flops += float(np.sum(4.0 * (rows + 1) * D * HQ))
        rows_done += blocks
        if spent >= budget_s:
            break
    return {
        "value": flops / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle, causal prefill S={S} B=1 Hq={HQ} Hkv={HKV} D={D}: "
                   f"{rows_done} query rows (all heads) in 256-row blocks spread over the sequence, "
                   f"{flops / 1e9:.1f} GFLOP algorithmic in {spent:.1f} s"),
    }


def cpu_baseline_decode(L: int, budget_s: float = 4.0):
    """Time the fp64 oracle on the whole batch-1 decode against an L-token cache, repeated
    until about budget_s seconds have been spent; reported as algorithmic GB/s, with the
    same measure on one BLAS thread beside it."""
    import oracle
    from gqa_inputs import bf16_bits, decode_inputs, seed_base
    qd, kc, vc, lens = decode_inputs(1, L, base=seed_base(1, 5))
    qb, kb, vb = bf16_bits(qd), bf16_bits(kc), bf16_bits(vc)
    ln = lens.numpy()

    def timed(budget):
        calls, spent = 0, 0.0
        while spent < budget or calls == 0:
            t0 = time.perf_counter()
            oracle.decode(qb, kb, vb, ln)
            spent += time.perf_counter() - t0
            calls += 1
        return calls, spent

    calls, spent = timed(budget_s)
    r = {
        "value": decode_bytes(L) * calls / spent / 1e9,
        "unit": "GB/s",
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle, whole decode B=1 L={L} Hq={HQ} Hkv={HKV} D={D}: "
                   f"{calls} calls in {spent:.1f} s"),
    }
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            c1, s1 = timed(budget_s / 2)
        r["one_thread"] = {"value": decode_bytes(L) * c1 / s1 / 1e9, "unit": "GB/s", "cores": 1,
                           "sample": f"same decode on one BLAS thread: {c1} calls in {s1:.1f} s"}
    except Exception as e:  # threadpoolctl missing or unable to limit this BLAS
        r["one_thread"] = {"value": None, "reason": f"BLAS threads not limitable here: {e}"}
    return r


def run_step_timing(S, L, steps, warmup):
    import torch
    import gqa_flash_attention_amd as gqa
    dev = torch.device("cuda:0")
    q, k, v, qd, kc, vc, lens = make_inputs(S, L, dev)
    out_p = torch.empty_like(q)
    out_d = torch.empty_like(qd)
    stream = torch.cuda.current_stream(dev)

    def step():
        gqa.prefill(q, k, v, causal=True, out=out_p)
        gqa.decode(qd, kc, vc, lens, out=out_d)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        gqa.prefill(q, k, v, causal=True, out=out_p)
        ev[i][1].record(stream)
        gqa.decode(qd, kc, vc, lens, out=out_d)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pf = sorted(ev[i][0].elapsed_time(ev[i][1]) for i in range(steps))
    dc = sorted(ev[i][1].elapsed_time(ev[i][2]) for i in range(steps))
    return wall, pf, dc


SWEEP_CHUNK_L = (2048, 4096, 8192, 16384, 32768, 65536)


def chunk_candidates(L: int):
    """Split sizes the decode chunk sweep visits at cache length L (B = 1): the library's
    own choice plus every power of two times 64 from 128 to 16384. Returns (default,
    runnable, not_run) where not_run lists (chunk, reason) for points that are not timed."""
    import gqa_flash_attention_amd as gqa
    default, _ = gqa.decode_plan(1, L, 32, 8, 128)
    pts = sorted({default} | {64 * 2 ** i for i in range(1, 9)})
    run, skip = [], []
    for c in pts:
        if c > L:
            skip.append((c, "longer than the cache: the single split that chunk = L already gives"))
        else:
            run.append(c)
    return default, run, skip


def sweep_chunks(path: str, rounds: int = 8):
    """Decode split-size sweep at B = 1 (SWEEP_CHUNK_L): every runnable point of
    chunk_candidates() timed in paired rounds (the points alternate in rotated order,
    caches rotated over >= 1 GB so the MALL holds none), median time per point and the
    median of per-round ratios against the library's default chunk. Parity of every
    point against the oracle is checked by tests/test_sweep_points_gpu.py on the same
    seeded inputs and points."""
    import statistics
    import torch
    import gqa_flash_attention_amd as gqa
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    with open(path, "w") as f:
        for L in SWEEP_CHUNK_L:
            default, run, skip = chunk_candidates(L)
            _, qd, kc, vc, lens = [None] + make_inputs(64, L, dev)[3:]
            per = 2 * L * 8 * 128 * 2
            nc = max(4, min(64, -(-(1 << 30) // per)))
            kcs = [kc.clone() for _ in range(nc)]
            vcs = [vc.clone() for _ in range(nc)]
            out = torch.empty_like(qd)
            wss = {c: gqa.decode_workspace(1, L, 32, 8, 128, c, device=dev)
                   for c in run}
            call = lambda c, i: gqa.decode(qd, kcs[i % nc], vcs[i % nc], lens, out=out, chunk=c, workspace=wss[c])
            for c in run:
                for i in range(2 * nc):
                    call(c, i)
            torch.cuda.synchronize()
            times = {c: [] for c in run}
            for r in range(rounds):
                order = run[r % len(run):] + run[:r % len(run)]
                for c in order:
                    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nc)]
                    for i in range(nc):
                        ev[i][0].record(st)
                        call(c, i)
                        ev[i][1].record(st)
                    torch.cuda.synchronize()
                    times[c].append(statistics.median(a.elapsed_time(b) for a, b in ev))
            for c in run:
                t = statistics.median(times[c])
                ratio = statistics.median(times[default][i] / times[c][i] for i in range(rounds))
                row = {"mode": "decode_chunk", "L": L, "chunk": c, "nsplit": -(-L // c), "default": c == default,
                       "status": "run", "us_median": round(t * 1e3, 2), "GBs": round(decode_bytes(L) / (t * 1e-3) / 1e9),
                       "speed_vs_default": round(ratio, 3)}
                print(json.dumps(row), flush=True)
                f.write(json.dumps(row) + "\n")
            for c, why in skip:
                row = {"mode": "decode_chunk", "L": L, "chunk": c, "status": "not_run", "reason": why}
                print(json.dumps(row), flush=True)
                f.write(json.dumps(row) + "\n")
            del kcs, vcs, wss
            torch.cuda.empty_cache()


SWEEP_FORM_S = (512, 1024, 2048, 3072, 4096, 8192, 16384, 32768)


def sweep_forms(path: str, rounds: int = 8):
    """Prefill workgroup-form sweep at B = 1 (SWEEP_FORM_S, causal): every form of
    gqa.PREFILL_FORMS timed in paired rounds (the forms alternate in rotated order, ~0.2 s
    of calls per form first so the clock settles), median time per form and the median of
    per-round ratios against the form the library picks. Parity of every point against
    the oracle is checked by tests/test_sweep_points_gpu.py on the same seeded inputs."""
    import statistics
    import torch
    import gqa_flash_attention_amd as gqa
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    forms = list(gqa.PREFILL_FORMS)
    with open(path, "w") as f:
        for S in SWEEP_FORM_S:
            q, k, v = make_inputs(S, 64, dev)[:3]
            waves, _, ks = gqa.prefill_plan(1, S, 32, 8)
            chosen = (waves, ks)
            out = torch.empty_like(q)
            per = prefill_flops(S) / 1.0e15            # seconds per call at ~1 PFLOP/s
            reps = max(2, min(400, int(0.05 / per)))
            for fm in forms:
                for _ in range(max(3, min(4000, int(0.2 / per)))):
                    gqa.prefill(q, k, v, out=out, form=fm)
            torch.cuda.synchronize()
            times = {fm: [] for fm in forms}
            for r in range(rounds):
                for fm in forms[r % len(forms):] + forms[:r % len(forms)]:
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(st)
                    for _ in range(reps):
                        gqa.prefill(q, k, v, out=out, form=fm)
                    e1.record(st)
                    torch.cuda.synchronize()
                    times[fm].append(e0.elapsed_time(e1) / reps)
            for fm in forms:
                t = statistics.median(times[fm])
                ratio = statistics.median(times[chosen][i] / times[fm][i] for i in range(rounds))
                row = {"mode": "prefill_form", "S": S, "waves": fm[0], "key_splits": fm[1],
                       "chosen": fm == chosen, "status": "run", "ms_median": round(t, 5),
                       "TFLOPs": round(prefill_flops(S) / (t * 1e-3) / 1e12, 1),
                       "speed_vs_chosen": round(ratio, 3)}
                print(json.dumps(row), flush=True)
                f.write(json.dumps(row) + "\n")
            del q, k, v, out
            torch.cuda.empty_cache()


SWEEP_TILE_S = (1024, 4096, 8192, 16384, 32768)


def sweep_tiles(path: str, rounds: int = 8):
    """Prefill tile-shape sweep at B = 1 (SWEEP_TILE_S, causal): every shape of
    gqa.PREFILL_TILES (rows per wave, keys per tile, waves per workgroup) timed in paired
    rounds as in sweep_forms, against the library's own 8-wave form (32, 64, 8). Parity of
    every point against the oracle: tests/test_sweep_points_gpu.py."""
    import statistics
    import torch
    import gqa_flash_attention_amd as gqa
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    shapes = list(gqa.PREFILL_TILES)
    ref = (32, 64, 8)
    with open(path, "w") as f:
        for S in SWEEP_TILE_S:
            q, k, v = make_inputs(S, 64, dev)[:3]
            out = torch.empty_like(q)
            per = prefill_flops(S) / 1.0e15
            reps = max(2, min(400, int(0.05 / per)))
            for tl in shapes:
                for _ in range(max(3, min(4000, int(0.2 / per)))):
                    gqa.prefill(q, k, v, out=out, tiles=tl)
            torch.cuda.synchronize()
            times = {tl: [] for tl in shapes}
            for r in range(rounds):
                for tl in shapes[r % len(shapes):] + shapes[:r % len(shapes)]:
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(st)
                    for _ in range(reps):
                        gqa.prefill(q, k, v, out=out, tiles=tl)
                    e1.record(st)
                    torch.cuda.synchronize()
                    times[tl].append(e0.elapsed_time(e1) / reps)
            for tl in shapes:
                t = statistics.median(times[tl])
                ratio = statistics.median(times[ref][i] / times[tl][i] for i in range(rounds))
                row = {"mode": "prefill_tiles", "S": S, "rows_per_wave": tl[0], "keys_per_tile": tl[1],
                       "waves": tl[2], "status": "run", "ms_median": round(t, 5),
                       "TFLOPs": round(prefill_flops(S) / (t * 1e-3) / 1e12, 1),
                       "speed_vs_32x64x8": round(ratio, 3)}
                print(json.dumps(row), flush=True)
                f.write(json.dumps(row) + "\n")
            del q, k, v, out
            torch.cuda.empty_cache()


PROBE_HBM_BYTES = 2 << 30                  # 8x the MALL
PROBE_HBM_WORKGROUPS = 512               # 2 per CU: the fastest count measured (256-32768)
PROBE_MFMA_WORKGROUPS, PROBE_MFMA_ROUNDS = 512, 6000


def probe_mfma_flops() -> float:
    """FLOPs of one MFMA probe call: workgroups x 4 waves x rounds x 64 MFMAs x 32768."""
    return float(PROBE_MFMA_WORKGROUPS * 4 * PROBE_MFMA_ROUNDS * 64 * 32768)


def measured_roofs():
    """Run the library's two roofline probes (gqa_attn_probe_*): the cold HBM read rate
    over a 2 GiB buffer (8x the MALL) and the register-resident bf16 MFMA rate with random
    operands, with the shader clock it ran at. Each is the median of 3 timed calls after
    one warm-up call, events on torch's current stream."""
    import torch
    from gqa_flash_attention_amd import _lib
    lib = _lib.get()
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    out = {}

    def timed(fn, n=3):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            fn()
            e1.record(st)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[len(ts) // 2]

    nbytes = PROBE_HBM_BYTES
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    wg = PROBE_HBM_WORKGROUPS
    sink = torch.empty(wg * 256, dtype=torch.int32, device=dev)
    ms = timed(lambda: _lib.check(lib.gqa_attn_probe_hbm_read(buf.data_ptr(), nbytes, wg, sink.data_ptr(),
                                                             sink.numel(), st.cuda_stream), "probe_hbm_read"))
    out["hbm"] = {"value": round(nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                  "method": f"gqa_attn_probe_hbm_read: 2 GiB read once with 16-byte non-temporal loads, {wg}x256 lanes, the workgroups of each XCD reading one 256-byte slice of every 2 KB row (the decode's pattern), median of 3"}
    del buf, sink
    wg, rounds = PROBE_MFMA_WORKGROUPS, PROBE_MFMA_ROUNDS
    sinkf = torch.empty(wg * 256, dtype=torch.float32, device=dev)
    ticks = torch.zeros(2 * wg, dtype=torch.int64, device=dev)
    ms = timed(lambda: _lib.check(lib.gqa_attn_probe_mfma_bf16(rounds, 12345, wg, sinkf.data_ptr(), sinkf.numel(),
                                                              ticks.data_ptr(), ticks.numel(), st.cuda_stream),
                                  "probe_mfma_bf16"))
    t = ticks.cpu().view(-1, 2).double()
    ghz = float((t[:, 0] / t[:, 1]).mean()) * 0.1
    flops = probe_mfma_flops()
    out["mfma_bf16"] = {"value": round(flops / (ms * 1e-3) / 1e12, 1), "unit": "TFLOP/s", "clock_ghz": round(ghz, 3),
                        "method": "gqa_attn_probe_mfma_bf16: v_mfma_f32_32x32x16_bf16 from registers, random bf16, "
                                  "2 waves/SIMD on every CU, median of 3"}
    return out


def calibration_copy(mib: int) -> None:
    """One plain device-to-device copy of a known size, run outside the timed region so a
    counter pass over this process can scale FETCH_SIZE / WRITE_SIZE to bytes."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


def main_line(args):
    import torch
    S, L = args.prefill_s, args.decode_l
    wall, pf, dc = run_step_timing(S, L, args.steps, args.warmup)
    pf_mean = sum(pf) / len(pf)
    dc_mean = sum(dc) / len(dc)

    def pct(xs, p):
        return xs[min(len(xs) - 1, int(p * (len(xs) - 1)))]
    fl = prefill_flops(S)
    by = decode_bytes(L)
    value = fl / (pf_mean * 1e-3) / 1e12
    dec_gbs = by / (dc_mean * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 activations; no dataset)",
        "config": {
            "workload": f"GQA forward, Llama-3-8B attention shape: causal prefill S={S} + decode L={L}, B=1",
            "B": 1, "Hq": HQ, "Hkv": HKV, "D": D, "prefill_S": S, "decode_L": L,
        },
        "decode": {
            "value": round(dec_gbs, 1), "unit": "GB/s",
            "ms": round(dc_mean, 5), "ms_min": round(dc[0], 5), "ms_median": round(dc[len(dc) // 2], 5),
            "ms_p05": round(pct(dc, 0.05), 5), "ms_p95": round(pct(dc, 0.95), 5),
            "bytes": by,
        },
        "prefill": {
            "ms": round(pf_mean, 4), "ms_min": round(pf[0], 4), "ms_median": round(pf[len(pf) // 2], 4),
            "ms_p05": round(pct(pf, 0.05), 4), "ms_p95": round(pct(pf, 0.95), 4),
            "flops": fl,
        },
        "roofline": {
            "bound": "mfma", "achieved": round(value, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(value / PEAK_BF16_TFLOPS, 4),
            "traffic": load_traffic(f"prefill_S{S}"),
            "kernel": "prefill_kernel<causal>",
        },
        "roofline_decode": {
            "bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
            "traffic": load_traffic(f"decode_L{L}"),
            "kernel": "decode_kernel<fused> (split-KV + in-kernel merge, one launch)",
        },
        "device": torch.cuda.get_device_name(0),
        "host_cpu": host_cpu_model(),
    }
    # Kernel time (rocprofv3 trace of `--kernel-sizes` on the same kernel sources): the
    # dispatch's own duration, without the launch gap the per-call events above include.
    for obj, key, work, unit, peak in ((line["roofline"], f"prefill_S{S}", fl, 1e12, PEAK_BF16_TFLOPS),
                                       (line["roofline_decode"], f"decode_L{L}", by, 1e9, PEAK_HBM_GBS)):
        kt = load_kernel_time(key)
        if kt is not None:
            rate = work / (kt["kernel_us_median"] * 1e-6) / unit
            obj["kernel_time"] = {"us_median": round(kt["kernel_us_median"], 2),
                                  "us_p05": round(kt["kernel_us_p05"], 2), "us_p95": round(kt["kernel_us_p95"], 2),
                                  "achieved": round(rate, 1), "frac": round(rate / peak, 4),
                                  "source": "profiles/kernel_time.json"}
    if args.probes:
        roofs = measured_roofs()
        line["roofline"]["measured_peak"] = roofs["mfma_bf16"]
        line["roofline"]["frac_of_measured"] = round(value / roofs["mfma_bf16"]["value"], 4)
        line["roofline_decode"]["measured_peak"] = roofs["hbm"]
        line["roofline_decode"]["frac_of_measured"] = round(dec_gbs / roofs["hbm"]["value"], 4)
    if args.cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(S, budget_s=args.cpu_budget)
        line["cpu_baseline_decode"] = cpu_baseline_decode(L)
        line["cpu_baseline_decode"]["cores"] = line["cpu_baseline"]["cores"]
        line["cpu_baseline"]["cpu_model"] = line["host_cpu"]
    if args.calib_copy_mb:
        calibration_copy(args.calib_copy_mb)
    print(json.dumps(line), flush=True)


def sweep(path, steps, warmup):
    """Every prefill and decode size of the workload, each timed on its own (events per call).
    Each size first runs ~0.2 s of calls (the board's power management needs that long to
    settle the clock; a fixed count of short calls would time a ramping clock), then at least
    `steps` timed calls and ~50 ms of them. Decode caches are rotated through >= 1 GB of
    distinct copies so the MALL holds none."""
    import torch
    import gqa_flash_attention_amd as gqa
    from gqa_inputs import decode_inputs, prefill_inputs, random_lens, randn_bf16_device, seed_base
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    rows = []

    def timed(fn, n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            evs[i][0].record(stream)
            fn(i)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in evs)

    def settle(fn, n0):
        """Run ~0.2 s of calls after n0 warm-up calls; return how many calls make ~50 ms."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n0):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        per = max(e0.elapsed_time(e1) / max(n0, 1), 1e-3)     # ms per call
        for i in range(min(20000, int(200.0 / per))):
            fn(i)
        torch.cuda.synchronize()
        return min(4000, int(50.0 / per))

    # the workload's sizes, then its ragged prefill lengths
    for S in (512, 2048, 4096, 8192, 16384, 32768, 1, 127, 3000):
        q, k, v = [x.to(dev) for x in prefill_inputs(1, S, base=seed_base(2, 0))]
        out = torch.empty_like(q)
        call = lambda i: gqa.prefill(q, k, v, out=out)
        n = settle(call, max(warmup, 3))
        ms = timed(call, max(steps, n))
        med = ms[len(ms) // 2]
        r = {"mode": "prefill", "S": S, "ms_median": med, "ms_min": ms[0],
             "tflops": prefill_flops(S) / (med * 1e-3) / 1e12}
        r["frac_of_peak"] = r["tflops"] / PEAK_BF16_TFLOPS
        print(json.dumps(r), flush=True)
        rows.append(r)
        del q, k, v, out
    for L in (2048, 4096, 8192, 16384, 32768, 65536):
        per = L * HKV * D * 2 * 2
        ncopies = max(2, min(64, -(-(1 << 30) // per)))
        qd, kc, vc, lens = decode_inputs(1, L, base=seed_base(1, 0))
        qd, lens = qd.to(dev), lens.to(dev)
        kcs = [kc.to(dev) for _ in range(ncopies)]
        vcs = [vc.to(dev) for _ in range(ncopies)]
        out = torch.empty_like(qd)
        call = lambda i: gqa.decode(qd, kcs[i % ncopies], vcs[i % ncopies], lens, out=out)
        n = settle(call, max(warmup, ncopies))
        ms = timed(call, max(steps, 2 * ncopies, n))
        med = ms[len(ms) // 2]
        r = {"mode": "decode", "L": L, "ms_median": med, "ms_min": ms[0], "copies_rotated": ncopies,
             "gbs": decode_bytes(L) / (med * 1e-3) / 1e9}
        r["frac_of_peak"] = r["gbs"] / PEAK_HBM_GBS
        print(json.dumps(r), flush=True)
        rows.append(r)
        del kcs, vcs
        torch.cuda.empty_cache()
    # decodes replayed from one HIP graph (16 calls on rotated caches, caller workspace):
    # the per-call cost of a decode loop once the launch gaps are gone
    for L in (2048, 16384, 65536):
        per = L * HKV * D * 2 * 2
        ncopies = max(2, min(16, -(-(1 << 30) // per)))
        qd, kc, vc, lens = decode_inputs(1, L, base=seed_base(1, 0))
        qd, lens = qd.to(dev), lens.to(dev)
        kcs = [kc.to(dev) for _ in range(ncopies)]
        vcs = [vc.to(dev) for _ in range(ncopies)]
        ws = gqa.decode_workspace(1, L, HQ, HKV, D, device=dev)
        outs = [torch.empty_like(qd) for _ in range(16)]
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for i in range(16):
                gqa.decode(qd, kcs[i % ncopies], vcs[i % ncopies], lens, out=outs[i], workspace=ws)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(16):
                gqa.decode(qd, kcs[i % ncopies], vcs[i % ncopies], lens, out=outs[i], workspace=ws)
        torch.cuda.synchronize()
        call = lambda i: graph.replay()
        n = settle(call, 3)
        ms = timed(call, max(steps, n))
        med = ms[len(ms) // 2] / 16
        r = {"mode": "decode_graph", "L": L, "calls_per_replay": 16, "ms_median_per_call": med,
             "gbs": decode_bytes(L) / (med * 1e-3) / 1e9}
        r["frac_of_peak"] = r["gbs"] / PEAK_HBM_GBS
        print(json.dumps(r), flush=True)
        rows.append(r)
        del graph, kcs, vcs, ws, outs
        torch.cuda.empty_cache()
    # batched decodes, every sequence at the full cache length (B*L = 256K-512K keys), caches
    # rotated over >= 1 GB so every call reads from HBM
    for B, L in ((32, 16384), (16, 32768), (8, 65536), (64, 4096)):
        per = B * L * HKV * D * 2 * 2
        ncopies = max(2, min(16, -(-(1 << 30) // per)))
        qd = randn_bf16_device((B, HQ, D), seed_base(4, 4), dev)
        kcs = [randn_bf16_device((B, L, HKV, D), seed_base(4, 4) + 10 + i, dev) for i in range(ncopies)]
        vcs = [randn_bf16_device((B, L, HKV, D), seed_base(4, 4) + 30 + i, dev) for i in range(ncopies)]
        lens = torch.full((B,), L, dtype=torch.int32, device=dev)
        out = torch.empty_like(qd)
        call = lambda i: gqa.decode(qd, kcs[i % ncopies], vcs[i % ncopies], lens, out=out)
        n = settle(call, max(warmup, ncopies))
        ms = timed(call, max(steps, n))
        med = ms[len(ms) // 2]
        r = {"mode": "decode_batched", "B": B, "L": L, "ms_median": med, "ms_min": ms[0],
             "copies_rotated": ncopies, "gbs": decode_bytes(B * L, B) / (med * 1e-3) / 1e9}
        r["frac_of_peak"] = r["gbs"] / PEAK_HBM_GBS
        print(json.dumps(r), flush=True)
        rows.append(r)
        del kcs, vcs
        torch.cuda.empty_cache()
    # the ragged batch: B = 16, capacity 50001, lengths U[1, 50001] (the parity tests' seed);
    # each cache copy is 3.3 GB, so every call reads cold from HBM
    B, L = 16, 50001
    lens = random_lens(B, 1, L, seed=seed_base(4, 3) + 3).to(dev)
    qd = randn_bf16_device((B, HQ, D), seed_base(4, 3), dev)
    kcs = [randn_bf16_device((B, L, HKV, D), seed_base(4, 3) + 10 + i, dev) for i in range(2)]
    vcs = [randn_bf16_device((B, L, HKV, D), seed_base(4, 3) + 20 + i, dev) for i in range(2)]
    out = torch.empty_like(qd)
    call = lambda i: gqa.decode(qd, kcs[i % 2], vcs[i % 2], lens, out=out)
    n = settle(call, max(warmup, 2))
    ms = timed(call, max(steps, n))
    med = ms[len(ms) // 2]
    total = int(lens.sum().item())
    r = {"mode": "decode_ragged", "B": B, "L": L, "sum_lens": total, "ms_median": med, "ms_min": ms[0],
         "gbs": decode_bytes(total, B) / (med * 1e-3) / 1e9}
    r["frac_of_peak"] = r["gbs"] / PEAK_HBM_GBS
    print(json.dumps(r), flush=True)
    rows.append(r)
    del kcs, vcs
    torch.cuda.empty_cache()
    with open(path, "w") as f:
        for r in rows:
            f.write(json.dumps(r) + "\n")


KERNEL_SIZES_PREFILL = (2048, 4096, 8192, 16384, 32768)
KERNEL_SIZES_DECODE = (2048, 4096, 8192, 16384, 32768, 65536)
# batched decodes, every sequence at the full cache length, as in --sweep
KERNEL_SIZES_DECODE_BATCHED = ((32, 16384), (16, 32768), (8, 65536), (64, 4096))


def kernel_sizes(path: str, timed: int = 200):
    """Every prefill and decode size of the workload (B = 1), one after another, for a
    rocprofv3 kernel trace: per size a fixed number of settling calls (~0.2 s) and then
    `timed` calls, each between HIP events on the kernels' stream. Decode caches rotate
    through >= 1 GB of copies, so no call finds its cache in the MALL. One JSON line per
    size records the call counts (kernel_stats.py --sizes matches them, in order, with the
    trace's dispatches) and the event figures. Run it under
        rocprofv3 --kernel-trace --output-format csv -d DIR -o sizes -- python3 bench.py --kernel-sizes OUT
    and summarize with python -m gqa_flash_attention_amd.kernel_stats --sizes DIR OUT."""
    import statistics
    import torch
    import gqa_flash_attention_amd as gqa
    from gqa_inputs import decode_inputs, prefill_inputs, seed_base
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    rows = []

    def run(kind, size, call, per_call_ms, extra):
        settle = max(5, min(5000, int(200.0 / per_call_ms)))
        for i in range(settle):
            call(i)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(timed)]
        for i in range(timed):
            evs[i][0].record(st)
            call(settle + i)
            evs[i][1].record(st)
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in evs)
        r = {"mode": kind, ("S" if kind == "prefill" else "L"): size, "settle_calls": settle, "timed_calls": timed,
             "event_ms_median": statistics.median(ms), "event_ms_p05": ms[int(0.05 * (timed - 1))],
             "event_ms_p95": ms[int(0.95 * (timed - 1))], "event_ms_min": ms[0], **extra}
        print(json.dumps(r), flush=True)
        rows.append(r)

    for S in KERNEL_SIZES_PREFILL:
        q, k, v = [x.to(dev) for x in prefill_inputs(1, S, base=seed_base(2, KERNEL_SIZES_PREFILL.index(S)))]
        out = torch.empty_like(q)
        run("prefill", S, lambda i: gqa.prefill(q, k, v, out=out), prefill_flops(S) / 1.0e12,
            {"flops": prefill_flops(S)})
        del q, k, v, out
    for L in KERNEL_SIZES_DECODE:
        per = L * HKV * D * 2 * 2
        nc = max(2, min(64, -(-(1 << 30) // per)))
        qd, kc, vc, lens = decode_inputs(1, L, base=seed_base(1, KERNEL_SIZES_DECODE.index(L)))
        qd, lens = qd.to(dev), lens.to(dev)
        kcs = [kc.to(dev) for _ in range(nc)]
        vcs = [vc.to(dev) for _ in range(nc)]
        out = torch.empty_like(qd)
        run("decode", L, lambda i: gqa.decode(qd, kcs[i % nc], vcs[i % nc], lens, out=out), 0.02,
            {"bytes": decode_bytes(L), "copies_rotated": nc})
        del kcs, vcs
        torch.cuda.empty_cache()
    from gqa_inputs import randn_bf16_device
    for B, L in KERNEL_SIZES_DECODE_BATCHED:
        qd = randn_bf16_device((B, HQ, D), seed_base(4, 4), dev)
        kcs = [randn_bf16_device((B, L, HKV, D), seed_base(4, 4) + 10 + i, dev) for i in range(2)]
        vcs = [randn_bf16_device((B, L, HKV, D), seed_base(4, 4) + 30 + i, dev) for i in range(2)]
        lens = torch.full((B,), L, dtype=torch.int32, device=dev)
        out = torch.empty_like(qd)
        run("decode", L, lambda i: gqa.decode(qd, kcs[i % 2], vcs[i % 2], lens, out=out), 0.3,
            {"B": B, "bytes": decode_bytes(B * L, B), "copies_rotated": 2})
        del kcs, vcs
        torch.cuda.empty_cache()
    # the ragged batch of --sweep and the parity tests: B = 16, lengths U[1, 50001]
    B, L = 16, 50001
    from gqa_inputs import random_lens
    lens_h = random_lens(B, 1, L, seed=seed_base(4, 3) + 3)
    qd = randn_bf16_device((B, HQ, D), seed_base(4, 3), dev)
    kcs = [randn_bf16_device((B, L, HKV, D), seed_base(4, 3) + 10 + i, dev) for i in range(2)]
    vcs = [randn_bf16_device((B, L, HKV, D), seed_base(4, 3) + 20 + i, dev) for i in range(2)]
    lens = lens_h.to(dev)
    out = torch.empty_like(qd)
    run("decode", L, lambda i: gqa.decode(qd, kcs[i % 2], vcs[i % 2], lens, out=out), 0.3,
        {"B": B, "ragged": True, "bytes": decode_bytes(int(lens_h.sum()), B), "copies_rotated": 2})
    del kcs, vcs
    torch.cuda.empty_cache()
    with open(path, "w") as f:
        for r in rows:
            f.write(json.dumps(r) + "\n")


READ_FLOOR_L = (16384, 32768, 65536)
READ_FLOOR_WORKGROUPS = (256, 512, 1024)


def read_floor(path: str, timed: int = 100, settle: int = 200):
    """The cold pure-read floor under a decode: the library's HBM read probe over exactly
    the bytes of a batch-1 decode's K and V (4096 * L) for each L of READ_FLOOR_L, with 256
    workgroups (one per CU, the decode's grid at batch 1), 512 and 1024, each buffer one of
    >= 1 GB of copies in rotation so no call finds it in the MALL. Per point `settle` calls,
    then `timed` calls between HIP events; one JSON line per point with its call counts, for
    kernel_stats.py --read-floor to match against a rocprofv3 kernel trace:
        rocprofv3 --kernel-trace --output-format csv -d DIR -o floor -- python3 bench.py --read-floor OUT
    Nothing but the read happens: no arithmetic, no merge. A decode of the same cache can
    not take less kernel time than the best of these points."""
    import statistics
    import torch
    from gqa_flash_attention_amd import _lib
    lib = _lib.get()
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    rows = []
    for L in READ_FLOOR_L:
        nbytes = L * HKV * D * 2 * 2
        nc = max(4, (1 << 30) // nbytes)
        bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(nc)]
        for wg in READ_FLOOR_WORKGROUPS:
            sink = torch.empty(wg * 256, dtype=torch.int32, device=dev)

            def call(i):
                _lib.check(lib.gqa_attn_probe_hbm_read(bufs[i % nc].data_ptr(), nbytes, wg, sink.data_ptr(),
                                                       sink.numel(), st.cuda_stream), "gqa_attn_probe_hbm_read")
            for i in range(settle):
                call(i)
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(timed)]
            for i in range(timed):
                ev[i][0].record(st)
                call(settle + i)
                ev[i][1].record(st)
            torch.cuda.synchronize()
            ms = statistics.median(a.elapsed_time(b) for a, b in ev)
            r = {"mode": "read_floor", "L": L, "bytes": nbytes, "workgroups": wg, "settle_calls": settle,
                 "timed_calls": timed, "event_us_median": round(ms * 1e3, 2)}
            print(json.dumps(r), flush=True)
            rows.append(r)
        del bufs
        torch.cuda.empty_cache()
    with open(path, "w") as f:
        for r in rows:
            f.write(json.dumps(r) + "\n")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prefill-s", type=int, default=32768)
    ap.add_argument("--decode-l", type=int, default=65536)
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--no-probes", dest="probes", action="store_false",
                    help="skip the measured HBM and MFMA roofs (gqa_attn_probe_*)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work in the CPU baseline")
    ap.add_argument("--sweep", metavar="OUT_JSONL", default=None)
    ap.add_argument("--sweep-chunks", metavar="OUT_JSONL", default=None,
                    help="decode split-size sweep with paired timing (see sweep_chunks)")
    ap.add_argument("--sweep-forms", metavar="OUT_JSONL", default=None,
                    help="prefill workgroup-form sweep with paired timing (see sweep_forms)")
    ap.add_argument("--sweep-tiles", metavar="OUT_JSONL", default=None,
                    help="prefill tile-shape sweep with paired timing (see sweep_tiles)")
    ap.add_argument("--read-floor", metavar="OUT_JSONL", default=None,
                    help="cold pure-read floor at the decode sizes, for a kernel trace (see read_floor)")
    ap.add_argument("--kernel-sizes", metavar="OUT_JSONL", default=None,
                    help="every prefill/decode size back to back, for a rocprofv3 kernel trace (see kernel_sizes)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after the timed steps, one device copy of this many MiB (for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(the attention hot path here runs on a single MI355X). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        sweep(args.sweep, args.steps, args.warmup)
    elif args.sweep_chunks:
        sweep_chunks(args.sweep_chunks)
    elif args.sweep_forms:
        sweep_forms(args.sweep_forms)
    elif args.sweep_tiles:
        sweep_tiles(args.sweep_tiles)
    elif args.read_floor:
        read_floor(args.read_floor)
    elif args.kernel_sizes:
        kernel_sizes(args.kernel_sizes)
    else:
        main_line(args)


if __name__ == "__main__":
    main()
