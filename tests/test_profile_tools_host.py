"""The profile post-processors on synthetic rocprofv3 output (CPU only): the per-launch HBM
bytes of traffic.py, the clock / MFMA utilisation / FLOP ratio / hit rate of counters.py and
the rates of kernel_stats.py are recomputed here from values chosen so every figure is known
in advance."""

import csv
import json
import os

import pytest

from gqa_flash_attention_amd import counters, traffic

import bench

FIELDS = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value",
          "Start_Timestamp", "End_Timestamp"]
PREFILL = "void gqa::prefill_kernel<true, true, 8>(gqa::PrefillArgs)"
DECODE = "void gqa::decode_kernel<4, true, true>(gqa::DecodeArgs)"


def _write(d, rows, agent=True):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "pmc_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(r)
    if agent:
        with open(os.path.join(d, "pmc_agent_info.csv"), "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Agent_Type", "Num_Xcc", "Simd_Count"])
            w.writeheader()
            w.writerow({"Agent_Type": "CPU", "Num_Xcc": 0, "Simd_Count": 0})
            w.writerow({"Agent_Type": "GPU", "Num_Xcc": 8, "Simd_Count": 1024})


def _row(did, name, counter, value, t0, ns, grid=1024):
    return {"Dispatch_Id": did, "Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter,
            "Counter_Value": value, "Start_Timestamp": t0, "End_Timestamp": t0 + ns}


def test_traffic_scales_by_the_calibration_copy(tmp_path):
    S, L = 2048, 4096
    mib = 16
    fetch, write = [], []
    # the calibration copy: FETCH_SIZE reads 2x the copied KiB, WRITE_SIZE 1x
    fetch.append(_row(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 2 * mib * 1024, 0, 10, grid=4096))
    write.append(_row(1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", mib * 1024, 0, 10, grid=4096))
    for i, (pf, df) in enumerate(((3000.0, 500.0), (3100.0, 520.0))):
        fetch += [_row(10 + 2 * i, PREFILL, "FETCH_SIZE", pf, 100, 10), _row(11 + 2 * i, DECODE, "FETCH_SIZE", df, 200, 10)]
        write += [_row(10 + 2 * i, PREFILL, "WRITE_SIZE", 700.0, 100, 10), _row(11 + 2 * i, DECODE, "WRITE_SIZE", 4.0, 200, 10)]
    _write(tmp_path / "f", fetch, agent=False)
    _write(tmp_path / "w", write, agent=False)
    res = traffic.summarize(str(tmp_path / "f"), str(tmp_path / "w"), mib, S, L)
    assert res["calibration"]["fetch_scale"] == pytest.approx(0.5)
    assert res["calibration"]["write_scale"] == pytest.approx(1.0)
    p = res["kernels"][f"prefill_S{S}"]
    assert p["fetch_bytes"] == pytest.approx(3050.0 * 1024 * 0.5)
    assert p["write_bytes"] == pytest.approx(700.0 * 1024)
    assert p["algorithmic_bytes"] == bench.prefill_bytes(S)
    d = res["kernels"][f"decode_L{L}"]
    assert d["hbm_bytes_per_launch"] == pytest.approx(510.0 * 1024 * 0.5 + 4.0 * 1024)
    assert d["ratio_to_algorithmic"] == pytest.approx(d["hbm_bytes_per_launch"] / bench.decode_bytes(L))


def test_counters_clock_utilisation_and_flop_ratio(tmp_path):
    S, L = 4096, 8192
    ns_p, ns_d = 2_000_000, 40_000          # dispatch durations
    ghz = 1.9                               # shader clock the GRBM counts imply
    util = 0.6                              # MFMA busy fraction of SIMD cycles
    sq, tcc = [], []
    did = 0
    for rep in range(5):                    # 2 warm-up dispatches per kernel, then 3
        for name, ns, flop_ratio in ((PREFILL, ns_p, 1.002), (DECODE, ns_d, 0.0)):
            did += 1
            t0 = 1_000_000_000 * did
            cyc = ghz * ns                  # one XCD's busy cycles
            for x in range(8):              # GRBM_GUI_ACTIVE: one row per XCD
                sq.append(_row(did, name, "GRBM_GUI_ACTIVE", cyc, t0, ns))
                tcc.append(_row(did, name, "GRBM_GUI_ACTIVE", cyc, t0, ns))
            mops = flop_ratio * bench.prefill_flops(S) / 512 if name == PREFILL else 0.0
            for se in range(4):             # SQ counters: rows per shader engine, summed
                sq.append(_row(did, name, "SQ_VALU_MFMA_BUSY_CYCLES", util * cyc * 1024 / 4, t0, ns))
                sq.append(_row(did, name, "SQ_VALU_MFMA_COEXEC_CYCLES", 0.1 * cyc * 1024 / 4, t0, ns))
                sq.append(_row(did, name, "SQ_INSTS_VALU_MFMA_MOPS_BF16", mops / 4, t0, ns))
                sq.append(_row(did, name, "SQ_ACTIVE_INST_LDS", 1000.0, t0, ns))
                sq.append(_row(did, name, "SQ_LDS_BANK_CONFLICT", 250.0 if name == DECODE else 0.0, t0, ns))
            tcc.append(_row(did, name, "TCC_HIT_sum", 900.0 if name == PREFILL else 10.0, t0, ns))
            tcc.append(_row(did, name, "TCC_MISS_sum", 100.0 if name == PREFILL else 990.0, t0, ns))
    _write(tmp_path / "sq", sq)
    _write(tmp_path / "tcc", tcc)
    res = counters.summarize(str(tmp_path / "sq"), str(tmp_path / "tcc"), S, L, warmup=2)
    assert (res["xcds"], res["simds"]) == (8, 1024)
    p = res["kernels"][f"prefill_S{S}"]
    d = res["kernels"][f"decode_L{L}"]
    assert p["dispatches"] == d["dispatches"] == 3
    assert p["clock_ghz"] == pytest.approx(ghz)
    assert p["mfma_util"] == pytest.approx(util)
    assert p["mfma_valu_coexec"] == pytest.approx(0.1)
    assert p["mfma_flops_over_algorithmic"] == pytest.approx(1.002)
    assert p["lds_bank_conflict_per_lds_cycle"] == 0.0
    assert p["l2_hit_rate"] == pytest.approx(0.9)
    assert d["lds_bank_conflict_per_lds_cycle"] == pytest.approx(0.25)
    assert d["l2_hit_rate"] == pytest.approx(0.01)
    assert d["duration_us"] == pytest.approx(40.0)


def test_kernel_stats_summary_rates(tmp_path):
    from gqa_flash_attention_amd import kernel_stats
    d = tmp_path / "prof"
    d.mkdir()
    stats = [("void gqa::prefill_kernel<true, true, 8>(gqa::PrefillArgs)", 30, 7.5e6),
             ("gqa::probe_mfma_bf16_kernel(int)", 4, 1.45e7),
             ("void gqa::decode_kernel<4, true, true>(gqa::DecodeArgs)", 30, 5.0e4),
             ("gqa::probe_hbm_read_kernel(int)", 4, 3.6e5)]
    with open(d / "bench_kernel_stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"])
        w.writeheader()
        for name, calls, ns in stats:
            w.writerow({"Name": name, "Calls": calls, "AverageNs": ns, "MinNs": int(ns), "MaxNs": int(ns), "Percentage": 1.0})
    S, L = 32768, 65536
    bj = {"value": 1180.0, "config": {"prefill_S": S, "decode_L": L},
          "prefill": {"ms": 7.45, "flops": bench.prefill_flops(S)},
          "decode": {"ms": 0.052, "value": 5160.0, "bytes": bench.decode_bytes(L)},
          "roofline": {"measured_peak": {"value": 1800.0, "clock_ghz": 1.8}},
          "roofline_decode": {"measured_peak": {"value": 6200.0}}}
    (tmp_path / "bench.json").write_text(json.dumps(bj))
    text = kernel_stats.summarize(str(d), str(tmp_path / "bench.json"), str(tmp_path / "out.md"))
    # rates from the averages: prefill 8.796e12 flop / 7.5 ms, decode 268.45 MB / 50 us
    assert f"prefill {bench.prefill_flops(S) / 7.5e6 / 1e3:.0f} TFLOP/s" in text
    assert f"decode {bench.decode_bytes(L) / 5.0e4:.0f} GB/s" in text
    assert f"MFMA probe {bench.probe_mfma_flops() / 1.45e7 / 1e3:.0f} TFLOP/s" in text
    assert (tmp_path / "out.md").read_text() == text


TRACE_FIELDS = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]


def _trace(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_kernel_trace.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=TRACE_FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_kernel_sizes_match_dispatches_in_order(tmp_path):
    from gqa_flash_attention_amd import kernel_stats
    # two prefill sizes and one decode size; a workspace fill kernel in between is ignored
    sizes = [{"mode": "prefill", "S": 4096, "settle_calls": 2, "timed_calls": 3, "event_ms_median": 0.2,
              "event_ms_p05": 0.19, "event_ms_p95": 0.21, "event_ms_min": 0.18, "flops": bench.prefill_flops(4096)},
             {"mode": "prefill", "S": 8192, "settle_calls": 1, "timed_calls": 3, "event_ms_median": 0.6,
              "event_ms_p05": 0.55, "event_ms_p95": 0.65, "event_ms_min": 0.5, "flops": bench.prefill_flops(8192)},
             {"mode": "decode", "L": 16384, "settle_calls": 1, "timed_calls": 2, "event_ms_median": 0.02,
              "event_ms_p05": 0.02, "event_ms_p95": 0.02, "event_ms_min": 0.02, "bytes": bench.decode_bytes(16384)},
             {"mode": "decode", "L": 4096, "B": 64, "settle_calls": 1, "timed_calls": 2, "event_ms_median": 0.2,
              "event_ms_p05": 0.2, "event_ms_p95": 0.2, "event_ms_min": 0.2, "bytes": bench.decode_bytes(64 * 4096)},
             {"mode": "decode", "L": 50001, "B": 16, "ragged": True, "settle_calls": 1, "timed_calls": 2,
              "event_ms_median": 0.3, "event_ms_p05": 0.3, "event_ms_p95": 0.3, "event_ms_min": 0.3,
              "bytes": bench.decode_bytes(390221)}]
    t, rows = 0, []

    def k(name, ns):
        nonlocal t
        rows.append({"Kind": "KERNEL_DISPATCH", "Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + ns})
        t += ns + 1000
    for ns in (999, 999, 100000, 110000, 120000):            # S = 4096: 2 settling, median 110 us
        k(PREFILL, ns)
    for ns in (1, 400000, 500000, 450000):                   # S = 8192: median 450 us
        k(PREFILL, ns)
    k("gqa::fill_words_kernel(unsigned int*, unsigned long, unsigned int)", 5)
    for ns in (7, 16000, 18000):                             # L = 16384: median 17 us
        k(DECODE, ns)
    for ns in (7, 150000, 160000):                           # B = 64, L = 4096: median 155 us
        k(DECODE, ns)
    for ns in (7, 240000, 260000):                           # ragged B = 16: median 250 us
        k(DECODE, ns)
    _trace(tmp_path / "tr", rows)
    with open(tmp_path / "sizes.jsonl", "w") as f:
        for r in sizes:
            f.write(json.dumps(r) + "\n")
    kernel_stats.summarize_sizes(str(tmp_path / "tr"), str(tmp_path / "sizes.jsonl"), str(tmp_path / "o.md"),
                                 str(tmp_path / "o.json"))
    res = json.load(open(tmp_path / "o.json"))["sizes"]
    assert res["prefill_S4096"]["kernel_us_median"] == pytest.approx(110.0)
    assert res["prefill_S8192"]["kernel_us_median"] == pytest.approx(450.0)
    assert res["decode_L16384"]["kernel_us_median"] == pytest.approx(17.0)
    assert res["decode_L16384"]["frac_kernel"] == pytest.approx(bench.decode_bytes(16384) / 17e-6 / 8e12)
    assert res["decode_B64_L4096"]["kernel_us_median"] == pytest.approx(155.0)
    assert res["decode_B16_L50001_ragged"]["gbs_kernel"] == pytest.approx(bench.decode_bytes(390221) / 250e-6 / 1e9)
    assert res["prefill_S8192"]["tflops_kernel"] == pytest.approx(bench.prefill_flops(8192) / 450e-6 / 1e12)
    # a dispatch count that does not add up is an error, not a silent mismatch
    rows.append({"Kind": "KERNEL_DISPATCH", "Kernel_Name": DECODE, "Start_Timestamp": t, "End_Timestamp": t + 1})
    _trace(tmp_path / "tr2", rows)
    with pytest.raises(SystemExit):
        kernel_stats.summarize_sizes(str(tmp_path / "tr2"), str(tmp_path / "sizes.jsonl"), str(tmp_path / "o.md"),
                                     str(tmp_path / "o.json"))


def test_read_floor_points_match_probe_dispatches(tmp_path):
    from gqa_flash_attention_amd import kernel_stats
    probe = "gqa::(anonymous namespace)::probe_hbm_read_kernel(unsigned int __vector(4) const*, unsigned long, unsigned int*, int)"
    pts = [{"mode": "read_floor", "L": 16384, "bytes": 16384 * 4096, "workgroups": wg, "settle_calls": 1,
            "timed_calls": 3, "event_us_median": 15.0} for wg in (256, 512)]
    t, rows = 0, []
    for durs in ((1, 12000, 12500, 13000), (1, 10800, 11000, 10900)):
        for ns in durs:
            rows.append({"Kind": "KERNEL_DISPATCH", "Kernel_Name": probe, "Start_Timestamp": t, "End_Timestamp": t + ns})
            t += ns + 100
    _trace(tmp_path / "tr", rows)
    with open(tmp_path / "f.jsonl", "w") as f:
        for r in pts:
            f.write(json.dumps(r) + "\n")
    text = kernel_stats.summarize_read_floor(str(tmp_path / "tr"), str(tmp_path / "f.jsonl"), str(tmp_path / "o.md"),
                                             None)
    assert "| 16384 | 67108864 | 256 | 12.50 |" in text
    assert "| 16384 | 67108864 | 512 | 10.90 |" in text
