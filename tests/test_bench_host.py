"""Host-side checks of bench.py (no GPU needed): the workload's work formulas, the decode
split-sweep points, the form-sweep sizes, the decode CPU baseline's record, and the
single-GPU guard of the command line."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_prefill_flops_follow_the_causal_half_formula():
    # 2*2*S*(S+1)/2*Hq*D for one sequence (the causal half of both contractions)
    assert bench.prefill_flops(32768) == 2 * 2 * 32768 * 32769 / 2 * 32 * 128
    assert abs(bench.prefill_flops(32768) - 8.796361457664e12) < 1.0
    assert abs(bench.prefill_flops(8192) - 549.8e9) < 0.1e9
    assert bench.prefill_flops(1) == 2 * 2 * 1 * 32 * 128
    assert bench.prefill_flops(100, B=3) == 3 * bench.prefill_flops(100)


def test_decode_bytes_count_kv_once_plus_q_and_out():
    # K and V read once for the 8 KV heads, plus q and out (32 heads x 128 bf16 each)
    assert bench.decode_bytes(65536) == 2 * 65536 * 8 * 128 * 2 + 2 * 32 * 128 * 2
    assert bench.decode_bytes(65536) == 268451840
    assert bench.decode_bytes(1000, B=4) == 2 * 1000 * 8 * 128 * 2 + 2 * 4 * 32 * 128 * 2


def test_chunk_candidates_cover_the_library_choice_and_the_powers_of_two():
    for L in bench.SWEEP_CHUNK_L:
        default, run, skip = bench.chunk_candidates(L)
        assert default in run
        assert all(c % 64 == 0 and 128 <= c <= 16384 for c in run)
        assert set(run) >= {c for c in (128, 256, 512, 1024, 2048, 4096, 8192, 16384) if c <= L}
        assert all(c > L for c, _ in skip)
    d, run, skip = bench.chunk_candidates(2048)
    assert max(run) <= 2048 and {c for c, _ in skip} == {4096, 8192, 16384}


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_form_sweep_covers_every_plan_boundary():
    # every workload prefill size, plus sizes on each side of the form boundaries (2048 | 2049,
    # 3392 | 3393 at batch 1) so each form is timed where the library picks it
    assert set(bench.SWEEP_FORM_S) >= {512, 2048, 4096, 8192, 16384, 32768}
    assert any(512 <= S <= 2048 for S in bench.SWEEP_FORM_S)
    assert any(2048 < S <= 3392 for S in bench.SWEEP_FORM_S)
    assert any(S > 3392 for S in bench.SWEEP_FORM_S)


def test_cpu_baseline_decode_record():
    r = bench.cpu_baseline_decode(256, budget_s=0.05)
    assert r["unit"] == "GB/s" and r["kind"] == "oracle" and r["value"] > 0
    calls = int(r["sample"].split(": ")[1].split(" calls")[0])
    assert calls >= 1
    assert "L=256" in r["sample"]
