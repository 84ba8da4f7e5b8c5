"""The two roofline probes (gqa_attn_probe_*), checked on the GPU.

- hbm_read must read every 16-byte chunk of the buffer exactly once: each lane's XOR of
  the chunks it visits is compared bit for bit with the same XOR computed on the host
  (lane t visits chunks t, t + stride, t + 2 stride, ... with stride = 256 * workgroups).
- mfma_bf16 must report tick counts from which a plausible shader clock follows, and its
  accumulators must be finite.
"""

import numpy as np
import pytest
import torch

from gqa_flash_attention_amd import _lib

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _expected_sinks(chunks, wg):
    """Per-lane XOR of the chunks each lane reads, for the two read patterns the probe's
    header documents."""
    n16, lanes = chunks.shape[0], wg * 256
    want = np.zeros(lanes, dtype=np.uint32)
    if wg % 8 == 0 and n16 % 128 == 0:
        rows, K = n16 // 128, wg // 8
        for w in range(wg):
            x, k = w % 8, w // 8
            for t in range(256):
                r = np.arange(16 * k + t // 16, rows, 16 * K)
                acc = np.bitwise_xor.reduce(chunks[r * 128 + 16 * x + t % 16], axis=0) if len(r) else np.zeros(4, np.uint32)
                want[w * 256 + t] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3]
    else:
        for t in range(lanes):
            acc = np.bitwise_xor.reduce(chunks[t::lanes], axis=0) if t < n16 else np.zeros(4, np.uint32)
            want[t] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3]
    return want


@pytest.mark.parametrize("nbytes,wg", [(1 << 20, 64), (3 * (1 << 20) + 16 * 37, 7), (3 * (1 << 20), 24),
                                       (1 << 20, 12), (16 << 20, 512)])   # the last: bench.py's workgroup count
def test_hbm_read_probe_visits_every_chunk_once(nbytes, wg):
    _say(f"probe_hbm_read bytes={nbytes} workgroups={wg}")
    lib = _lib.get()
    rng = np.random.default_rng(nbytes + wg)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to("cuda:0")
    sink = torch.zeros(wg * 256, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream()
    _lib.check(lib.gqa_attn_probe_hbm_read(buf.data_ptr(), nbytes, wg, sink.data_ptr(), sink.numel(),
                                           st.cuda_stream), "probe_hbm_read")
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    chunks = host.reshape(-1, 4)                       # 16-byte chunks
    assert np.array_equal(got, _expected_sinks(chunks, wg))
    # every chunk is read exactly once: the lanes' XORs combine to the XOR of the buffer
    total = np.bitwise_xor.reduce(chunks, axis=0)
    assert np.bitwise_xor.reduce(got) == total[0] ^ total[1] ^ total[2] ^ total[3]


def test_mfma_probe_reports_a_plausible_clock():
    _say("probe_mfma_bf16 rounds=200 workgroups=256")
    lib = _lib.get()
    wg, rounds = 256, 200
    sink = torch.zeros(wg * 256, dtype=torch.float32, device="cuda:0")
    ticks = torch.zeros(2 * wg, dtype=torch.int64, device="cuda:0")
    st = torch.cuda.current_stream()
    _lib.check(lib.gqa_attn_probe_mfma_bf16(rounds, 7, wg, sink.data_ptr(), sink.numel(), ticks.data_ptr(),
                                            ticks.numel(), st.cuda_stream), "probe_mfma_bf16")
    torch.cuda.synchronize()
    t = ticks.cpu().view(-1, 2).double()
    assert bool((t > 0).all())
    ghz = (t[:, 0] / t[:, 1] * 0.1)
    assert 0.3 < float(ghz.min()) and float(ghz.max()) < 3.0
    # 64 MFMAs per round per wave take at least 64 * 32 shader cycles
    assert float(t[:, 0].min()) >= rounds * 64 * 32
    assert bool(torch.isfinite(sink).all())
