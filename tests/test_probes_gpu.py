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


@pytest.mark.parametrize("nbytes,wg", [(1 << 20, 64), (3 * (1 << 20) + 16 * 37, 7)])
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
    n16, stride = chunks.shape[0], wg * 256
    want = np.zeros(stride, dtype=np.uint32)
    for t in range(stride):
        acc = np.bitwise_xor.reduce(chunks[t::stride], axis=0) if t < n16 else np.zeros(4, np.uint32)
        want[t] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3]
    assert np.array_equal(got, want)


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
