"""The hot path under HIP graph capture. The prefill and a decode with a caller-owned
workspace allocate nothing and enqueue only their kernels (the decode's merge counters are
reset by the kernel itself, no memset), so both can be captured once and replayed; so can
a decode on the library's own workspace once an eager call on the capturing stream has
created it. Each graph is replayed several times with eager work between the replays (new
inputs copied in place); every replay must equal, bit for bit, the same calls made
eagerly."""

import pytest
import torch

import gqa_flash_attention_amd as gqa
from gqa_inputs import decode_inputs, prefill_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)


def test_prefill_and_decode_replay_from_a_graph():
    d = torch.device("cuda:0")
    B, S, L = 2, 520, 9000
    _say(f"graph: prefill B={B} S={S} + decode B={B} L={L}, 5 replays with new inputs")
    pq, pk, pv = [t.to(d) for t in prefill_inputs(B, S, base=9800)]
    dq, kc, vc, lens = [t.to(d) for t in decode_inputs(B, L, base=9810, lens=[L, L // 3])]
    ws = gqa.decode_workspace(B, L, 32, 8, 128, device=d)
    pout = torch.empty_like(pq)
    dout = torch.empty_like(dq)
    # warm up on a side stream, as graph capture requires
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gqa.prefill(pq, pk, pv, out=pout)
        gqa.decode(dq, kc, vc, lens, out=dout, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gqa.prefill(pq, pk, pv, out=pout)
        gqa.decode(dq, kc, vc, lens, out=dout, workspace=ws)
    torch.cuda.synchronize()
    for r in range(5):
        # eager work between replays: fresh inputs written into the captured buffers
        npq, npk, npv = [t.to(d) for t in prefill_inputs(B, S, base=9900 + 10 * r)]
        ndq, nkc, nvc, _ = [t.to(d) for t in decode_inputs(B, L, base=9950 + 10 * r)]
        for dst, src in ((pq, npq), (pk, npk), (pv, npv), (dq, ndq), (kc, nkc), (vc, nvc)):
            dst.copy_(src)
        want_p = gqa.prefill(pq, pk, pv)
        want_d = gqa.decode(dq, kc, vc, lens)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(pout, want_p), f"replay {r}: prefill differs"
        assert torch.equal(dout, want_d), f"replay {r}: decode differs"


def test_decode_on_the_library_workspace_replays_from_a_graph():
    d = torch.device("cuda:0")
    B, L = 1, 16384
    _say(f"graph: decode B={B} L={L} on the library workspace of the capturing stream, 5 replays")
    dq, kc, vc, lens = [t.to(d) for t in decode_inputs(B, L, base=9870)]
    dout = torch.empty_like(dq)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gqa.decode(dq, kc, vc, lens, out=dout)   # creates and clears this stream's workspace
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        gqa.decode(dq, kc, vc, lens, out=dout)
    torch.cuda.synchronize()
    for r in range(5):
        ndq, nkc, nvc, _ = [t.to(d) for t in decode_inputs(B, L, base=9880 + 10 * r)]
        for dst, src in ((dq, ndq), (kc, nkc), (vc, nvc)):
            dst.copy_(src)
        want = gqa.decode(dq, kc, vc, lens)      # default stream, its own workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dout, want), f"replay {r}: decode differs"


def test_graph_replay_survives_a_larger_eager_decode_on_the_same_stream():
    # The library workspace a graph was captured on must outlive its replacement: an eager
    # decode that needs more workspace on the capturing stream gets a new, larger buffer,
    # and the old one (which the graph's kernel still addresses) is kept until
    # gqa_attn_release.
    d = torch.device("cuda:0")
    B, L = 1, 4096
    _say(f"graph: decode B={B} L={L} captured on a stream's library workspace; a larger eager decode (B=64, "
         f"L=1024: a 2 MB workspace against 1 MB) grows that workspace; 3 replays after it")
    dq, kc, vc, lens = [t.to(d) for t in decode_inputs(B, L, base=9890)]
    dout = torch.empty_like(dq)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gqa.decode(dq, kc, vc, lens, out=dout)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        gqa.decode(dq, kc, vc, lens, out=dout)
    torch.cuda.synchronize()
    bq, bkc, bvc, blens = [t.to(d) for t in decode_inputs(64, 1024, base=9895)]
    with torch.cuda.stream(s):
        big = gqa.decode(bq, bkc, bvc, blens)     # grows the capturing stream's workspace
    torch.cuda.synchronize()
    for r in range(3):
        ndq, nkc, nvc, _ = [t.to(d) for t in decode_inputs(B, L, base=9896 + 10 * r)]
        for dst, src in ((dq, ndq), (kc, nkc), (vc, nvc)):
            dst.copy_(src)
        want = gqa.decode(dq, kc, vc, lens)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dout, want), f"replay {r}: decode differs"
    with torch.cuda.stream(s):
        again = gqa.decode(bq, bkc, bvc, blens)
    torch.cuda.synchronize()
    assert torch.equal(big, again)


def test_decodes_from_two_host_threads_on_one_stream():
    # Both threads use the library workspace of the same stream, with shapes that make it
    # grow; lookup, growth and launch happen under one lock, so neither thread can launch
    # into a buffer the other has replaced. Every output must equal a single-threaded call.
    import threading
    d = torch.device("cuda:0")
    shapes = [(1, 2048), (2, 8192), (64, 1024), (4, 16384)]   # (64, 1024) grows the workspace past 1 MB
    _say(f"two host threads, one stream, decodes of shapes {shapes} in turn, 6 rounds each")
    ins = {sh: [t.to(d) for t in decode_inputs(sh[0], sh[1], base=9990 + sh[0] + sh[1] // 1024)] for sh in shapes}
    ref = {sh: gqa.decode(*ins[sh]) for sh in shapes}
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    outs = {0: [], 1: []}
    errors = []

    def worker(k):
        try:
            with torch.cuda.stream(s):
                for r in range(6):
                    sh = shapes[(r + 2 * k) % len(shapes)]
                    outs[k].append((sh, gqa.decode(*ins[sh])))
        except Exception as e:  # surfaced below
            errors.append(e)

    th = [threading.Thread(target=worker, args=(k,)) for k in (0, 1)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k in (0, 1):
        for sh, o in outs[k]:
            assert torch.equal(o, ref[sh]), f"thread {k} shape {sh} differs"
