"""Calls on several streams. The binding passes torch's current stream; the library
enqueues on it only, and keeps one decode workspace per (device, stream), so decodes on
different streams may overlap. Outputs on side streams must equal, bit for bit, the same
calls on the default stream (every kernel is deterministic for a fixed shape)."""

import pytest
import torch

import gqa_flash_attention_amd as gqa
from gqa_inputs import decode_inputs, prefill_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)


def test_decodes_on_two_streams_overlap_safely():
    d = torch.device("cuda:0")
    _say("decode B=2 L=20000 and B=3 L=7000 interleaved on two side streams, 50 calls each")
    a = [t.to(d) for t in decode_inputs(2, 20000, base=9700)]
    b = [t.to(d) for t in decode_inputs(3, 7000, base=9710)]
    ref_a = gqa.decode(*a).clone()
    ref_b = gqa.decode(*b).clone()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs_a, outs_b = [], []
    for _ in range(50):
        with torch.cuda.stream(s1):
            outs_a.append(gqa.decode(*a))
        with torch.cuda.stream(s2):
            outs_b.append(gqa.decode(*b))
    torch.cuda.synchronize()
    assert all(torch.equal(o, ref_a) for o in outs_a)
    assert all(torch.equal(o, ref_b) for o in outs_b)


def test_prefill_on_a_side_stream_matches_the_default_stream():
    d = torch.device("cuda:0")
    _say("prefill B=2 S=777 on a side stream vs the default stream")
    q, k, v = [t.to(d) for t in prefill_inputs(2, 777, base=9720)]
    ref = gqa.prefill(q, k, v).clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = gqa.prefill(q, k, v)
    s.synchronize()
    assert torch.equal(out, ref)
