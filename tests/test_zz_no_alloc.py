"""gqa_attn_decode_noalloc, the decode for callers that cannot allocate, against the
library's own decode (gqa_attn_decode): both through the C ABI, on the same inputs, two
calls in a row with the second smaller, then against the fp64 oracle. The two entry points
run the same kernel with the same split, so their outputs must agree bit for bit."""

import pytest
import torch

import oracle
from gqa_flash_attention_amd import _lib
from gqa_inputs import bf16_bits, decode_inputs
from parity_util import assert_close, gpu_f64

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _call(fn, q, kc, vc, lens, out):
    B, Hq, D = q.shape
    L, Hkv = kc.shape[1], kc.shape[2]
    st = torch.cuda.current_stream(q.device).cuda_stream
    rc = fn(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), lens.data_ptr(), out.data_ptr(),
            B, L, Hq, Hkv, D, 0.08838834764831845, st)
    assert rc == 0, (rc, _lib.get().gqa_attn_last_error())


@pytest.mark.parametrize("shapes", [[(2, 20000, [20000, 7001]), (1, 3000, [2999])],
                                    [(1, 65536, [65536]), (3, 700, [700, 1, 0])]])
def test_noalloc_decode_matches_the_library_decode(shapes):
    lib = _lib.get()
    d = torch.device("cuda:0")
    for i, (B, L, lens) in enumerate(shapes):
        _say(f"noalloc decode call {i}: B={B} L={L} lens={lens}")
        q, kc, vc, ln = decode_inputs(B, L, base=12000 + 37 * i + L, lens=lens, poison=True)
        qd, kd, vd, ld = [t.to(d) for t in (q, kc, vc, ln)]
        got = torch.full_like(qd, float("nan"))
        want = torch.full_like(qd, float("nan"))
        _call(lib.gqa_attn_decode_noalloc, qd, kd, vd, ld, got)
        _call(lib.gqa_attn_decode, qd, kd, vd, ld, want)
        torch.cuda.synchronize()
        assert torch.equal(got.cpu(), want.cpu()), f"call {i}: noalloc and library decode differ"
        assert_close(gpu_f64(got), oracle.decode(bf16_bits(q), bf16_bits(kc), bf16_bits(vc), ln),
                     f"noalloc decode B={B} L={L}")
