"""CPU oracle for grouped-query attention forward (test infrastructure only).

This package is the checker, not the product. Only the test suite, the smoke
entry point and the CPU-baseline leg of the benchmark may import it. The HIP
library never calls into it and it never calls into the HIP library; the two
share no code.

Everything here is plain numpy in float64, written from the definition of
softmax attention (see ``oracle.attention`` for the readings taken where the
pages are silent).
"""

from .attention import (  # noqa: F401
    bf16_bits_to_f64,
    default_scale,
    kv_head,
    prefill,
    decode,
    weights,
    decode_partials,
    combine_partials,
    round_to_bf16,
)
