"""fp64 CPU oracle for the MiMo-V2-Flash hybrid attention layer.

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path never imports it and shares no code
with it.  See ``mimo_oracle.c`` for what is computed and where the pages state it.
"""
from .oracle import (  # noqa: F401
    OracleParams,
    RouterParams,
    build,
    decode,
    decode_fp8,
    e4m3_decode,
    e4m3_encode,
    extend,
    layer_prefill,
    num_threads,
    omega,
    prefill,
    prefill_f64,
    rotate,
    router,
    router_sigmoid,
    scores,
)
