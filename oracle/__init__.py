"""CPU float64 oracle for paged-KV GQA decode attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only users.  The HIP library never imports it and it
never imports the HIP library.
"""
from .oracle import (  # noqa: F401
    build,
    decode,
    decode_split,
    f16_to_f64,
    bf16_to_f64,
    max_threads,
)
