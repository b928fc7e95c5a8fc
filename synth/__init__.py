"""Seeded synthetic inputs for CSA2 decode.

This package is the one piece shared by the CPU oracle's tests, the GPU
parity tests and the benchmark. It draws random numbers and *encodes* them
into the cache formats (values -> bytes). It decodes nothing and holds none
of the scoring, selection or attention arithmetic: those live, written
independently, in ``oracle/`` (CPU, fp64) and in the HIP kernels.
"""

from .fp_encode import encode_e4m3, encode_fp4_blocks  # noqa: F401
from .workloads import (  # noqa: F401
    CONFIGS,
    Cache,
    DecodeWorkload,
    LayerInputs,
    PrefillWorkload,
    Window,
    make_decode_workload,
    make_prefill_workload,
    take_queries,
    take_requests,
    make_small_decode,
)
