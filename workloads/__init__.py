"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

Holds no loss arithmetic: only random draws, bf16 rounding of the draws and
the mask recipe. Both the fp64 oracle and the HIP path consume what it makes.
"""

from .synth import (  # noqa: F401
    CONFIGS,
    Workload,
    bf16_bits,
    bf16_to_f32,
    make_workload,
    zipf_uniform_teacher,
    uniform_teacher,
    packed_document_mask,
)
