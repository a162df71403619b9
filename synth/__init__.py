"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This package draws random tensors and describes workload shapes.  It holds
none of the BitLinear arithmetic (no scales, no rounding to codes, no
accumulation): those live separately in the HIP library and in the oracle.
"""
from .generators import (  # noqa: F401
    GOLDEN_GAMMA,
    fnv1a64,
    splitmix64_mix,
    stream_key,
    uniform53,
    standard_normal,
    student_t3,
    outlier_channels,
    make_weight,
    make_acts,
)
from .workloads import WORKLOADS, Projection, workload  # noqa: F401
