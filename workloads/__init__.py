"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This package generates inputs only. It holds none of the log-probability
arithmetic: no max, no sum-exp, no softmax, no gradient.
"""

from .synth import (  # noqa: F401
    Case,
    SWEEP_SIZES,
    sweep_positions,
    tiny_case,
    mid_case,
    headline_case,
    shard_case,
    long_case,
    sweep_probe_rows,
    sweep_filler_rows,
    random_case,
    case_digest,
)
