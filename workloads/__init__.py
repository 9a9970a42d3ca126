"""Seeded synthetic inputs shared by the tests, the bench and the oracle's callers.

This package holds data preparation only (random draws, masks, bf16 rounding of
the drawn values).  It contains none of the loss or gradient arithmetic, so the
oracle and the HIP path can both be fed from it without sharing any of the
method's code.
"""

from .synth import (  # noqa: F401
    CONFIGS,
    FusedConfig,
    CEConfig,
    FusedInputs,
    CEInputs,
    bf16_round,
    make_fused,
    make_ce,
    zipf_targets,
    make_config,
    ce_targets,
    IGNORE_INDEX,
)
