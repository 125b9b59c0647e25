"""Seeded synthetic inputs for generalized dot-product attention (GDPA).

This package holds only the input recipe: which random numbers are drawn, in which order, with
which shapes, and how they are rounded to the compute dtype. It contains none of the operator's
arithmetic, so both the fp64 oracle (``oracle/``) and the HIP path
(``generalized_attention_amd``) can take their inputs from it without sharing any code.

The shapes follow the workloads the Kunlun pages describe for the GDPA operator: jagged behaviour
sequences with lengths in the hundreds to thousands, short per-sample key/value blocks produced
from a context vector, several event types with their own head count and head width, and a
sliding-window self-attention variant (Kunlun paper review, sections 2.3 and 2.5; Kunlun
reproduction README, "Core equations").
"""

from .recipe import (  # noqa: F401
    CONFIGS,
    Group,
    GroupSpec,
    Workload,
    make_workload,
    widen,
)
from .accounting import group_work, workload_work  # noqa: F401
