"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This package only draws random numbers and encodes them (fp32 -> bf16 bit patterns).
It holds none of the sampler's arithmetic: no guidance combine, no reductions, no
selection and no noise transform.  Both the CPU oracle and the HIP library consume
exactly these arrays.
"""

from .workloads import (  # noqa: F401
    ARWorkload,
    DiffusionWorkload,
    DraftWorkload,
    RevealWorkload,
    bf16_from_f32,
    diffusion,
    draft,
    mixed,
    omnivoice,
    reveal,
    stress,
    tiny,
    WORKLOADS,
    ar,
)
