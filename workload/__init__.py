"""Seeded synthetic decode workloads for the dynamic-visual-fixation attention path.

This package holds only input generation: shapes, random draws and the
synthetic fixation trajectory that stands in for a real document page.  It
contains none of the attention method's arithmetic, and both the CPU oracle
and the GPU library consume what it produces.
"""

from .synth import (  # noqa: F401
    WORKLOADS,
    Workload,
    Structure,
    Generator,
    DeviceGenerator,
    make_structure,
    SIGMA_SWEEP,
    TAU_SWEEP,
    bf16_round,
    bf16_bits,
    bits_to_f32,
    get_workload,
)
