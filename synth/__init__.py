"""Seeded synthetic inputs shared by the tests, the oracle runs and the benchmark.

This package only draws random numbers and rounds them to the storage type the
device path reads.  It holds none of the recurrence, composition, seam or
convolution arithmetic: those live in ``oracle/`` (CPU reference) and in the
HIP kernels (device path), which never import each other.
"""

from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    chain_inputs,
    conv_chain_inputs,
    layer_inputs,
    layer_conv_inputs,
    random_elements,
    rne_bf16,
    request_order,
    segment_lengths,
)
