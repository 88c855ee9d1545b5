"""Seeded synthetic inputs for the paged KV-cache hot path.

This package only *draws* inputs: sequence lengths, physical block placement,
q/k/v values and the contents of the cache before the store.  It performs no
store and no attention arithmetic, so both the CPU oracle and the GPU library
can consume what it returns without sharing any of the method's code.
"""

from .gen import (  # noqa: F401
    BLOCK_SIZE,
    HEAD_DIM,
    POISON_BITS,
    SENTINEL_BITS,
    Spec,
    Workload,
    build,
    config,
    config_specs,
    small_specs,
    bits_view,
)
