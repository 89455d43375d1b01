"""Seeded synthetic inputs for the block-sparse video-attention path.

This package only builds inputs: Q/K/V tensors, cluster labels, caller-given block masks
and per-head thresholds, with the shapes and value structure of the video workloads the
pages describe. It holds none of the method's arithmetic (no layout, centroid, scoring,
top-p, attention or repair step). The oracle tests, the GPU tests and the benchmark all
draw their inputs from here, so both sides of every parity check read the same bits.
"""

from .workloads import (  # noqa: F401
    Workload,
    bf16_bits,
    bf16_bits_to_f32,
    grid_tile_labels,
    make_config,
    make_custom,
    CONFIG_NAMES,
)
