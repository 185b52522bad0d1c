"""Seeded synthetic workloads shared by the tests, the bench and the oracle.

This package holds only tensor shapes and seeded random draws. It contains
none of the optimizer-step arithmetic: both the HIP library and the CPU
oracle receive the bytes produced here and compute on them independently.
"""

from .shapes import (  # noqa: F401
    llama_tensors,
    llama_7b_tensors,
    llama_65b_tensors,
    llama_7b_split_1024,
    tiny_shard_sizes,
)
from .gen import (  # noqa: F401
    CHUNK,
    chunk_rng,
    normal_draw,
    draw_grads,
    draw_master,
    draw_prior_moments,
    round_to,
    f16_bits_to_f32,
    bf16_bits_to_f32,
)
