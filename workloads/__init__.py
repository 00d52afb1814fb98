"""Seeded synthetic inputs for MLA tree-verify attention.

This package holds no attention arithmetic. It draws random numbers, rounds
them to bf16 bit patterns, shapes draft trees and page tables, and names the
workload configurations. Both the CPU oracle and the HIP path consume what it
produces; neither shares any other code with the other.
"""

from .gen import (  # noqa: F401
    Case,
    CONFIGS,
    HEAD_DIM_QK,
    HEAD_DIM_V,
    SM_SCALE,
    f32_to_bf16_bits,
    make_case,
    sweep_case,
    tree_chain,
    tree_depth_capped,
    tree_uniform,
)
