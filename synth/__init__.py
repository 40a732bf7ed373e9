"""Seeded synthetic workloads shared by the tests, the bench and the smoke run.

This package only builds inputs: segment boundaries and bf16 tensors drawn
from a seeded generator. It holds none of the attention arithmetic, so the
oracle and the HIP path can both consume it without sharing any of the
method's code.
"""

from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    make_inputs,
    round_to_bf16_bits,
    bf16_bits_to_f32,
    sample_query_rows,
    real_query_tokens,
    TENSOR_NAMES,
    custom_workload,
)
from .norm_rope import (  # noqa: F401
    NORM_ROPE_WORKLOADS,
    NormRopeWorkload,
    make_norm_rope_inputs,
    rope_table,
)
from .cat_pad import CAT_PAD_CASES, CatPadCase, make_cat_pad_inputs  # noqa: F401
