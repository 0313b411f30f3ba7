"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This package only draws random numbers and shapes them into the workloads
(Gaussian-mixture keys, normal values, queries near a mixture centre, random
initial centroid indices). It contains none of the method's arithmetic: no
normalisation, no clustering, no scoring, no attention.

The workloads stand in for the long-context tasks the ClusterKV abstract
(arXiv 2412.03213) evaluates on: 32k-token contexts with a 1k-2k KV budget.
No dataset is used.
"""

from .mixture import (  # noqa: F401
    CONFIGS,
    WorkloadConfig,
    bf16_bits_to_f32,
    f64_to_bf16_bits,
    make_unit_inputs,
    make_layer_inputs,
    make_queries,
    make_init_indices,
    make_new_tokens,
    make_planted_groups,
)
