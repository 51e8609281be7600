"""Seeded synthetic inputs shared by the tests, the bench and the smoke run.

This package draws random numbers and packs them into the input formats
(contexts, block tables, BF16 query bits, BF16/FP8 latent bytes).  It holds
none of the attention method's arithmetic: no ownership rule, no row
boundary, no softmax, no merge.  Both the float64 oracle and the HIP path
consume what it produces, and neither depends on the other.
"""
from .workloads import CONFIGS, Workload, make_config, make_workload, random_rank_partials, random_segment_partials  # noqa: F401
