"""Seeded synthetic workloads shared by the tests, the benchmark and smoke().

This package only draws random inputs and routes tokens (the router is not
part of the expert path: the path takes token-sorted rows, per-expert offsets
and per-row routing weights as given).  It holds none of the quantization or
GEMM arithmetic, and neither the oracle nor the library depends on it.
"""
from .gen import (CONFIGS, MlpCase, LinearCase, make_linear_case,
                  make_mlp_case, zipf_counts, skewed_counts_with_empty,
                  topk_softmax_routing, sort_by_expert, slot_grid_routing,
                  offsets_from_counts)

__all__ = ["CONFIGS", "MlpCase", "LinearCase", "make_linear_case",
           "make_mlp_case", "zipf_counts", "skewed_counts_with_empty",
           "topk_softmax_routing", "sort_by_expert", "slot_grid_routing",
           "offsets_from_counts"]
