"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws inputs: sparsity patterns in CSR form (``row_ptr``,
``col_idx``) and dense value arrays.  It holds none of the arithmetic of the
operators themselves, so that the CPU oracle and the GPU library can both be fed
from it without sharing any of the code they are checked on.

The graphs are stand-ins, by shape, for the workloads named on the AutoSAGE
page (abstract: Reddit and OGBN-Products aggregation, plus synthetic sparsity and
skew stress tests) and for the fused CSR attention problem of the POPCORNBENCH
trace page (problem statement: per-destination softmax over incoming edge scores,
then aggregation of source values).  No dataset is read or reproduced.

Conventions (the trace page's problem statement): rows are destination nodes,
``col_idx`` holds source nodes, int32 indices, row-major dense arrays.
"""

from .graphs import (  # noqa: F401
    CSR,
    poisson_graph,
    powerlaw_degrees,
    lognormal_degrees,
    rank_size_lengths,
    sample_columns,
    csr_from_degrees,
    configuration_model_symmetric,
    window_global_pattern,
    random_small_graph,
    pattern_hash,
)
from .dense import dense_normal, dense_uniform, to_bf16_bits, bf16_bits_to_f32  # noqa: F401
from .configs import CONFIG_SEED_BASE, config_seed, make_config, CONFIG_NAMES  # noqa: F401
