"""CPU oracle (test infrastructure; see scape_oracle's header for who may use it)."""

from .scape_oracle import (  # noqa: F401
    Hyper, OracleOptimizer, PartitionState, accumulate, adams_update, bias_reciprocal,
    compress, dense_adams_step, magnitude_keys, mask_overlap, owner, reduce_mean, statistic_keys,
    step_partition, topk_indices,
)
