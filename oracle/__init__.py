"""CPU oracle (test infrastructure only; see logp_oracle's header)."""

from .logp_oracle import (  # noqa: F401
    InvalidTargetError,
    entropy,
    entropy_bwd,
    linear_entropy,
    linear_logits,
    linear_logp_bwd,
    linear_logp_bwd_weight_rows,
    linear_logp_fwd,
    logp_bwd,
    logp_fwd,
    merge_partials,
    round_bf16,
    num_tiles,
    shard_tile_ranges,
    tile_partials,
    tiled_logp_fwd,
)
