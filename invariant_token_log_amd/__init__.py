"""Batch-invariant selected-token log-probability for AMD Instinct MI355X.

The computation runs in the HIP library libinvariant_logp.so (C ABI declared
in include/invariant_logp.h); this package only marshals PyTorch tensors into
it.  There is no CPU or PyTorch fallback: a missing library raises.
"""

from ._lib import NOALLOC_SCRATCH_BYTES, LogpError, contract_id, lib, status_str  # noqa: F401
from .ops import (  # noqa: F401
    LINEAR_TILE,
    PreparedWeight,
    batch_invariant_logp,
    linear_logp,
    linear_logp_bwd,
    linear_logp_bwd_workspace_bytes,
    linear_logp_fwd,
    linear_logp_fwd_noalloc,
    logp_bwd,
    logp_fwd,
    prepare_weight,
)
