"""MI355X (gfx950) shared-prefix tree attention.

Causal attention over a DFS-linearized forest of token segments in which
every query attends only to its ancestor path plus its own segment causally,
forward and deterministic backward, as hand-written HIP kernels behind the C
ABI in ``include/tree_attn.h``.  This package is the thin Python binding.
"""

from .binding import (  # noqa: F401
    BF16,
    FP32,
    EdgePlan,
    MambaPlan,
    Plan,
    TreeAttnError,
    bwd_workspace_bytes,
    conv_bwd,
    conv_fwd,
    edge_loss_bwd,
    edge_loss_fwd,
    fragment,
    fwd_workspace_bytes,
    library,
    ssm_bwd,
    ssm_fwd,
    ssm_states_bytes,
    tree_attn_bwd,
    tree_attn_bwd_noalloc,
    tree_attn_bwd_stages,
    tree_attn_fwd,
)
