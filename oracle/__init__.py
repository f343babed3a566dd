"""CPU oracle for shared-prefix tree attention (test infrastructure only).

Plain, slow, float64 NumPy implementation of what the tree-attention path
computes.  Only the test suite, the smoke check and the benchmark's CPU
baseline leg may import this package; the product path (the HIP library and
its Python binding) never does, and shares no code with it.

Parity status of every public function is listed in ``tree_attention``'s
module docstring; none is "parity unpinned".
"""

from .tree_attention import (  # noqa: F401
    ancestors,
    visible_tokens,
    visible_mask,
    position_in_sequence,
    subtree_end,
    pairs,
    segment_pairs,
    forward,
    backward,
    forward_rows,
    backward_rows,
    backward_keys,
    masked_dense_forward,
    masked_dense_backward,
)
from .fragments import fragment  # noqa: F401
from .edge_loss import edge_logits, edge_loss_forward, edge_loss_backward  # noqa: F401
from .mamba_tree import (  # noqa: F401
    previous_token,
    conv_forward,
    conv_backward,
    ssm_states,
    ssm_forward,
    ssm_backward,
)
