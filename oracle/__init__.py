"""fp64 CPU oracle (test infrastructure only; see ``oracle.attention``)."""
from .attention import (  # noqa: F401
    MASK_CAUSAL, MASK_NONE, MASK_PADDING, MASK_PADDING_CAUSAL, backward, backward_blocked, backward_from_lse,
    backward_head, backward_head_blocked, backward_rows, forward, forward_blocked, forward_head,
    forward_head_blocked, forward_rows, is_causal, is_padded, key_range, kv_head, loss, segments, valid_rows,
    visible, visible_block,
)
