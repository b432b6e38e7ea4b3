"""fp64 CPU oracle (test infrastructure only; see ``oracle.attention``)."""
from .attention import (  # noqa: F401
    MASK_CAUSAL, MASK_NONE, MASK_PADDING, MASK_PADDING_CAUSAL, backward, backward_head,
    backward_from_lse, backward_rows, forward, forward_head, forward_rows, is_causal, is_padded, kv_head, loss, segments, valid_rows, visible,
    visible_block,
)
