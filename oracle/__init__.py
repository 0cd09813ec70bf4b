"""Plain, slow, float64 CPU oracle for exact masked scaled dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) imports, links or calls this package; only the tests, the
smoke check and the CPU-baseline leg of the benchmark do.  It shares no code,
tables or helpers with the GPU path.

Modules
-------
attention : numpy float64 definition of the forward and backward, materialising
            S, A, G_A, c and G_S for every (batch, query head).
tiny      : an independent pure-Python (lists, no numpy) re-derivation of the
            same quantities for tiny shapes, used to cross-check ``attention``.
projection: the projections around the core (Q/K/V = X W, G_W = X^T G, G_X
            summed over the branches that share an input), self- and
            cross-attention.

Parity status: every function here is pinned by tests/test_oracle_*.py against
values printed on the pages, closed forms, invariants, central finite
differences and a library routine (torch float64 autograd); none is unpinned.
"""

from .attention import (  # noqa: F401
    OracleError,
    InvalidArgument,
    EmptyRow,
    kv_group,
    visible_mask,
    validate,
    head_forward,
    head_backward,
    attention_forward,
    attention_backward,
    attention_group,
    attention_backward_packed,
    attention_backward_rope,
    rope_rotate,
    rope_table,
    offsets_per_sequence,
    scores,
    masked_softmax,
    score_grad,
)
from .projection import (  # noqa: F401
    self_attention_backward,
    cross_attention_backward,
    split_qkv_weight,
    to_heads,
    from_heads,
)
