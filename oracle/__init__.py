"""CPU oracle for the exact attention forward pass (with or without dropout)
and the rotary embedding.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path (the HIP library
and its Python binding) never calls it and shares no code with it.
"""

from .attention import (  # noqa: F401
    attention,
    attention_blocked,
    attention_bruteforce,
    online_softmax_ul,
    online_softmax_normalised,
    row_probabilities,
)
from .rotary import (  # noqa: F401
    inverse_frequencies,
    pair_indices,
    rotate,
    rotate_dense,
    rotate_packed,
)
from .dropout import (  # noqa: F401
    attention_dropout,
    drop_threshold,
    keep_halves,
    keep_mask,
    philox4x32_10,
)
