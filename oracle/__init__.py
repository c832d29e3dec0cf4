"""fp64 CPU oracle (test infrastructure only; see mla_oracle's header)."""

from .mla_oracle import (  # noqa: F401
    attend_absorbed,
    attend_unabsorbed,
    mla_decode,
    rope,
    rope_frequencies,
    sequence_rows,
    softmax,
)
