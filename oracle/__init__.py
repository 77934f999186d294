"""CPU oracle for the flash-attention forward and backward (test
infrastructure only).

This package is test infrastructure.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import it.
The HIP product path never imports, links or calls anything in here, and this
package imports nothing from the product package.

Every function computes in float64 from the definition of scaled-dot-product
attention, materialising the full score matrix of one (batch or sequence, head)
at a time.  See ``oracle.attention`` for the definitions and their sources.
"""

from .attention import (
    attention_head,
    attention_head_bwd,
    sdpa_dense,
    sdpa_dense_bwd,
    sdpa_compact_varlen,
    sdpa_compact_varlen_bwd,
    sdpa_padded_varlen,
    sdpa_padded_varlen_bwd,
    lengths_from_cu,
)

__all__ = [
    "attention_head",
    "attention_head_bwd",
    "sdpa_dense",
    "sdpa_dense_bwd",
    "sdpa_compact_varlen",
    "sdpa_compact_varlen_bwd",
    "sdpa_padded_varlen",
    "sdpa_padded_varlen_bwd",
    "lengths_from_cu",
]
