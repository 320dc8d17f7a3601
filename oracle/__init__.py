"""CPU oracle of the Parallax attention forward and backward pass (test
infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package; the product path never does.
"""
from .parallax_oracle import (  # noqa: F401
    conjugate_gradient,
    decode,
    decode_explicit,
    decode_stream,
    explicit_row,
    lla_prefill,
    lla_row,
    prefill,
    prefill_explicit,
    prefill_head,
    prefill_backward,
    prefill_chunk,
    prefill_head_backward,
    prefill_head_train,
    prefill_rows,
    prefill_train,
    softmax_weights,
)
