"""CPU oracle of the verify pass -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this package.  It never imports the HIP library.
"""
from .dspk_oracle import (  # noqa: F401
    GROUP, decode_fp16, decode_bf16, unpack_codes, dequantize, qlinear,
    argmax_lowest, lmhead_argmax, accept_greedy, sequential_greedy,
    softmax_t, inverse_cdf, accept_sample,
    expected_committed, choose_cap, CapController,
    penalized_logits, truncate, accept_sample_filtered,
)
