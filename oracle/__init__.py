"""CPU float64 oracle for fused exact attention (test infrastructure only).

This package is the reference the tests compare against, not the product.
Only the test suite, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. It shares no code with the HIP library in ``forward_backward_amd``
and imports nothing from it.

Every function is the plain dense definition of scaled-dot-product attention
with the masks the probjax benchmark pages describe, evaluated in float64 on
the exact input values the GPU receives (bf16 or fp32, widened exactly).

Pins (see ``tests/test_oracle.py``): central finite differences, torch float64
CPU ``scaled_dot_product_attention`` with autograd, a pure-Python brute force,
closed forms (constant V, single valid key, zero scale, causal row 0, empty
rows, the zero-width local window), GQA against repeated K/V, key-deletion
invariance under the KV length mask, and local windows against torch's band
helpers and a brute force.  Nothing in this package is "parity unpinned".
"""

from .attention import (  # noqa: F401
    attention_probs,
    attention_fwd,
    attention_bwd,
    attention_decode,
    valid_mask,
)
