"""Fused exact attention for MI355X (gfx950): forward, backward and split-KV decode.

The compute lives in the HIP library ``libattn.so`` (C ABI declared in
``include/attn.h``); ``forward_backward_amd.attn`` marshals torch tensors into
that ABI.  Importing this package does not load the library; the first call
does, and fails loudly if it has not been built.
"""
