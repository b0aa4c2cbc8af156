"""Work and roofline accounting for the attention workloads (host arithmetic only).

FLOP convention of the probjax benchmark pages (it reproduces the ``tflops``
field of every complete record of the page "gpu_attention_h100.json"):
forward = 4 * B * H * Tq * Tkv * D, halved for causal masking; forward plus
backward = 3.5 times the forward.
"""

from __future__ import annotations

# MI355X published peaks (dense, no sparsity).
PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6, "fp8": 5033.2, "fp32": 157.3, "fp64": 78.6}
PEAK_HBM_GBS = 8000.0


def attention_flops(B, H, Tq, Tkv, D, causal=False, mode="fwd"):
    """Nominal FLOPs of one call by the pages' convention."""
    f = 4.0 * B * H * Tq * Tkv * D
    if causal:
        f *= 0.5
    if mode == "fwd":
        return f
    if mode in ("fwd_bwd", "fwd+bwd"):
        return 3.5 * f
    if mode == "bwd":
        return 2.5 * f
    raise ValueError(mode)


def effective_flops(H, Tq, kv_lens, D, mode="fwd"):
    """FLOPs over the keys actually inside each batch's KV length (non-causal)."""
    f = sum(4.0 * H * Tq * int(n) * D for n in kv_lens)
    return {"fwd": f, "fwd_bwd": 3.5 * f, "fwd+bwd": 3.5 * f, "bwd": 2.5 * f}[mode]


def visible_pairs(Tq, Tkv, causal=False, window=None, kv_len=None):
    """Number of (query, key) pairs the masks leave visible (host arithmetic only)."""
    n = Tkv if kv_len is None else min(max(int(kv_len), 0), Tkv)
    left, right = (-1, -1) if window is None else window
    total = 0
    for i in range(Tq):
        lo = 0 if left < 0 else max(i - left, 0)
        hi = n - 1
        if causal:
            hi = min(hi, i)
        if right >= 0:
            hi = min(hi, i + right)
        total += max(hi - lo + 1, 0)
    return total


def decode_bytes(B, Tq, Hq, Hkv, D, kv_lens, elem_bytes=2):
    """Algorithmic HBM bytes of one decode call: K and V rows inside each KV length once, Q and O once."""
    kv = sum(int(n) for n in kv_lens) * Hkv * D * elem_bytes * 2
    qo = 2 * B * Tq * Hq * D * elem_bytes
    return kv + qo
