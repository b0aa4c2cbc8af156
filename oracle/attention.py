"""Dense float64 scaled-dot-product attention: forward, analytic backward, decode.

Test infrastructure only (see the package docstring): the product path never
imports this module.

Notation follows the probjax benchmark pages ("Attention performance" and
"H100 (Hopper)"): tensors are ``[batch, seq, heads, head_dim]``; query head
``h`` reads KV head ``h // G`` with ``G = Hq / Hkv`` ("Attention performance",
section "Grouped-query attention and decoding"); a per-batch KV length masks
keys at or past it, and a query row with no valid key returns zeros
("H100 (Hopper)", section "Mosaic GPU"); causal masking is the equal-length
form, key j visible to query i iff j <= i ("Attention performance", section
"When to use which"); a local window, one of the position-only masks the
fused kernel takes ("Attention performance", section on the default
attention function), keeps key j for query i iff i - left <= j <= i + right,
a negative bound meaning no bound on that side.  The forward keeps the output
and the log-sum-exp ("Attention performance", section "Memory").

Everything here is the plain definition evaluated per (batch, head) on whole
score matrices: no tiling, no online softmax, no fusion.  Inputs may be any
real arrays; they are widened to float64 exactly.
"""

from __future__ import annotations

import numpy as np


def _clamped_len(kv_lens, b: int, tkv: int) -> int:
    """KV length of batch ``b``: ``Tkv`` when no mask is given, else clamped to [0, Tkv]."""
    if kv_lens is None:
        return tkv
    return int(min(max(int(kv_lens[b]), 0), tkv))


def valid_mask(tq: int, tkv: int, causal: bool, kv_len: int, window=None) -> np.ndarray:
    """Boolean ``[Tq, Tkv]``: key j is visible to query i.

    KV-length mask: j < kv_len ("H100 (Hopper)", section "Mosaic GPU").
    Causal, equal-length form: j <= i ("Attention performance", section
    "When to use which": the fast paths take equal-length causal masking).
    Local window ``(left, right)``: i - left <= j <= i + right, a negative
    bound meaning none on that side; equal lengths, like the causal form.
    The masks combine by AND.
    """
    i = np.arange(tq)[:, None]
    j = np.arange(tkv)[None, :]
    valid = j < kv_len
    if causal:
        if tq != tkv:
            raise ValueError("causal masking is defined here for equal lengths only")
        valid = valid & (j <= i)
    if window is not None:
        left, right = int(window[0]), int(window[1])
        if tq != tkv:
            raise ValueError("window masks are defined here for equal lengths only")
        if left >= 0:
            valid = valid & (j >= i - left)
        if right >= 0:
            valid = valid & (j <= i + right)
    return np.broadcast_to(valid, (tq, tkv))


def _head_probs(q_bh, k_bh, scale, valid):
    """Softmax probabilities and natural-log LSE of one (batch, head).

    S = scale * q k^T; P = softmax over the valid keys of each row, 0 on the
    others; LSE = log of the softmax denominator (in the natural log).  A row
    with no valid key has P = 0 and LSE = -inf.
    """
    s = scale * (q_bh @ k_bh.T)
    has_key = valid.any(axis=1)
    s_valid = np.where(valid, s, -np.inf)
    row_max = np.where(has_key, s_valid.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(valid, np.exp(s_valid - row_max[:, None]), 0.0)
    denom = e.sum(axis=1)
    safe = np.where(has_key, denom, 1.0)
    p = np.where(has_key[:, None], e / safe[:, None], 0.0)
    lse = np.where(has_key, row_max + np.log(safe), -np.inf)
    return p, lse


def _head_grads(p, q_bh, k_bh, v_bh, do_bh, scale):
    """Analytic gradients of sum(dO * O) for one (batch, query head), O = P V.

    dP = dO V^T; D_i = sum_j P_ij dP_ij; dS = P * (dP - D) (softmax Jacobian);
    dQ = scale * dS K; dK = scale * dS^T Q; dV = P^T dO.
    """
    dp = do_bh @ v_bh.T
    d_row = (p * dp).sum(axis=1)
    ds = p * (dp - d_row[:, None])
    return scale * (ds @ k_bh), scale * (ds.T @ q_bh), p.T @ do_bh


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [batch, seq, heads, head_dim]")
    b, tq, hq, d = q.shape
    bk, tkv, hkv, dk = k.shape
    if k.shape != v.shape or bk != b or dk != d:
        raise ValueError("k and v must be [batch, Tkv, Hkv, head_dim] matching q")
    if hkv == 0 or hq % hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    return b, tq, tkv, hq, hkv, d


def attention_probs(q, k, scale, causal=False, kv_lens=None, b=0, h=0, window=None):
    """P ``[Tq, Tkv]`` and LSE ``[Tq]`` of query head ``h`` of batch ``b``."""
    q = _as64(q)
    k = _as64(k)
    _, tq, tkv, hq, hkv, _ = _check_shapes(q, k, k)
    kh = h // (hq // hkv)
    valid = valid_mask(tq, tkv, causal, _clamped_len(kv_lens, b, tkv), window)
    return _head_probs(q[b, :, h, :], k[b, :, kh, :], float(scale), valid)


def attention_fwd(q, k, v, scale, causal=False, kv_lens=None, heads=None, window=None):
    """O = softmax(scale * Q K^T + mask) V and its LSE.

    Returns ``o`` float64 ``[B, Tq, Hq, D]`` and ``lse`` float64 ``[B, Hq, Tq]``
    (natural log; -inf on rows with no valid key, where O is 0).
    ``heads``: optional iterable of (b, h) to evaluate; other entries are NaN.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    bsz, tq, tkv, hq, hkv, d = _check_shapes(q, k, v)
    g = hq // hkv
    o = np.full((bsz, tq, hq, d), np.nan)
    lse = np.full((bsz, hq, tq), np.nan)
    todo = [(b, h) for b in range(bsz) for h in range(hq)] if heads is None else list(heads)
    for b, h in todo:
        kh = h // g
        valid = valid_mask(tq, tkv, causal, _clamped_len(kv_lens, b, tkv), window)
        p, lse_bh = _head_probs(q[b, :, h, :], k[b, :, kh, :], float(scale), valid)
        o[b, :, h, :] = p @ v[b, :, kh, :]
        lse[b, h, :] = lse_bh
    return o, lse


def attention_bwd(q, k, v, do, scale, causal=False, kv_lens=None, kv_heads=None, window=None):
    """Gradients of L = sum(dO * O) with respect to Q, K and V.

    For each (b, h) with KV head kh = h // G:
      dP = dO V^T;  D_i = sum_j P_ij dP_ij;  dS = P * (dP - D);
      dQ = scale * dS K;  dK[kh] += scale * dS^T Q;  dV[kh] += P^T dO,
    summing dK and dV over the G query heads that share the KV head.
    ``kv_heads``: optional iterable of (b, kh) to evaluate (all G query heads
    of each group are included); other entries are NaN.
    Returns ``dq``, ``dk``, ``dv`` in float64.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    bsz, tq, tkv, hq, hkv, d = _check_shapes(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dO must have the shape of Q")
    g = hq // hkv
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    todo = [(b, kh) for b in range(bsz) for kh in range(hkv)] if kv_heads is None else list(kv_heads)
    for b, kh in todo:
        valid = valid_mask(tq, tkv, causal, _clamped_len(kv_lens, b, tkv), window)
        k_bh = k[b, :, kh, :]
        v_bh = v[b, :, kh, :]
        dk_acc = np.zeros((tkv, d))
        dv_acc = np.zeros((tkv, d))
        for h in range(kh * g, (kh + 1) * g):
            q_bh = q[b, :, h, :]
            do_bh = do[b, :, h, :]
            p, _ = _head_probs(q_bh, k_bh, float(scale), valid)
            dq_h, dk_h, dv_h = _head_grads(p, q_bh, k_bh, v_bh, do_bh, float(scale))
            dq[b, :, h, :] = dq_h
            dk_acc += dk_h
            dv_acc += dv_h
        dk[b, :, kh, :] = dk_acc
        dv[b, :, kh, :] = dv_acc
    return dq, dk, dv


def attention_decode(q, k_cache, v_cache, scale, kv_lens=None):
    """Few queries over a long KV cache: the same exact attention, non-causal.

    Splitting the keys and combining partial results by their LSE
    ("Attention performance", section "Grouped-query attention and
    decoding") is exact, so the oracle evaluates the plain definition.
    Returns ``o`` ``[B, Tq, Hq, D]`` and ``lse`` ``[B, Hq, Tq]`` in float64.
    """
    return attention_fwd(q, k_cache, v_cache, scale, causal=False, kv_lens=kv_lens)
