"""Pins of the float64 oracle against facts other than itself (CPU only).

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign, a transposed operand, a wrong head or mask index) fails at least
one of them; ``test_pins_catch_planted_mistakes`` plants such slips in a copy
of the oracle and checks that they are caught.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention_bwd, attention_decode, attention_fwd, attention_probs, valid_mask


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / den) if den > 0 else float(np.max(np.abs(a)))


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def make(b, tq, tkv, hq, hkv, d, seed):
    return (rnd((b, tq, hq, d), seed), rnd((b, tkv, hkv, d), seed + 1),
            rnd((b, tkv, hkv, d), seed + 2), rnd((b, tq, hq, d), seed + 3))


# ---------------------------------------------------------------- finite differences

def _loss(q, k, v, do, scale, causal, kv_lens):
    o, _ = attention_fwd(q, k, v, scale, causal, kv_lens)
    return float(np.sum(do * o))


def _fd(q, k, v, do, scale, causal, kv_lens, which, h=1e-6):
    arrs = {"q": q, "k": k, "v": v}
    x = arrs[which]
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        orig = x[idx]
        x[idx] = orig + h
        lp = _loss(arrs["q"], arrs["k"], arrs["v"], do, scale, causal, kv_lens)
        x[idx] = orig - h
        lm = _loss(arrs["q"], arrs["k"], arrs["v"], do, scale, causal, kv_lens)
        x[idx] = orig
        g[idx] = (lp - lm) / (2 * h)
    return g


FD_CASES = [
    # b, tq, tkv, hq, hkv, d, causal, kv_lens
    (1, 3, 6, 2, 2, 3, False, None),
    (1, 5, 5, 2, 2, 3, True, None),
    (2, 4, 6, 2, 2, 3, False, [2, 6]),
    (2, 5, 5, 4, 2, 3, True, [3, 5]),
    (1, 4, 5, 3, 1, 2, False, [4]),
]


@pytest.mark.parametrize("case", FD_CASES)
def test_backward_matches_finite_differences(case):
    b, tq, tkv, hq, hkv, d, causal, kv_lens = case
    q, k, v, do = make(b, tq, tkv, hq, hkv, d, seed=11)
    scale = 0.7
    dq, dk, dv = attention_bwd(q, k, v, do, scale, causal, kv_lens)
    for name, an in (("q", dq), ("k", dk), ("v", dv)):
        num = _fd(q, k, v, do, scale, causal, kv_lens, name)
        assert rel(an, num) < 1e-6, (name, rel(an, num))


# ---------------------------------------------------------------- independent library routine

TORCH_CASES = [
    (2, 16, 24, 4, 2, 8, False, [24, 7]),
    (2, 24, 24, 4, 4, 8, True, None),
    (1, 20, 20, 6, 2, 16, True, [13]),
    (2, 9, 33, 2, 1, 8, False, None),
]


@pytest.mark.parametrize("case", TORCH_CASES)
def test_matches_torch_sdpa_float64(case):
    b, tq, tkv, hq, hkv, d, causal, kv_lens = case
    q, k, v, do = make(b, tq, tkv, hq, hkv, d, seed=5)
    scale = 1.0 / math.sqrt(d)
    o, lse = attention_fwd(q, k, v, scale, causal, kv_lens)
    dq, dk, dv = attention_bwd(q, k, v, do, scale, causal, kv_lens)

    tq_ = torch.tensor(q.transpose(0, 2, 1, 3), requires_grad=True)
    tk_ = torch.tensor(k.transpose(0, 2, 1, 3), requires_grad=True)
    tv_ = torch.tensor(v.transpose(0, 2, 1, 3), requires_grad=True)
    mask = torch.ones(b, 1, tq, tkv, dtype=torch.bool)
    if kv_lens is not None:
        for bi, n in enumerate(kv_lens):
            mask[bi, :, :, n:] = False
    if causal:
        mask &= torch.ones(tq, tkv, dtype=torch.bool).tril()
    to = torch.nn.functional.scaled_dot_product_attention(
        tq_, tk_, tv_, attn_mask=mask, scale=scale, enable_gqa=(hq != hkv))
    to.backward(torch.tensor(do.transpose(0, 2, 1, 3)))
    t = lambda x: x.detach().numpy().transpose(0, 2, 1, 3)  # noqa: E731
    assert rel(o, t(to)) < 1e-12
    assert rel(dq, t(tq_.grad)) < 1e-12
    assert rel(dk, t(tk_.grad)) < 1e-12
    assert rel(dv, t(tv_.grad)) < 1e-12
    # LSE is the log of the softmax denominator: exp(S - LSE) sums to one over valid keys.
    for bi in range(b):
        n = tkv if kv_lens is None else kv_lens[bi]
        for h in range(hq):
            s = scale * q[bi, :, h, :] @ k[bi, :, h // (hq // hkv), :].T
            valid = valid_mask(tq, tkv, causal, n)
            tot = np.where(valid, np.exp(s - lse[bi, h][:, None]), 0.0).sum(axis=1)
            assert np.allclose(tot, 1.0, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- pure-Python brute force

def _brute(q, k, v, scale, causal, kv_len):
    tq, d = len(q), len(q[0])
    out, lses = [], []
    for i in range(tq):
        scores = []
        for j in range(len(k)):
            if j < kv_len and (not causal or j <= i):
                scores.append((j, scale * sum(q[i][c] * k[j][c] for c in range(d))))
        if not scores:
            out.append([0.0] * d)
            lses.append(-math.inf)
            continue
        z = sum(math.exp(s) for _, s in scores)
        out.append([sum(math.exp(s) / z * v[j][c] for j, s in scores) for c in range(d)])
        lses.append(math.log(z))
    return out, lses


@pytest.mark.parametrize("causal,kv_len", [(False, 4), (False, 2), (True, 4), (True, 3), (False, 0)])
def test_forward_matches_brute_force(causal, kv_len):
    q, k, v, _ = make(1, 4, 4, 1, 1, 3, seed=3)
    o, lse = attention_fwd(q, k, v, 0.9, causal, [kv_len])
    bo, blse = _brute(q[0, :, 0].tolist(), k[0, :, 0].tolist(), v[0, :, 0].tolist(), 0.9, causal, kv_len)
    assert np.allclose(o[0, :, 0], np.array(bo), rtol=0, atol=1e-13)
    assert np.array_equal(np.isinf(lse[0, 0]), np.isinf(blse))
    fin = np.isfinite(blse)
    assert np.allclose(lse[0, 0][fin], np.array(blse)[fin], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- invariants and closed forms

def test_softmax_rows_sum_to_one_and_vanish_off_mask():
    q, k, _, _ = make(2, 7, 9, 2, 1, 4, seed=9)
    for causal, kv in ((False, [9, 4]), (False, [3, 1])):
        for b in range(2):
            p, _ = attention_probs(q, k, 0.5, causal, kv, b=b, h=1)
            valid = valid_mask(7, 9, causal, kv[b])
            assert np.allclose(p.sum(axis=1), 1.0, atol=1e-14)
            assert np.all(p[~valid] == 0.0)
            assert np.all(p[valid] > 0.0)


def test_constant_v_returns_v_and_zero_dq_dk():
    q, k, _, do = make(1, 6, 6, 2, 2, 4, seed=21)
    row = rnd((4,), 99)
    v = np.broadcast_to(row, (1, 6, 2, 4)).copy()
    for causal in (False, True):
        o, _ = attention_fwd(q, k, v, 0.8, causal)
        assert np.allclose(o, np.broadcast_to(row, o.shape), atol=1e-14)
        dq, dk, _ = attention_bwd(q, k, v, do, 0.8, causal)
        assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13


def test_single_valid_key():
    # kv_len = 1: O_i = V_0; dQ = dK = 0; dV_0 = sum over rows and group heads of dO; dV_j = 0 for j > 0.
    q, k, v, do = make(1, 5, 7, 4, 2, 3, seed=31)
    o, lse = attention_fwd(q, k, v, 0.6, False, [1])
    dq, dk, dv = attention_bwd(q, k, v, do, 0.6, False, [1])
    for h in range(4):
        kh = h // 2
        assert np.allclose(o[0, :, h], np.broadcast_to(v[0, 0, kh], (5, 3)), atol=1e-15)
        assert np.allclose(lse[0, h], 0.6 * q[0, :, h] @ k[0, 0, kh], atol=1e-14)
    assert np.max(np.abs(dq)) < 1e-15 and np.max(np.abs(dk)) < 1e-15
    for kh in range(2):
        expect = do[0, :, 2 * kh:2 * kh + 2].sum(axis=(0, 1))
        assert np.allclose(dv[0, 0, kh], expect, atol=1e-13)
        assert np.all(dv[0, 1:, kh] == 0.0)


def test_zero_scale_gives_mean_of_valid_rows():
    q, k, v, _ = make(2, 4, 6, 1, 1, 3, seed=41)
    o, lse = attention_fwd(q, k, v, 0.0, False, [6, 2])
    assert np.allclose(o[0, :, 0], v[0, :6, 0].mean(axis=0), atol=1e-14)
    assert np.allclose(o[1, :, 0], v[1, :2, 0].mean(axis=0), atol=1e-14)
    assert np.allclose(lse[0, 0], math.log(6)) and np.allclose(lse[1, 0], math.log(2))


def test_causal_first_row_is_first_value():
    q, k, v, _ = make(1, 5, 5, 2, 1, 3, seed=51)
    o, lse = attention_fwd(q, k, v, 1.3, True)
    for h in range(2):
        assert np.allclose(o[0, 0, h], v[0, 0, 0], atol=1e-15)
        assert np.isclose(lse[0, h, 0], 1.3 * q[0, 0, h] @ k[0, 0, 0])


def test_rows_without_valid_key_are_zero():
    q, k, v, do = make(2, 3, 5, 2, 2, 4, seed=61)
    o, lse = attention_fwd(q, k, v, 0.5, False, [0, 5])
    dq, dk, dv = attention_bwd(q, k, v, do, 0.5, False, [0, 5])
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))
    assert np.all(dq[0] == 0.0) and np.all(dk[0] == 0.0) and np.all(dv[0] == 0.0)
    assert np.all(np.isfinite(lse[1])) and np.any(o[1] != 0.0)


def test_gqa_equals_mha_on_repeated_kv():
    q, k, v, do = make(2, 8, 8, 6, 2, 4, seed=71)
    kr = np.repeat(k, 3, axis=2)
    vr = np.repeat(v, 3, axis=2)
    for causal, kv in ((False, [8, 5]), (True, None)):
        o, lse = attention_fwd(q, k, v, 0.5, causal, kv)
        o2, lse2 = attention_fwd(q, kr, vr, 0.5, causal, kv)
        assert np.allclose(o, o2, atol=1e-15) and np.allclose(lse, lse2, atol=1e-15)
        dq, dk, dv = attention_bwd(q, k, v, do, 0.5, causal, kv)
        dq2, dk2, dv2 = attention_bwd(q, kr, vr, do, 0.5, causal, kv)
        assert np.allclose(dq, dq2, atol=1e-14)
        assert np.allclose(dk, dk2.reshape(2, 8, 2, 3, 4).sum(axis=3), atol=1e-14)
        assert np.allclose(dv, dv2.reshape(2, 8, 2, 3, 4).sum(axis=3), atol=1e-14)


def test_kv_length_full_equals_unmasked_and_masked_keys_are_inert():
    q, k, v, do = make(2, 6, 9, 2, 2, 4, seed=81)
    o, lse = attention_fwd(q, k, v, 0.5)
    o2, lse2 = attention_fwd(q, k, v, 0.5, False, [9, 9])
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    # Masked keys can be deleted (batch 1 keeps 4 keys) without changing O, LSE or dQ.
    om, lsem = attention_fwd(q, k, v, 0.5, False, [9, 4])
    dqm, dkm, dvm = attention_bwd(q, k, v, do, 0.5, False, [9, 4])
    ot, lset = attention_fwd(q[1:], k[1:, :4], v[1:, :4], 0.5)
    dqt, dkt, dvt = attention_bwd(q[1:], k[1:, :4], v[1:, :4], do[1:], 0.5)
    assert np.allclose(om[1], ot[0], atol=1e-15) and np.allclose(lsem[1], lset[0], atol=1e-15)
    assert np.allclose(dqm[1], dqt[0], atol=1e-14)
    assert np.allclose(dkm[1, :4], dkt[0], atol=1e-14) and np.allclose(dvm[1, :4], dvt[0], atol=1e-14)
    assert np.all(dkm[1, 4:] == 0.0) and np.all(dvm[1, 4:] == 0.0)
    # Changing masked keys and values changes nothing.
    k2, v2 = k.copy(), v.copy()
    k2[1, 4:] = 1e3
    v2[1, 4:] = -7.0
    om2, _ = attention_fwd(q, k2, v2, 0.5, False, [9, 4])
    assert np.array_equal(om, om2)


def test_decode_is_plain_attention():
    q, k, v, _ = make(2, 3, 40, 8, 2, 4, seed=91)
    o, lse = attention_decode(q, k, v, 0.5, [40, 17])
    o2, lse2 = attention_fwd(q, k, v, 0.5, False, [40, 17])
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_partial_head_selection():
    q, k, v, do = make(2, 5, 5, 4, 2, 3, seed=101)
    o, lse = attention_fwd(q, k, v, 0.5, True)
    os_, lses = attention_fwd(q, k, v, 0.5, True, heads=[(1, 3)])
    assert np.array_equal(os_[1, :, 3], o[1, :, 3]) and np.isnan(os_[0]).all()
    dq, dk, dv = attention_bwd(q, k, v, do, 0.5, True)
    dqs, dks, dvs = attention_bwd(q, k, v, do, 0.5, True, kv_heads=[(0, 1)])
    assert np.array_equal(dqs[0, :, 2:], dq[0, :, 2:]) and np.array_equal(dks[0, :, 1], dk[0, :, 1])
    assert np.isnan(dqs[1]).all() and np.isnan(dvs[0, :, 0]).all()


# ---------------------------------------------------------------- local window masks

WINDOW_FD_CASES = [
    # b, tq=tkv, hq, hkv, d, causal, kv_lens, (left, right)
    (1, 6, 2, 2, 3, False, None, (2, 1)),
    (2, 6, 4, 2, 3, True, [4, 6], (1, -1)),
    (1, 7, 3, 1, 2, False, [5], (-1, 0)),
]


@pytest.mark.parametrize("case", WINDOW_FD_CASES)
def test_window_backward_matches_finite_differences(case):
    b, t, hq, hkv, d, causal, kv_lens, window = case
    q, k, v, do = make(b, t, t, hq, hkv, d, seed=17)
    scale = 0.6
    dq, dk, dv = attention_bwd(q, k, v, do, scale, causal, kv_lens, window=window)

    def loss():
        o, _ = attention_fwd(q, k, v, scale, causal, kv_lens, window=window)
        return float(np.sum(do * o))

    for name, x, an in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            orig = x[idx]
            x[idx] = orig + 1e-6
            lp = loss()
            x[idx] = orig - 1e-6
            lm = loss()
            x[idx] = orig
            num[idx] = (lp - lm) / 2e-6
        assert rel(an, num) < 1e-6, (name, rel(an, num))


@pytest.mark.parametrize("window,causal,kv_lens", [((3, 2), False, None), ((5, 0), True, [17, 9]),
                                                   ((0, 4), False, [12, 20]), ((2, -1), False, None)])
def test_window_matches_torch_sdpa_float64(window, causal, kv_lens):
    b, t, hq, hkv, d = 2, 20, 4, 2, 8
    q, k, v, do = make(b, t, t, hq, hkv, d, seed=23)
    scale = 1.0 / math.sqrt(d)
    o, lse = attention_fwd(q, k, v, scale, causal, kv_lens, window=window)
    dq, dk, dv = attention_bwd(q, k, v, do, scale, causal, kv_lens, window=window)
    left, right = window
    # The band built with torch's own triangular helpers: tril keeps j <= i + right,
    # triu keeps j >= i - left.
    band = torch.ones(t, t, dtype=torch.bool)
    if right >= 0:
        band = band.tril(right)
    if left >= 0:
        band = band.triu(-left)
    if causal:
        band = band & torch.ones(t, t, dtype=torch.bool).tril()
    mask = band.expand(b, 1, t, t).clone()
    if kv_lens is not None:
        for bi, n in enumerate(kv_lens):
            mask[bi, :, :, n:] = False
    tq_ = torch.tensor(q.transpose(0, 2, 1, 3), requires_grad=True)
    tk_ = torch.tensor(k.transpose(0, 2, 1, 3), requires_grad=True)
    tv_ = torch.tensor(v.transpose(0, 2, 1, 3), requires_grad=True)
    to = torch.nn.functional.scaled_dot_product_attention(tq_, tk_, tv_, attn_mask=mask, scale=scale,
                                                          enable_gqa=True)
    to.backward(torch.tensor(do.transpose(0, 2, 1, 3)))
    t_ = lambda x: x.detach().numpy().transpose(0, 2, 1, 3)  # noqa: E731
    assert rel(o, t_(to)) < 1e-12
    assert rel(dq, t_(tq_.grad)) < 1e-12
    assert rel(dk, t_(tk_.grad)) < 1e-12
    assert rel(dv, t_(tv_.grad)) < 1e-12


def _brute_window(q, k, v, scale, left, right):
    out = []
    for i in range(len(q)):
        js = [j for j in range(len(k)) if (left < 0 or j >= i - left) and (right < 0 or j <= i + right)]
        sc = [scale * sum(a * b for a, b in zip(q[i], k[j])) for j in js]
        z = sum(math.exp(x) for x in sc)
        out.append([sum(math.exp(x) / z * v[j][c] for j, x in zip(js, sc)) for c in range(len(v[0]))])
    return out


@pytest.mark.parametrize("window", [(1, 1), (0, 2), (3, 0), (-1, 1)])
def test_window_forward_matches_brute_force(window):
    q, k, v, _ = make(1, 6, 6, 1, 1, 3, seed=29)
    o, _ = attention_fwd(q, k, v, 0.8, window=window)
    bo = _brute_window(q[0, :, 0].tolist(), k[0, :, 0].tolist(), v[0, :, 0].tolist(), 0.8, *window)
    assert np.allclose(o[0, :, 0], np.array(bo), rtol=0, atol=1e-13)


def test_window_closed_forms():
    b, t, h, d = 2, 9, 3, 4
    q, k, v, do = make(b, t, t, h, h, d, seed=31)
    scale = 0.4
    # A zero-width window: query i sees only key i, so O_i = V_i, LSE_i = S_ii,
    # dP - D vanishes (one key), dQ = dK = 0 and dV_i = dO_i.
    o, lse = attention_fwd(q, k, v, scale, window=(0, 0))
    assert np.allclose(o, v, rtol=0, atol=1e-14)
    s_diag = scale * np.einsum("bthd,bthd->bht", q, k)
    assert np.allclose(lse, s_diag, rtol=0, atol=1e-13)
    dq, dk, dv = attention_bwd(q, k, v, do, scale, window=(0, 0))
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
    assert np.allclose(dv, do, rtol=0, atol=1e-14)
    # Windows that reach past every key are no mask; a left bound of at least
    # T with right bound 0 is the causal mask.
    plain = attention_fwd(q, k, v, scale)
    for w in ((t, t), (-1, -1), (t + 5, -1)):
        ow, lw = attention_fwd(q, k, v, scale, window=w)
        assert np.array_equal(ow, plain[0]) and np.array_equal(lw, plain[1])
    causal = attention_fwd(q, k, v, scale, causal=True)
    ow, lw = attention_fwd(q, k, v, scale, window=(t, 0))
    assert np.array_equal(ow, causal[0]) and np.array_equal(lw, causal[1])


# ---------------------------------------------------------------- planted mistakes are caught

def _pins_pass():
    """Cheap subset of the pins above; returns False when any of them fails."""
    try:
        test_backward_matches_finite_differences(FD_CASES[3])
        test_matches_torch_sdpa_float64(TORCH_CASES[0])
        test_matches_torch_sdpa_float64(TORCH_CASES[1])
        test_gqa_equals_mha_on_repeated_kv()
        test_single_valid_key()
        test_forward_matches_brute_force(True, 3)
        test_window_matches_torch_sdpa_float64((3, 2), False, None)
        test_window_closed_forms()
    except AssertionError:
        return False
    return True


def test_pins_catch_planted_mistakes(monkeypatch):
    from oracle import attention as A
    assert _pins_pass()
    good_probs, good_mask = A._head_probs, A.valid_mask

    def lse_off(q_bh, k_bh, scale, valid):
        p, lse = good_probs(q_bh, k_bh, scale, valid)
        return p, lse - 1e-3                           # LSE shifted

    def transposed_scores(q_bh, k_bh, scale, valid):
        if q_bh.shape[0] == k_bh.shape[0]:
            s = scale * (k_bh @ q_bh.T)               # S^T instead of S
            e = np.where(valid, np.exp(s - s.max(axis=1, keepdims=True)), 0)
            p = e / np.maximum(e.sum(axis=1, keepdims=True), 1e-300)
            return p, np.log(np.maximum(e.sum(axis=1), 1e-300)) + s.max(axis=1)
        return good_probs(q_bh, k_bh, scale, valid)

    def causal_off_by_one(tq, tkv, causal, kv_len, window=None):
        m = good_mask(tq, tkv, False, kv_len, window).copy()
        if causal:
            m &= np.arange(tkv)[None, :] < np.arange(tq)[:, None] + 2
        return m

    def window_off_by_one(tq, tkv, causal, kv_len, window=None):
        m = good_mask(tq, tkv, causal, kv_len).copy()
        if window is not None:
            i, j = np.arange(tq)[:, None], np.arange(tkv)[None, :]
            if window[0] >= 0:
                m &= j > i - window[0]                   # drops key i - left
            if window[1] >= 0:
                m &= j <= i + window[1]
        return m

    for name, fn in (("_head_probs", lse_off), ("_head_probs", transposed_scores),
                     ("valid_mask", causal_off_by_one), ("valid_mask", window_off_by_one)):
        monkeypatch.setattr(A, name, fn)
        assert not _pins_pass(), f"planted mistake in {name} ({fn.__name__}) went unnoticed"
        monkeypatch.undo()

    good_grads = A._head_grads

    def grads_without_d_term(p, q_bh, k_bh, v_bh, do_bh, scale):
        ds = p * (do_bh @ v_bh.T)                      # softmax Jacobian's D term dropped
        return scale * (ds @ k_bh), scale * (ds.T @ q_bh), p.T @ do_bh

    def grads_dk_sign(p, q_bh, k_bh, v_bh, do_bh, scale):
        dq, dk, dv = good_grads(p, q_bh, k_bh, v_bh, do_bh, scale)
        return dq, -dk, dv

    def grads_dv_transposed_p(p, q_bh, k_bh, v_bh, do_bh, scale):
        dq, dk, dv = good_grads(p, q_bh, k_bh, v_bh, do_bh, scale)
        if p.shape[0] == p.shape[1]:
            dv = p @ do_bh                             # P instead of P^T
        return dq, dk, dv

    def grads_dq_missing_scale(p, q_bh, k_bh, v_bh, do_bh, scale):
        dq, dk, dv = good_grads(p, q_bh, k_bh, v_bh, do_bh, scale)
        return dq / scale, dk, dv

    for fn in (grads_without_d_term, grads_dk_sign, grads_dv_transposed_p, grads_dq_missing_scale):
        monkeypatch.setattr(A, "_head_grads", fn)
        assert not _pins_pass(), f"planted mistake {fn.__name__} went unnoticed"
        monkeypatch.undo()
    assert _pins_pass()
