"""Edge cases of the HIP path (needs an MI355X): empty problems, and inputs
whose unused parts hold NaN.

Every key at or past a batch's KV length, and every element outside the
tensors, must be neither read into a result nor written: the tests place
each tensor inside a larger NaN-filled buffer, set the K/V rows past the KV
length to NaN as well, and require results equal to the oracle's on clean
data (a NaN that reached any product, even multiplied by a zero weight,
would show) with the guard regions left bit-for-bit untouched.
"""

import numpy as np
import pytest

import oracle
from forward_backward_amd.inputs import Case
from helpers import TOL, check_lse, device_inputs, rel_err, to_host64

pytestmark = pytest.mark.gpu

PRE, POST = 256, 8192  # guard elements before / after each tensor (keeps 16-byte alignment)


def _tdtype(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


class Guarded:
    """A tensor view inside a NaN-filled buffer with guard regions on both sides."""

    def __init__(self, shape, tdtype, src=None):
        import torch
        n = int(np.prod(shape))
        self.buf = torch.full((PRE + n + POST,), float("nan"), dtype=tdtype, device="cuda")
        self.view = self.buf[PRE:PRE + n].view(shape)
        if src is not None:
            self.view.copy_(src)
        self.n = n

    def guards_intact(self):
        import torch
        ref = torch.full((1,), float("nan"), dtype=self.buf.dtype, device="cuda")
        bits = torch.int16 if self.buf.dtype == torch.bfloat16 else torch.int32
        want = ref.view(bits)
        head = self.buf[:PRE].view(bits)
        tail = self.buf[PRE + self.n:].view(bits)
        return bool(torch.all(head == want)) and bool(torch.all(tail == want))


def _poison_rows(t, kv_lens):
    """NaN in K/V rows at or past each batch's KV length (inside the tensor)."""
    for b, n in enumerate(kv_lens):
        t[b, n:] = float("nan")


POISON = [
    Case("d128_gqa_kvlen", 3, 200, 333, 8, 2, 128, kv_lens=(333, 150, 0), workload_id=300),
    Case("d64_causal_kvlen", 2, 333, 333, 4, 2, 64, causal=True, kv_lens=(200, 65), workload_id=301),
    Case("d128_causal_kvlen_short", 2, 257, 257, 2, 1, 128, causal=True, kv_lens=(1, 130), workload_id=302),
    Case("fp32_d128_kvlen", 2, 70, 150, 2, 1, 128, "fp32", kv_lens=(149, 3), workload_id=303),
]


@pytest.mark.parametrize("case", POISON, ids=lambda c: c.name)
def test_poisoned_padding_fwd_bwd(case):
    import torch
    from forward_backward_amd import attn
    host, dev, f64 = device_inputs(case)
    print(f"[poison fwd/bwd] {case.name}", flush=True)
    td = _tdtype(case.dtype)
    q, k, v, do = (Guarded(tuple(dev[n].shape), td, dev[n]) for n in ("q", "k", "v", "do"))
    _poison_rows(k.view, case.kv_lens)
    _poison_rows(v.view, case.kv_lens)
    o = Guarded(tuple(dev["q"].shape), td)
    lse = Guarded((case.B, case.Hq, case.Tq), torch.float32)
    dq = Guarded(tuple(dev["q"].shape), td)
    dk = Guarded(tuple(dev["k"].shape), td)
    dv = Guarded(tuple(dev["k"].shape), td)
    kw = dict(scale=case.scale, causal=case.causal, kv_lens=dev["kv_lens"])
    attn.fwd(q.view, k.view, v.view, out=o.view, lse=lse.view, **kw)
    ws = attn.bwd_workspace(q.view, k.view, causal=case.causal, kv_lens=dev["kv_lens"])
    attn.bwd_preprocess(o.view, lse.view, do.view, ws, q.view, k.view, **kw)
    attn.bwd_dkdv(q.view, k.view, v.view, lse.view, do.view, ws, dk.view, dv.view, **kw)
    attn.bwd_dq(q.view, k.view, v.view, lse.view, do.view, ws, dq.view, **kw)
    torch.cuda.synchronize()

    for name, g in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv), ("q", q), ("k", k), ("v", v),
                    ("do", do)):
        assert g.guards_intact(), f"{case.name}: guard region of {name} was written"
    ro, rlse = oracle.attention_fwd(f64["q"], f64["k"], f64["v"], case.scale, case.causal, f64["kv_lens"])
    rdq, rdk, rdv = oracle.attention_bwd(f64["q"], f64["k"], f64["v"], f64["do"], case.scale, case.causal,
                                         f64["kv_lens"])
    got = {"o": to_host64(o.view), "dq": to_host64(dq.view), "dk": to_host64(dk.view), "dv": to_host64(dv.view)}
    for name, ref in (("o", ro), ("dq", rdq), ("dk", rdk), ("dv", rdv)):
        assert np.all(np.isfinite(got[name])), f"{case.name}: non-finite values in {name}"
        err = rel_err(got[name], ref)
        print(f"    {name} rel err {err:.3e}", flush=True)
        assert err <= TOL[case.dtype], f"{case.name}: {name} rel err {err:.3e}"
    check_lse(to_host64(lse.view), rlse)
    for b, n in enumerate(case.kv_lens):
        assert np.all(got["dk"][b, n:] == 0.0) and np.all(got["dv"][b, n:] == 0.0)


DECODE_POISON = [
    Case("dec_d128_g4", 3, 4, 1500, 8, 2, 128, kv_lens=(1500, 513, 0), workload_id=310, decode=True),
    Case("dec_d64_g8", 2, 1, 700, 16, 2, 64, kv_lens=(64, 699), workload_id=311, decode=True),
]


@pytest.mark.parametrize("case", DECODE_POISON, ids=lambda c: c.name)
def test_poisoned_padding_decode(case):
    import torch
    from forward_backward_amd import attn
    host, dev, f64 = device_inputs(case, with_do=False)
    print(f"[poison decode] {case.name}", flush=True)
    q, k, v = (Guarded(tuple(dev[n].shape), torch.bfloat16, dev[n]) for n in ("q", "k", "v"))
    _poison_rows(k.view, case.kv_lens)
    _poison_rows(v.view, case.kv_lens)
    o, lse = attn.decode(q.view, k.view, v.view, kv_lens=dev["kv_lens"], scale=case.scale)
    torch.cuda.synchronize()
    for name, g in (("q", q), ("k", k), ("v", v)):
        assert g.guards_intact(), f"{case.name}: guard region of {name} was written"
    ro, rlse = oracle.attention_decode(f64["q"], f64["k"], f64["v"], case.scale, f64["kv_lens"])
    go = to_host64(o)
    assert np.all(np.isfinite(go))
    err = rel_err(go, ro)
    assert err <= TOL["bf16"], f"{case.name}: O rel err {err:.3e}"
    check_lse(to_host64(lse), rlse)


EMPTY = [
    # name, B, Tq, Tkv, causal, dtype
    ("batch0", 0, 64, 64, False, "bf16"),
    ("q0", 2, 0, 100, False, "bf16"),
    ("kv0", 2, 100, 0, False, "bf16"),
    ("t0_causal", 2, 0, 0, True, "bf16"),
    ("fp32_q0", 2, 0, 50, False, "fp32"),
    ("fp32_kv0", 2, 50, 0, False, "fp32"),
]


@pytest.mark.parametrize("name,B,Tq,Tkv,causal,dtype", EMPTY, ids=[e[0] for e in EMPTY])
@pytest.mark.parametrize("D", [64, 128])
def test_empty_problems(name, B, Tq, Tkv, causal, dtype, D):
    import torch
    from forward_backward_amd import attn
    print(f"[empty] {name} D={D}", flush=True)
    td = _tdtype(dtype)
    Hq, Hkv = 4, 2
    gen = torch.Generator().manual_seed(7)
    q = torch.randn((B, Tq, Hq, D), generator=gen).to(td).cuda()
    k = torch.randn((B, Tkv, Hkv, D), generator=gen).to(td).cuda()
    v = torch.randn((B, Tkv, Hkv, D), generator=gen).to(td).cuda()
    do = torch.randn((B, Tq, Hq, D), generator=gen).to(td).cuda()
    o, lse = attn.fwd(q, k, v, causal=causal)
    dq, dk, dv = attn.bwd(q, k, v, o, lse, do, causal=causal)
    torch.cuda.synchronize()
    assert o.shape == q.shape and lse.shape == (B, Hq, Tq)
    assert dq.shape == q.shape and dk.shape == k.shape and dv.shape == v.shape
    # no key: zero output, -inf LSE, zero dQ; no query: zero dK and dV
    if Tkv == 0:
        assert bool(torch.all(o == 0)) and bool(torch.all(torch.isneginf(lse))) and bool(torch.all(dq == 0))
    if Tq == 0:
        assert bool(torch.all(dk == 0)) and bool(torch.all(dv == 0))
    if dtype == "bf16" and not causal:
        od, lsed = attn.decode(q, k, v)
        torch.cuda.synchronize()
        assert od.shape == q.shape
        if Tkv == 0:
            assert bool(torch.all(od == 0)) and bool(torch.all(torch.isneginf(lsed)))


def test_inputs_at_addresses_with_bit31_of_the_low_word_set():
    """Tile copies take their base address in scalar registers, split in 32-bit
    halves; a low half with bit 31 set must not spill into the high half (a
    sign extension there once made the copies read far outside the tensors).
    The inputs are placed inside one large buffer at an address whose low
    32 bits are >= 2^31, then checked against a copy at an ordinary address."""
    import torch
    from forward_backward_amd import attn
    from helpers import device_inputs, rel_err, to_host64
    case = Case("bit31_d128_T512_gqa", 1, 512, 512, 4, 2, 128, workload_id=130)
    _, dev, _ = device_inputs(case)
    big = torch.empty(2**32 + 2**26, dtype=torch.uint8, device="cuda")
    base = big.data_ptr()
    off = (2**31 + 4096 - (base & 0xFFFFFFFF)) % 2**32  # low word of base + off is 2^31 + 4096
    placed = {}
    for name in ("q", "k", "v", "do"):
        t = dev[name]
        nbytes = t.numel() * 2
        view = big[off:off + nbytes].view(torch.bfloat16).view(t.shape)
        view.copy_(t)
        assert (view.data_ptr() & 0xFFFFFFFF) >= 2**31
        placed[name] = view
        off += (nbytes + 4095) // 4096 * 4096
    o_a, lse_a = attn.fwd(placed["q"], placed["k"], placed["v"], scale=case.scale)
    g_a = attn.bwd(placed["q"], placed["k"], placed["v"], o_a, lse_a, placed["do"], scale=case.scale)
    o_b, lse_b = attn.fwd(dev["q"], dev["k"], dev["v"], scale=case.scale)
    g_b = attn.bwd(dev["q"], dev["k"], dev["v"], o_b, lse_b, dev["do"], scale=case.scale)
    torch.cuda.synchronize()
    assert torch.equal(o_a.view(torch.int16), o_b.view(torch.int16)) and torch.equal(lse_a, lse_b)
    for a, b in zip(g_a, g_b):
        assert rel_err(to_host64(a), to_host64(b)) == 0.0
    del big


def test_tensors_past_2_31_elements():
    """Offsets past 2^31 elements: B = 16384, T = 1024, 2 query heads over one KV
    head, head_dim 128 (K and V hold 2^31 elements each, Q, O and the gradients
    2^32), with per-batch KV lengths. The inputs repeat 7 seeded batches along
    the batch axis: batch b holds the data of batch b % 7. Those 7 are checked
    against the oracle, and every batch's outputs must equal those of its
    source batch bit for bit (the kernels' arithmetic does not depend on where
    a batch sits), which an offset that wrapped at 2^31 or 2^32 would break."""
    import torch
    from forward_backward_amd import attn
    small = Case("big_src_d128_T1024_gqa_kvlen", 7, 1024, 1024, 2, 1, 128,
                 kv_lens=(1024, 1, 700, 0, 1000, 129, 513), workload_id=320)
    host, dev, f64 = device_inputs(small)
    B = 16384
    print(f"[2^31 elements] B={B} T=1024 Hq=2 Hkv=1 d128", flush=True)
    idx = torch.arange(B, device="cuda") % small.B
    big = {n: torch.index_select(dev[n], 0, idx).contiguous() for n in ("q", "k", "v", "do")}
    assert big["k"].numel() >= 2**31 and big["q"].numel() >= 2**32
    lens = torch.index_select(dev["kv_lens"], 0, idx).contiguous()
    o, lse = attn.fwd(big["q"], big["k"], big["v"], scale=small.scale, kv_lens=lens)
    dq, dk, dv = attn.bwd(big["q"], big["k"], big["v"], o, lse, big["do"], scale=small.scale, kv_lens=lens)
    torch.cuda.synchronize()
    outs = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
    for name, t in outs.items():
        bits = t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
        same = torch.equal(bits, torch.index_select(bits[:small.B], 0, idx))
        assert same, f"{name}: a batch differs from its source batch"
    del big
    ro, rlse = oracle.attention_fwd(f64["q"], f64["k"], f64["v"], small.scale, False, f64["kv_lens"])
    rdq, rdk, rdv = oracle.attention_bwd(f64["q"], f64["k"], f64["v"], f64["do"], small.scale, False, f64["kv_lens"])
    for name, g, r in (("o", o[:small.B], ro), ("dq", dq[:small.B], rdq), ("dk", dk[:small.B], rdk),
                       ("dv", dv[:small.B], rdv)):
        err = rel_err(to_host64(g), r)
        print(f"    {name} rel err {err:.3e}", flush=True)
        assert err <= TOL["bf16"], f"{name}: rel err {err:.3e}"
    check_lse(to_host64(lse[:small.B]), rlse)
